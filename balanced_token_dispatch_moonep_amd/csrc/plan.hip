// Online redundant-expert planning on the GPU.
//
// Pages cited: [TC] thakicloud.com "The Busiest Rank Sets Your Step Time: Running
// MoonEP's Planning Code Ourselves"; [TD] twodots.gr "MoonEP balances AI experts in
// MoE models ..."; [AL] agentlenshq.com "MoonshotAI/MoonEP".
//
// The planner reads the router's top-K choices and decides, with no host
// synchronisation, which experts get a temporary copy on which rank so that every
// rank serves exactly C = S*K rows [TC, "What the technique is" and its flowchart;
// TD, summary; AL, How it works].  Four launches:
//
//   plan_hist   one wave per 64-token chunk: an LDS bitmap per expert (bit t = token t of
//               the chunk picked the expert), built with LDS atomic OR (order-free, so the
//               result is deterministic); its popcounts are the chunk's expert counts.
//               A bit already set flags a duplicate expert within a token.
//   plan_scan   one wave per expert: exclusive prefix of the chunk counts in (rank, token)
//               order with wave shuffles -> each chunk's first pair index per expert; the
//               total is the expert's load L[e].
//   plan_decide one workgroup: rank loads, donors/receivers, the duplicate chain with
//               best-fit picks done as wave-wide argmin/argmax (at most one remote home
//               group per rank [TC, Installation and integration]), prefetch slots or
//               home-row fallback [TD, memory contract], cu_seqlens per rank and weight
//               row, instance offsets, GEMM group tables, the weight-gradient work order
//               (targets by rows, descending) and statistics.
//   plan_dest   one wave per chunk: pair index g = chunk prefix + popcount of the lower
//               bits of the expert's bitmap; the instance holding g gives the final row
//               (the send side computes the receiver's position [TC, "What the technique
//               is"]).
//
// Ties always go to the lower rank / expert id; integer arithmetic only, so the
// result is bit-identical from run to run.
#include <climits>
#include <mutex>

#include "common.h"

namespace moonep {

constexpr int kBad = MOONEP_ST_BAD_ID | MOONEP_ST_DUP_ID | MOONEP_ST_CAPACITY | MOONEP_ST_OVERFLOW;

__global__ __launch_bounds__(64) void plan_hist(const int32_t* __restrict__ topk, PlanWs w) {
    extern __shared__ unsigned long long sbm[];   // [E]
    const int ch = blockIdx.x;
    const int r = ch / w.NC, c = ch % w.NC;
    const int t = threadIdx.x;
    for (int e = t; e < w.E; e += 64) sbm[e] = 0ull;
    __syncthreads();
    const int s = c * kChunk + t;
    int st = 0;
    if (s < w.S) {
        const int32_t* tp = topk + ((size_t)r * w.S + s) * w.K;
        for (int k = 0; k < w.K; ++k) {
            const int e = tp[k];
            if ((unsigned)e >= (unsigned)w.E) {
                st |= MOONEP_ST_BAD_ID;
                continue;
            }
            const unsigned long long old = atomicOr(&sbm[e], 1ull << t);
            if ((old >> t) & 1ull) st |= MOONEP_ST_DUP_ID;
        }
    }
    const unsigned long long bad = __ballot(st & MOONEP_ST_BAD_ID);
    const unsigned long long dup = __ballot(st & MOONEP_ST_DUP_ID);
    __syncthreads();
    for (int e = t; e < w.E; e += 64) {
        const unsigned long long b = sbm[e];
        w.bm[(size_t)ch * w.E + e] = b;
        w.cnt[(size_t)e * w.NCH + ch] = __popcll(b);
    }
    if (t == 0) w.chunk_status[ch] = (bad ? MOONEP_ST_BAD_ID : 0) | (dup ? MOONEP_ST_DUP_ID : 0);
}

__global__ __launch_bounds__(256) void plan_scan(PlanWs w) {
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (e >= w.E) return;
    int32_t* row = w.cnt + (size_t)e * w.NCH;
    int run = 0;
    for (int base = 0; base < w.NCH; base += 64) {
        const int i = base + lane;
        const int v = i < w.NCH ? row[i] : 0;
        int x = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (i < w.NCH) row[i] = run + x - v;
        run += __shfl(x, 63, 64);
    }
    if (lane == 0) w.L[e] = run;
}

// wave-wide min / max of a 32-bit value (DPP-based reductions of the device library)
extern "C" __device__ int __ockl_wfred_min_i32(int);
extern "C" __device__ int __ockl_wfred_max_i32(int);

// lowest lane whose flag is set (flags wave-uniformly nonzero)
__device__ __forceinline__ int first_lane(bool f) {
    return __builtin_ctzll(__ballot(f));
}

struct DecideShared {
    int L[kMaxE];
    int avail[kMaxE];
    int ent[kMaxE][5];     // e, q, a, j, w
    int P[kMaxR], X[kMaxR];
    int don[kMaxR], rec[kMaxR];
    int nd, nr, nent, status, ngroups, nred;
    int rank_nent[kMaxR];
    alignas(16) int trows[kMaxE + kMaxR * kMaxB];   // rows of each dW target (-1 padding)
};

__global__ __launch_bounds__(256) void plan_decide(PlanWs w, uint32_t flags, int32_t* __restrict__ cu,
                                                   int32_t* __restrict__ stats) {
    __shared__ DecideShared sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = w.R, E = w.E, B = w.B, G = w.G, C = w.C;
    const int ncu = E + B + 1;
    if (tid == 0) {
        sh.status = 0;
        sh.nent = 0;
        sh.ngroups = 0;
        sh.nred = 0;
    }
    __syncthreads();
    int st = 0;
    for (int i = tid; i < w.NCH; i += 256) st |= w.chunk_status[i];
    if (st) atomicOr(&sh.status, st);
    for (int e = tid; e < E; e += 256) {
        const int l = w.L[e];
        sh.L[e] = l;
        sh.avail[e] = l;
    }
    if (tid < R) sh.rank_nent[tid] = 0;
    __syncthreads();

    // rank loads P[q] = rows wanting q's home group, X[q] = P[q] - C
    if (tid < R) {
        int p = 0;
        for (int i = 0; i < G; ++i) p += sh.L[tid * G + i];
        sh.P[tid] = p;
        sh.X[tid] = p - C;
    }
    __syncthreads();

    // donors by excess desc, receivers by deficit desc; ties to the lower rank
    if (tid == 0 && !(sh.status & kBad)) {
        int nd = 0, nr = 0;
        for (int q = 0; q < R; ++q) {
            const int x = sh.X[q];
            if (x > 0) {
                int i = nd++;
                while (i > 0 && sh.X[sh.don[i - 1]] < x) { sh.don[i] = sh.don[i - 1]; --i; }
                sh.don[i] = q;
            } else if (x < 0) {
                int i = nr++;
                while (i > 0 && sh.X[sh.rec[i - 1]] > x) { sh.rec[i] = sh.rec[i - 1]; --i; }
                sh.rec[i] = q;
            }
        }
        sh.nd = nd;
        sh.nr = nr;
    }
    __syncthreads();

    // the duplicate chain, on wave 0; lane i holds the remaining rows of the donor's expert i
    if (wave == 0 && !(sh.status & kBad)) {
        int fail = 0;
        int nent = 0;
        auto ship = [&](int d, int t, int amt) {
            const int e = d * G + lane;
            int av = lane < G ? sh.avail[e] : 0;
            while (amt > 0 && !fail) {
                // best fit: fewest remaining rows that still cover amt (ties: lower id)
                const bool cover = lane < G && av >= amt;
                int pick;
                if (__ballot(cover)) {
                    const int m = __ockl_wfred_min_i32(cover ? av : INT_MAX);
                    pick = first_lane(cover && av == m);
                } else {
                    // otherwise the most remaining rows (ties: lower id), all of them
                    const int m = __ockl_wfred_max_i32(lane < G ? av : -1);
                    pick = first_lane(lane < G && av == m);
                }
                const int pav = __shfl(av, pick, 64);
                const int a = pav < amt ? pav : amt;
                if (a <= 0 || nent >= E) {
                    fail = a <= 0 ? MOONEP_ST_CAPACITY : MOONEP_ST_OVERFLOW;
                    break;
                }
                if (lane == 0) {
                    sh.ent[nent][0] = d * G + pick;
                    sh.ent[nent][1] = t;
                    sh.ent[nent][2] = a;
                }
                if (lane == pick) av -= a;
                ++nent;
                amt -= a;
            }
            if (lane < G) sh.avail[e] = av;
        };
        int j = 0, carry_t = -1, carry_s = 0;
        const int nd = sh.nd, nr = sh.nr;
        for (int di = 0; di < nd && !fail; ++di) {
            const int d = sh.don[di];
            int rem = sh.X[d];
            if (carry_t >= 0) {
                ship(d, carry_t, carry_s);
                rem -= carry_s;
                carry_t = -1;
            }
            while (rem > 0 && j < nr && !fail) {
                const int t = sh.rec[j];
                const int need = -sh.X[t];
                ship(d, t, need);
                rem -= need;
                ++j;
            }
            if (rem < 0) {
                carry_t = d;
                carry_s = -rem;
            } else if (rem > 0) {
                fail = MOONEP_ST_CAPACITY;
            }
        }
        if (!fail && (carry_t >= 0 || j != nr)) fail = MOONEP_ST_CAPACITY;
        if (lane == 0) {
            sh.nent = fail ? 0 : nent;
            if (fail) sh.status |= fail;
        }
    }
    __syncthreads();

    const bool bad = (sh.status & kBad) != 0;
    const int nent = sh.nent;
    // slots in creation order per rank: w = E + j for j < B, else the home row (fallback)
    if (tid == 0) {
        for (int i = 0; i < nent; ++i) {
            const int q = sh.ent[i][1];
            const int jj = sh.rank_nent[q]++;
            sh.ent[i][3] = jj;
            sh.ent[i][4] = jj < B ? E + jj : sh.ent[i][0];
        }
    }
    // keep[e] = rows left at home
    for (int e = tid; e < E; e += 256) w.keep[e] = bad ? 0 : sh.avail[e];
    // row counts per (rank, weight row), shifted by one for the scan
    for (int i = tid; i < R * ncu; i += 256) {
        const int q = i / ncu, wr = i % ncu - 1;
        int n = 0;
        if (!bad && wr >= 0 && wr < E && wr / G == q) n = sh.avail[wr];
        cu[i] = n;
    }
    __syncthreads();
    if (tid == 0 && !bad) {
        for (int i = 0; i < nent; ++i) cu[sh.ent[i][1] * ncu + sh.ent[i][4] + 1] += sh.ent[i][2];
    }
    __syncthreads();
    // inclusive scan per rank, one wave per rank
    for (int q = wave; q < R; q += 4) {
        int32_t* row = cu + q * ncu;
        int run = 0;
        for (int base = 0; base < ncu; base += 64) {
            const int i = base + lane;
            const int v = i < ncu ? row[i] : 0;
            int x = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            if (i < ncu) row[i] = run + x;
            run += __shfl(x, 63, 64);
        }
        if (lane == 0 && !bad && run != C) atomicOr(&sh.status, MOONEP_ST_CAPACITY);
    }
    __syncthreads();
    const int status_now = sh.status;
    const bool ok = (status_now & kBad) == 0;

    // instances of each expert: home first, then replicas in creation order
    for (int e = tid; e < E; e += 256) {
        int n = 0;
        if (ok) {
            const int h = e / G;
            int stt = sh.avail[e];
            int32_t* in = w.inst + (size_t)e * kMaxR * 3;
            in[0] = 0;
            in[1] = stt;
            in[2] = h * C + cu[h * ncu + e];
            n = 1;
            int nred = 0, nfb = 0;
            for (int i = 0; i < nent; ++i) {
                if (sh.ent[i][0] != e) continue;
                const int q = sh.ent[i][1], a = sh.ent[i][2], jj = sh.ent[i][3], wr = sh.ent[i][4];
                const int row0 = q * C + cu[q * ncu + wr];
                in[n * 3 + 0] = stt;
                in[n * 3 + 1] = a;
                in[n * 3 + 2] = row0 - stt;
                ++n;
                stt += a;
                if (wr >= E) {
                    w.red_slot[(size_t)e * kMaxR + nred++] = q * B + jj;
                } else {
                    w.fb_seg[(size_t)e * kMaxR + nfb] = Segment{row0, a};
                    ++nfb;
                }
            }
            w.red_n[e] = nred;
            w.fb_n[e] = nfb;
            if (nred > 0) atomicAdd(&sh.nred, 1);
            w.home_seg[e] = Segment{h * C + cu[h * ncu + e], sh.avail[e]};
        } else {
            w.red_n[e] = 0;
            w.fb_n[e] = 0;
            w.home_seg[e] = Segment{0, 0};
        }
        w.ninst[e] = n;
    }
    // zero row segment read by masked GEMM tile loads
    for (int i = tid; i < kZeroElems / 2; i += 256) reinterpret_cast<uint32_t*>(w.zeros)[i] = 0u;
    // slot tables
    for (int i = tid; i < R * B; i += 256) {
        w.slot_e[i] = -1;
        w.slot_row0[i] = 0;
        w.slot_rows[i] = 0;
    }
    __syncthreads();
    if (ok) {
        for (int i = tid; i < nent; i += 256) {
            const int wr = sh.ent[i][4];
            if (wr >= E) {
                const int q = sh.ent[i][1], jj = sh.ent[i][3];
                w.slot_e[q * B + jj] = sh.ent[i][0];
                w.slot_row0[q * B + jj] = q * C + cu[q * ncu + wr];
                w.slot_rows[q * B + jj] = sh.ent[i][2];
            }
        }
    }
    // GEMM groups: non-empty home groups in expert order, then replicas in creation order
    if (wave == 0 && ok) {
        int n = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + lane;
            const bool f = e < E && sh.avail[e] > 0;
            const unsigned long long m = __ballot(f);
            if (f) {
                const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
                const int h = e / G;
                w.groups[pos] = Group{h * C + cu[h * ncu + e], sh.avail[e], e, e};
            }
            n += __popcll(m);
        }
        for (int i = lane; i < nent; i += 64) {
            const int e = sh.ent[i][0], q = sh.ent[i][1], a = sh.ent[i][2], jj = sh.ent[i][3],
                      wr = sh.ent[i][4];
            w.groups[n + i] = Group{q * C + cu[q * ncu + wr], a, wr < E ? wr : -1 - (q * B + jj), e};
        }
        if (lane == 0) sh.ngroups = n + nent;
    }
    // entries table (for inspection)
    for (int i = tid; i < nent; i += 256)
        for (int f = 0; f < 5; ++f) w.entries[i * 5 + f] = sh.ent[i][f];
    // dW targets (home experts with their fallback replicas, then slots) by rows, descending:
    // the weight-gradient GEMM hands out the largest first (longest-processing-time order)
    const int ntarget = E + R * B;
    const int n4 = (ntarget + 3) / 4;
    for (int t = ntarget + tid; t < n4 * 4; t += 256) sh.trows[t] = -1;
    for (int t = tid; t < ntarget; t += 256) {
        int rows = 0;
        if (ok) {
            if (t < E) {
                rows = sh.avail[t];
                for (int i = 0; i < nent; ++i)
                    if (sh.ent[i][0] == t && sh.ent[i][4] < E) rows += sh.ent[i][2];
            } else {
                for (int i = 0; i < nent; ++i)
                    if (sh.ent[i][4] >= E && sh.ent[i][1] * B + sh.ent[i][3] == t - E) rows = sh.ent[i][2];
            }
        }
        sh.trows[t] = rows;
    }
    __syncthreads();
    // rank = targets with more rows, or as many and a lower index (four per broadcast LDS read)
    for (int t = tid; t < ntarget; t += 256) {
        const int r = sh.trows[t];
        int rank = 0;
        const int4* tv = reinterpret_cast<const int4*>(sh.trows);
#pragma unroll 4
        for (int u4 = 0; u4 < n4; ++u4) {
            const int4 v = tv[u4];
            const int u = u4 * 4;
            rank += (v.x > r) || (v.x == r && u < t);
            rank += (v.y > r) || (v.y == r && u + 1 < t);
            rank += (v.z > r) || (v.z == r && u + 2 < t);
            rank += (v.w > r) || (v.w == r && u + 3 < t);
        }
        w.dw_order[rank] = t;
    }
    __syncthreads();

    if (tid == 0) {
        int nslot = 0, nfb = 0, fbrows = 0, migr = 0, maxper = 0;
        for (int i = 0; i < nent; ++i) {
            migr += sh.ent[i][2];
            if (sh.ent[i][4] >= E) ++nslot;
            else { ++nfb; fbrows += sh.ent[i][2]; }
        }
        for (int q = 0; q < R; ++q) maxper = sh.rank_nent[q] > maxper ? sh.rank_nent[q] : maxper;
        int bound = 0, maxp = 0, minp = 0x7fffffff, nd = 0, nr = 0, maxl = 0, total = 0;
        for (int q = 0; q < R; ++q) {
            bound += sh.X[q] > 0 ? sh.X[q] : 0;
            maxp = sh.P[q] > maxp ? sh.P[q] : maxp;
            minp = sh.P[q] < minp ? sh.P[q] : minp;
            nd += sh.X[q] > 0;
            nr += sh.X[q] < 0;
            total += cu[q * ncu + E + B];
        }
        for (int e = 0; e < E; ++e) maxl = sh.L[e] > maxl ? sh.L[e] : maxl;
        int status = sh.status;
        if (ok && nfb > 0 && (flags & MOONEP_TRAINING)) status |= MOONEP_ST_TRAIN_FALLBACK;
        const int nred = ok ? sh.nred : 0;
        const int v[MOONEP_NSTATS] = {status, nent, nslot, nfb, fbrows, migr, bound, maxl, maxp, minp,
                                      nd, nr, maxper, total, 0, 0};
        for (int i = 0; i < MOONEP_NSTATS; ++i) stats[i] = v[i];
        w.hdr[HDR_STATUS] = status;
        w.hdr[HDR_NENTRIES] = nent;
        w.hdr[HDR_NGROUPS] = ok ? sh.ngroups : 0;
        w.hdr[HDR_NSLOTREP] = nslot;
        w.hdr[HDR_NRED] = nred;
    }
}

__global__ __launch_bounds__(64) void plan_dest(const int32_t* __restrict__ topk, PlanWs w,
                                                int32_t* __restrict__ dest) {
    const int ch = blockIdx.x;
    const int r = ch / w.NC, c = ch % w.NC;
    const int t = threadIdx.x;
    const int s = c * kChunk + t;
    if (s >= w.S) return;
    const bool bad = (w.hdr[HDR_STATUS] & kBad) != 0;
    const unsigned long long low = (1ull << t) - 1ull;
    const size_t pbase = ((size_t)r * w.S + s) * w.K;
    for (int k = 0; k < w.K; ++k) {
        const int e = topk[pbase + k];
        int d = -1;
        if (!bad && (unsigned)e < (unsigned)w.E) {
            const int g = w.cnt[(size_t)e * w.NCH + ch] + __popcll(w.bm[(size_t)ch * w.E + e] & low);
            const int ni = min(w.ninst[e], kMaxR);
            const int32_t* in = w.inst + (size_t)e * kMaxR * 3;
            for (int i = 0; i < ni; ++i) {
                const int st = in[i * 3], rows = in[i * 3 + 1];
                if (g >= st && g < st + rows) {
                    d = in[i * 3 + 2] + g;
                    break;
                }
            }
            if (d < 0 || d >= w.R * w.C) d = -1;
        }
        dest[pbase + k] = d;
    }
}

}  // namespace moonep

using namespace moonep;

extern "C" size_t moonep_plan_workspace_bytes(const moonep_dims_t* dims) {
    if (check_dims(dims, false) != MOONEP_OK) return 0;
    return plan_ws_layout(dims, nullptr, nullptr);
}

namespace moonep {

// The four planning launches on a workspace laid out by plan_ws_layout (arguments checked).
static int launch_plan(const moonep_dims_t* dims, const int32_t* topk, void* plan_ws, int32_t* cu_seqlens,
                       int32_t* dest, int32_t* stats, void* stream) {
    PlanWs w;
    plan_ws_layout(dims, plan_ws, &w);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(plan_hist, dim3(w.NCH), dim3(64), (size_t)w.E * 8, s, topk, w);
    MOONEP_LAUNCH_CHECK();
    hipLaunchKernelGGL(plan_scan, dim3((w.E + 3) / 4), dim3(256), 0, s, w);
    MOONEP_LAUNCH_CHECK();
    hipLaunchKernelGGL(plan_decide, dim3(1), dim3(256), 0, s, w, dims->flags, cu_seqlens, stats);
    MOONEP_LAUNCH_CHECK();
    hipLaunchKernelGGL(plan_dest, dim3(w.NCH), dim3(64), 0, s, topk, w, dest);
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

// Plan workspace of moonep_plan_noalloc: one static array per GPU, held until the process ends.
// In host code `scratch` only stands in for the symbol; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[MOONEP_NOALLOC_WS_BYTES];
constexpr int kMaxDevices = 64;

static int scratch_of_current_device(void** out) {
    static std::mutex mu;
    static void* ptrs[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOONEP_EHIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOONEP_EHIP;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return MOONEP_OK;
}

}  // namespace moonep

extern "C" int moonep_plan(const moonep_dims_t* dims, const int32_t* topk, void* plan_ws,
                           int32_t* cu_seqlens, int32_t* dest, int32_t* stats, void* stream) {
    const int rc = check_dims(dims, false);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(topk);
    MOONEP_CHECK_PTR(plan_ws);
    MOONEP_CHECK_PTR(cu_seqlens);
    MOONEP_CHECK_PTR(dest);
    MOONEP_CHECK_PTR(stats);
    return launch_plan(dims, topk, plan_ws, cu_seqlens, dest, stats, stream);
}

extern "C" int moonep_plan_noalloc(const moonep_dims_t* dims, const int32_t* topk, int32_t* cu_seqlens,
                                   int32_t* dest, int32_t* stats, void* stream) {
    int rc = check_dims(dims, false);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(topk);
    MOONEP_CHECK_PTR(cu_seqlens);
    MOONEP_CHECK_PTR(dest);
    MOONEP_CHECK_PTR(stats);
    if (plan_ws_layout(dims, nullptr, nullptr) > (size_t)MOONEP_NOALLOC_WS_BYTES) return MOONEP_ETOOBIG;
    void* ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc != MOONEP_OK) return rc;
    return launch_plan(dims, topk, ws, cu_seqlens, dest, stats, stream);
}
