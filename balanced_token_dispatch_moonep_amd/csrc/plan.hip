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

// Exclusive prefix of each expert's chunk counts in (rank, token) order, one wave per expert.
// The counts are loaded eight 64-chunk batches at a time before they are scanned, so the loads
// of a batch are in flight together rather than one after another.
constexpr int kScanBatch = 8;
__global__ __launch_bounds__(256) void plan_scan(PlanWs w) {
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (e >= w.E) return;
    int32_t* row = w.cnt + (size_t)e * w.NCH;
    int run = 0;
    for (int base = 0; base < w.NCH; base += 64 * kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int b = 0; b < kScanBatch; ++b) {
            const int i = base + b * 64 + lane;
            v[b] = i < w.NCH ? row[i] : 0;
        }
#pragma unroll
        for (int b = 0; b < kScanBatch; ++b) {
            int x = v[b];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            const int i = base + b * 64 + lane;
            if (i < w.NCH) row[i] = run + x - v[b];
            run += __shfl(x, 63, 64);
        }
    }
    if (lane == 0) w.L[e] = run;
}

// Wave-wide min / max of a 32-bit value: DPP exchanges inside each row of 16 lanes (quad
// swaps, half-row and row mirrors), then the four row results.  Every lane must be active.
template <bool MAX>
__device__ __forceinline__ int wave_reduce(int v) {
    auto op = [](int a, int b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    v = op(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    v = op(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = op(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));   // row_mirror
    return op(op(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
              op(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// lowest lane whose flag is set (flags wave-uniformly nonzero)
__device__ __forceinline__ int first_lane(bool f) {
    return __builtin_ctzll(__ballot(f));
}

// Per-expert replica counters, packed: all replicas (bits 0-9), slot replicas (10-19),
// fallback replicas (20-29).  An expert has at most R - 1 < 1024 replicas.
constexpr int kCntAll = 1, kCntSlot = 1 << 10, kCntFb = 1 << 20;

struct DecideShared {
    int L[kMaxE];                 // rows routed to each expert
    int avail[kMaxE];             // rows not (yet) given to a replica; keep[] after the chain
    int ecnt[kMaxE];              // packed replica counters of each expert
    // plan entries (replicas) in creation order
    int ent_e[kMaxE], ent_q[kMaxE], ent_a[kMaxE];
    int ent_j[kMaxE];             // creation index among rank q's entries (slot E+j if j < B)
    int ent_pre[kMaxE];           // rows of e given to earlier replicas of e
    int ent_k[kMaxE];             // index among e's replicas | index among those of its kind << 16
    int rank_ent[kMaxR][kMaxG];   // entry ids on each rank by creation index
    int rank_w[kMaxR][kMaxG];     // their weight rows
    int rank_a[kMaxR][kMaxG];     // their rows
    int rank_n[kMaxR];            // entries on each rank
    int homepre[kMaxE];           // rows kept by the experts of e's home group before e
    int nzpre[kMaxE];             // experts of e's home group before e that keep rows
    int hometot[kMaxR];           // rows kept by each rank's home group
    int nzbase[kMaxR + 1];        // experts that keep rows in the home groups before each rank
    int P[kMaxR], X[kMaxR], don[kMaxR], rec[kMaxR];
    int nd, nr, nent, status, nred;
    int migr, nslot, nfb, fbrows, maxl;
};

// Rows on rank q whose weight row is below w, i.e. cu_seqlens[q][w] (home rows in expert order,
// then the rank's replicas by weight row), from the home prefix and the rank's few replicas.
__device__ __forceinline__ int cu_at(const DecideShared& sh, int q, int w, int E, int G, int B) {
    const int h0 = q * G;
    int s = w <= h0 ? 0 : w >= h0 + G ? sh.hometot[q] : sh.homepre[w];
    const int n = sh.rank_n[q];
    for (int j = 0; j < n; ++j) s += sh.rank_w[q][j] < w ? sh.rank_a[q][j] : 0;
    return s;
}

constexpr int kDecideThreads = 512;

__global__ __launch_bounds__(kDecideThreads) void plan_decide(PlanWs w, uint32_t flags, int32_t* __restrict__ cu,
                                                              int32_t* __restrict__ stats) {
    extern __shared__ __attribute__((aligned(16))) char decide_smem[];
    DecideShared& sh = *reinterpret_cast<DecideShared*>(decide_smem);
    constexpr int NT = kDecideThreads, NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = w.R, E = w.E, B = w.B, G = w.G, C = w.C;
    const int ncu = E + B + 1;
    if (tid == 0) {
        sh.status = 0; sh.nent = 0; sh.nd = 0; sh.nr = 0; sh.nred = 0;
        sh.migr = 0; sh.nslot = 0; sh.nfb = 0; sh.fbrows = 0; sh.maxl = 0;
    }
    if (tid < R) sh.rank_n[tid] = 0;
    __syncthreads();
    int st = 0;
    for (int i = tid; i < w.NCH; i += NT) st |= w.chunk_status[i];
    if (st) atomicOr(&sh.status, st);
    int ml = 0;
    for (int e = tid; e < E; e += NT) {
        const int l = w.L[e];
        sh.L[e] = l;
        sh.avail[e] = l;
        sh.ecnt[e] = 0;
        ml = max(ml, l);
    }
    atomicMax(&sh.maxl, ml);
    __syncthreads();

    // rank loads P[q] = rows wanting q's home group, X[q] = P[q] - C
    if (tid < R) {
        int p = 0;
        for (int i = 0; i < G; ++i) p += sh.L[tid * G + i];
        sh.P[tid] = p;
        sh.X[tid] = p - C;
    }
    __syncthreads();

    // donors by excess desc, receivers by deficit desc, ties to the lower rank: each rank
    // counts the ranks of its kind ahead of it
    if (tid < R && !(sh.status & kBad)) {
        const int x = sh.X[tid];
        if (x != 0) {
            int pos = 0;
            for (int q = 0; q < R; ++q) {
                const int y = sh.X[q];
                if (y != 0 && (x > 0) == (y > 0)) pos += (x > 0 ? y > x : y < x) || (y == x && q < tid);
            }
            if (x > 0) {
                sh.don[pos] = tid;
                atomicAdd(&sh.nd, 1);
            } else {
                sh.rec[pos] = tid;
                atomicAdd(&sh.nr, 1);
            }
        }
    }
    __syncthreads();

    // the duplicate chain, on wave 0; lane i holds the remaining rows of the donor's expert i
    if (wave == 0 && !(sh.status & kBad)) {
        int fail = 0;
        int nent = 0;
        // ship(d, t, amt): amt rows of donor group d's experts to rank t, best fit first.  Every
        // rank receives from one ship call only, so the entries this call makes on t are t's
        // entries j = 0, 1, ... in creation order.  Lane i holds expert d*G+i while picking;
        // the call's entry j is kept in lane j's registers and all are written after the call.
        auto ship = [&](int d, int t, int amt) {
            const int e = d * G + lane;
            int av = lane < G ? sh.avail[e] : 0;
            const int lv = lane < G ? sh.L[e] : 0;
            int cnt = lane < G ? sh.ecnt[e] : 0;
            int j = 0;
            int my_e = 0, my_a = 0, my_pre = 0, my_k = 0;
            while (amt > 0 && !fail) {
                // best fit: fewest remaining rows that still cover amt (ties: lower id)
                const bool cover = lane < G && av >= amt;
                int m, pick;
                if (__ballot(cover)) {
                    m = wave_reduce<false>(cover ? av : INT_MAX);
                    pick = first_lane(cover && av == m);
                } else {
                    // otherwise the most remaining rows (ties: lower id), all of them
                    m = wave_reduce<true>(lane < G ? av : -1);
                    pick = first_lane(lane < G && av == m);
                }
                const int a = m < amt ? m : amt;
                if (a <= 0 || nent + j >= E || j >= kMaxG) {
                    fail = a <= 0 ? MOONEP_ST_CAPACITY : MOONEP_ST_OVERFLOW;
                    break;
                }
                // the picked expert's counters and the rows it gave earlier replicas (read with
                // every lane active)
                const int pc = __builtin_amdgcn_readlane(cnt, pick);
                const int pre = __builtin_amdgcn_readlane(lv - av, pick);
                const bool slot = j < B;
                const int kind = slot ? (pc >> 10) & 0x3FF : (pc >> 20) & 0x3FF;
                if (lane == j) {
                    my_e = d * G + pick;
                    my_a = a;
                    my_pre = pre;
                    my_k = (pc & 0x3FF) | (kind << 16);
                }
                if (lane == pick) {
                    cnt += kCntAll + (slot ? kCntSlot : kCntFb);
                    av -= a;
                }
                ++j;
                amt -= a;
            }
            if (lane < G) {
                sh.avail[e] = av;
                sh.ecnt[e] = cnt;
            }
            if (lane < j) {
                const int i = nent + lane;
                sh.ent_e[i] = my_e;
                sh.ent_q[i] = t;
                sh.ent_a[i] = my_a;
                sh.ent_j[i] = lane;
                sh.ent_pre[i] = my_pre;
                sh.ent_k[i] = my_k;
                sh.rank_ent[t][lane] = i;
                sh.rank_w[t][lane] = lane < B ? E + lane : my_e;
                sh.rank_a[t][lane] = my_a;
            }
            if (lane == 0) sh.rank_n[t] = j;
            nent += j;
        };
        const int nd = sh.nd, nr = sh.nr;
        // lane r holds donor r and receiver r (in order) with their excess / deficit
        const int l_don = lane < nd ? sh.don[lane] : 0, l_rec = lane < nr ? sh.rec[lane] : 0;
        const int l_dx = lane < nd ? sh.X[l_don] : 0, l_rd = lane < nr ? -sh.X[l_rec] : 0;
        int carry_t = -1, carry_s = 0;
        if (!(flags & MOONEP_PLAN_LOWMIG)) {
            // Chain: a donor repays the shortfall it inherited, then covers whole receivers in
            // order; over-covering the last one leaves it short, which the next donor repays.
            int jr = 0;
            for (int di = 0; di < nd && !fail; ++di) {
                const int d = __builtin_amdgcn_readlane(l_don, di);
                int rem = __builtin_amdgcn_readlane(l_dx, di);
                if (carry_t >= 0) {
                    ship(d, carry_t, carry_s);
                    rem -= carry_s;
                    carry_t = -1;
                }
                while (rem > 0 && jr < nr && !fail) {
                    const int t = __builtin_amdgcn_readlane(l_rec, jr);
                    const int need = __builtin_amdgcn_readlane(l_rd, jr);
                    ship(d, t, need);
                    rem -= need;
                    ++jr;
                }
                if (rem < 0) {
                    carry_t = d;
                    carry_s = -rem;
                } else if (rem > 0) {
                    fail = MOONEP_ST_CAPACITY;
                }
            }
            if (!fail && (carry_t >= 0 || jr != nr)) fail = MOONEP_ST_CAPACITY;
        } else {
            // Low-migration chain: a donor repays an inherited shortfall; the last donor covers
            // every receiver left; any other covers the largest remaining receiver that fits
            // whole, again and again, then either covers the smallest remaining one whole (short
            // by s, repaid by the next donor) or hands its rem rows to the next donor, which
            // ships them on: the first only if s < rem and it was handed nothing itself.
            bool left = lane < nr;           // receiver `lane` not covered yet
            int handed = 0;
            for (int di = 0; di < nd && !fail; ++di) {
                const int d = __builtin_amdgcn_readlane(l_don, di);
                int rem = __builtin_amdgcn_readlane(l_dx, di) + handed;
                const bool may_repay = handed == 0;
                handed = 0;
                if (carry_t >= 0) {
                    ship(d, carry_t, carry_s);
                    rem -= carry_s;
                    carry_t = -1;
                }
                if (di == nd - 1) {
                    for (unsigned long long m = __ballot(left); m && !fail; m &= m - 1) {
                        const int r = __builtin_ctzll(m);
                        const int need = __builtin_amdgcn_readlane(l_rd, r);
                        ship(d, __builtin_amdgcn_readlane(l_rec, r), need);
                        rem -= need;
                    }
                    left = false;
                }
                while (rem > 0 && !fail && __ballot(left)) {
                    const unsigned long long fit = __ballot(left && l_rd <= rem);
                    int r, need;
                    if (fit) {
                        r = __builtin_ctzll(fit);
                        need = __builtin_amdgcn_readlane(l_rd, r);
                    } else {
                        need = wave_reduce<false>(left ? l_rd : INT_MAX);
                        r = first_lane(left && l_rd == need);
                        if (!(may_repay && need - rem < rem)) {
                            if (di + 1 >= nd) {
                                fail = MOONEP_ST_CAPACITY;
                                break;
                            }
                            ship(d, __builtin_amdgcn_readlane(l_don, di + 1), rem);
                            handed = rem;
                            rem = 0;
                            break;
                        }
                    }
                    ship(d, __builtin_amdgcn_readlane(l_rec, r), need);
                    rem -= need;
                    if (lane == r) left = false;
                }
                if (rem < 0) {
                    carry_t = d;
                    carry_s = -rem;
                } else if (rem > 0) {
                    fail = MOONEP_ST_CAPACITY;
                }
            }
            if (!fail && (carry_t >= 0 || handed || __ballot(left))) fail = MOONEP_ST_CAPACITY;
        }
        if (lane == 0) {
            sh.nent = fail ? 0 : nent;
            if (fail) sh.status |= fail;
        }
    }
    __syncthreads();

    // rows kept by each home group before each expert, and how many of those experts keep rows
    // (wave-wide scans per rank; G <= 64)
    for (int q = wave; q < R; q += NW) {
        const int v = lane < G ? sh.avail[q * G + lane] : 0;
        int x = v;
        int c = v > 0;
        const int c0 = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            const int z = __shfl_up(c, o, 64);
            if (lane >= o) {
                x += y;
                c += z;
            }
        }
        if (lane < G) {
            sh.homepre[q * G + lane] = x - v;
            sh.nzpre[q * G + lane] = c - c0;
        }
        if (lane == 63) {
            sh.hometot[q] = x;
            sh.nzbase[q + 1] = c;
        }
    }
    __syncthreads();
    // non-empty home groups before each rank (R <= 64: one wave)
    if (wave == 0) {
        const int v = lane < R ? sh.nzbase[lane + 1] : 0;
        int x = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane < R) sh.nzbase[lane + 1] = x;
        if (lane == 0) sh.nzbase[0] = 0;
    }
    // every rank must total exactly S*K rows [TC, text under Table 1]
    if (tid < R && !(sh.status & kBad) && cu_at(sh, tid, E + B, E, G, B) != C)
        atomicOr(&sh.status, MOONEP_ST_CAPACITY);
    __syncthreads();
    const bool ok = (sh.status & kBad) == 0;
    const int nent = ok ? sh.nent : 0;

    // per expert: rows kept at home, the home instance, segment and GEMM group, replica counts
    for (int e = tid; e < E; e += NT) {
        const int av = sh.avail[e];
        w.keep[e] = ok ? av : 0;
        int n = 0, nred = 0, nfb = 0;
        Segment hs{0, 0};
        if (ok) {
            const int h = e / G;
            hs = Segment{h * C + cu_at(sh, h, e, E, G, B), av};
            int32_t* in = w.inst + (size_t)e * kMaxR * 3;
            in[0] = 0;
            in[1] = av;
            in[2] = hs.row0;
            const int c = sh.ecnt[e];
            n = 1 + (c & 0x3FF);
            nred = (c >> 10) & 0x3FF;
            nfb = (c >> 20) & 0x3FF;
            if (nred > 0) atomicAdd(&sh.nred, 1);
            // GEMM groups: non-empty home groups in expert order, then the entries'
            if (av > 0) w.groups[sh.nzbase[h] + sh.nzpre[e]] = Group{hs.row0, av, e, e};
        }
        w.ninst[e] = n;
        w.red_n[e] = nred;
        w.fb_n[e] = nfb;
        w.home_seg[e] = hs;
    }
    // slot tables: slot (q, j) holds rank q's replica j if it has one
    for (int i = tid; i < R * B; i += NT) {
        const int q = i / B, jj = i % B;
        int e = -1, row0 = 0, rows = 0;
        if (ok && jj < sh.rank_n[q]) {
            const int ei = sh.rank_ent[q][jj];
            e = sh.ent_e[ei];
            row0 = q * C + cu_at(sh, q, E + jj, E, G, B);
            rows = sh.ent_a[ei];
        }
        w.slot_e[i] = e;
        w.slot_row0[i] = row0;
        w.slot_rows[i] = rows;
    }
    // zero row segment read by masked GEMM tile loads
    for (int i = tid; i < kZeroElems / 2; i += NT) reinterpret_cast<uint32_t*>(w.zeros)[i] = 0u;
    __syncthreads();

    // per entry: its instance, reduce slot or fallback segment, GEMM group
    const int nhome = sh.nzbase[R];
    int migr = 0, nslot = 0, nfb = 0, fbrows = 0;
    for (int i = tid; i < nent; i += NT) {
        const int e = sh.ent_e[i], q = sh.ent_q[i], a = sh.ent_a[i], jj = sh.ent_j[i];
        const int k = sh.ent_k[i] & 0xFFFF, kk = sh.ent_k[i] >> 16;
        const int wr = jj < B ? E + jj : e;
        const int row0 = q * C + cu_at(sh, q, wr, E, G, B);
        const int stt = sh.avail[e] + sh.ent_pre[i];      // home rows first, then replicas in order
        int32_t* in = w.inst + ((size_t)e * kMaxR + 1 + k) * 3;
        in[0] = stt;
        in[1] = a;
        in[2] = row0 - stt;
        if (wr >= E) {
            w.red_slot[(size_t)e * kMaxR + kk] = q * B + jj;
            ++nslot;
        } else {
            w.fb_seg[(size_t)e * kMaxR + kk] = Segment{row0, a};
            ++nfb;
            fbrows += a;
        }
        migr += a;
        int32_t* en = w.entries + (size_t)i * 5;
        en[0] = e;
        en[1] = q;
        en[2] = a;
        en[3] = jj;
        en[4] = wr;
        w.groups[nhome + i] = Group{row0, a, wr < E ? wr : -1 - (q * B + jj), e};
    }
    if (migr) atomicAdd(&sh.migr, migr);
    if (nslot) atomicAdd(&sh.nslot, nslot);
    if (nfb) atomicAdd(&sh.nfb, nfb);
    if (fbrows) atomicAdd(&sh.fbrows, fbrows);
    // cu_seqlens: rows of rank q whose weight row is below p, every (q, p) at once
    for (int i = tid; i < R * ncu; i += NT) {
        const int q = i / ncu, p = i % ncu;
        cu[i] = ok ? cu_at(sh, q, p, E, G, B) : 0;
    }
    __syncthreads();

    if (tid == 0) {
        int maxper = 0, bound = 0, maxp = 0, minp = 0x7fffffff, nd = 0, nr = 0;
        for (int q = 0; q < R; ++q) {
            if (ok) maxper = max(maxper, sh.rank_n[q]);
            bound += sh.X[q] > 0 ? sh.X[q] : 0;
            maxp = max(maxp, sh.P[q]);
            minp = min(minp, sh.P[q]);
            nd += sh.X[q] > 0;
            nr += sh.X[q] < 0;
        }
        int status = sh.status;
        if (ok && sh.nfb > 0 && (flags & MOONEP_TRAINING)) status |= MOONEP_ST_TRAIN_FALLBACK;
        const int v[MOONEP_NSTATS] = {status, nent, sh.nslot, sh.nfb, sh.fbrows, sh.migr, bound, sh.maxl,
                                      maxp, minp, nd, nr, maxper, ok ? R * C : 0, 0, 0};
        for (int i = 0; i < MOONEP_NSTATS; ++i) stats[i] = v[i];
        w.hdr[HDR_STATUS] = status;
        w.hdr[HDR_NENTRIES] = nent;
        w.hdr[HDR_NGROUPS] = ok ? nhome + nent : 0;
        w.hdr[HDR_NSLOTREP] = sh.nslot;
        w.hdr[HDR_NRED] = ok ? sh.nred : 0;
    }
}

// Final row of every (token, k) of one 64-token chunk, one lane per token.  The loads of up to
// eight k at a time (chunk prefix, bitmap, instance count and the first two instances) are
// issued together, then the instance holding the pair is looked up.
constexpr int kDestBatch = 8;
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
    const long long nrows = (long long)w.R * w.C;
    for (int k0 = 0; k0 < w.K; k0 += kDestBatch) {
        int e[kDestBatch], g[kDestBatch], ni[kDestBatch];
        int4 i01[kDestBatch];
        int2 i2[kDestBatch];
#pragma unroll
        for (int b = 0; b < kDestBatch; ++b) {
            const int k = k0 + b;
            e[b] = k < w.K ? topk[pbase + k] : -1;
        }
#pragma unroll
        for (int b = 0; b < kDestBatch; ++b) {
            const bool v = !bad && (unsigned)e[b] < (unsigned)w.E;
            const int ee = v ? e[b] : 0;
            const int32_t* in = w.inst + (size_t)ee * kMaxR * 3;
            g[b] = v ? w.cnt[(size_t)ee * w.NCH + ch] + __popcll(w.bm[(size_t)ch * w.E + ee] & low) : -1;
            ni[b] = v ? min(w.ninst[ee], kMaxR) : 0;
            i01[b] = v ? *reinterpret_cast<const int4*>(in) : make_int4(0, 0, 0, 0);
            i2[b] = v ? *reinterpret_cast<const int2*>(in + 4) : make_int2(0, 0);
        }
#pragma unroll
        for (int b = 0; b < kDestBatch; ++b) {
            const int k = k0 + b;
            if (k >= w.K) break;
            int d = -1;
            if (g[b] >= 0) {
                // instances 0 (home) and 1 come from the batch loads, later ones from memory
                if (ni[b] > 0 && g[b] >= i01[b].x && g[b] < i01[b].x + i01[b].y) {
                    d = i01[b].z + g[b];
                } else if (ni[b] > 1 && g[b] >= i01[b].w && g[b] < i01[b].w + i2[b].x) {
                    d = i2[b].y + g[b];
                } else {
                    const int32_t* in = w.inst + (size_t)e[b] * kMaxR * 3;
                    for (int i = 2; i < ni[b]; ++i) {
                        const int st = in[i * 3], rows = in[i * 3 + 1];
                        if (g[b] >= st && g[b] < st + rows) {
                            d = in[i * 3 + 2] + g[b];
                            break;
                        }
                    }
                }
                if (d < 0 || d >= nrows) d = -1;
            }
            dest[pbase + k] = d;
        }
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
    static const bool decide_smem_ok =
        hipFuncSetAttribute(reinterpret_cast<const void*>(plan_decide), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sizeof(DecideShared)) == hipSuccess;
    if (!decide_smem_ok) return MOONEP_EHIP;
    hipLaunchKernelGGL(plan_decide, dim3(1), dim3(kDecideThreads), sizeof(DecideShared), s, w, dims->flags,
                       cu_seqlens, stats);
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
