// Online redundant-expert planning on the GPU.
//
// Pages cited: [TC] thakicloud.com "The Busiest Rank Sets Your Step Time: Running
// MoonEP's Planning Code Ourselves"; [TD] twodots.gr "MoonEP balances AI experts in
// MoE models ..."; [AL] agentlenshq.com "MoonshotAI/MoonEP".
//
// The planner reads the router's top-K choices and decides, with no host
// synchronisation, which experts get a temporary copy on which rank so that every
// rank serves exactly C = S*K rows [TC, "What the technique is" and its flowchart;
// TD, summary; AL, How it works].  Three launches:
//
//   plan_hist   one workgroup per segment of up to 8 consecutive 64-token chunks, one wave per
//               chunk (its topk loads issued before its atomics): an LDS bitmap per chunk and
//               expert (bit t = token t of the chunk picked the expert), built with LDS atomic
//               OR (order-free, so the result is deterministic); per expert, the exclusive
//               prefix of the chunk popcounts within the segment and the segment total.  A bit
//               already set flags a duplicate expert within a token.
//   plan_decide one workgroup: expert loads L[e] (sums of the segment totals) and each
//               segment's offset per expert, rank loads, donors/receivers, the duplicate chain
//               with best-fit picks done as wave-wide minima (at most one remote home group per
//               rank [TC, Installation and integration]), prefetch slots or home-row fallback
//               [TD, memory contract], cu_seqlens per rank and weight row, instance offsets,
//               GEMM group tables and statistics.
//   plan_dest   one wave per chunk: pair index g = segment offset + prefix within the segment
//               + popcount of the lower bits of the expert's bitmap; the instance holding g
//               gives the final row (the send side computes the receiver's position [TC, "What
//               the technique is"]).
//
// Ties always go to the lower rank / expert id; integer arithmetic only, so the
// result is bit-identical from run to run.
#include <climits>
#include <mutex>

#include "common.h"

namespace moonep {

constexpr int kBad = MOONEP_ST_BAD_ID | MOONEP_ST_DUP_ID | MOONEP_ST_CAPACITY | MOONEP_ST_OVERFLOW;

// One workgroup per segment of SEG consecutive chunks (in (rank, token) order), one wave per
// chunk (with more chunks than waves a wave takes several, its topk loads for all of them issued
// before any chunk's atomics): LDS bitmaps per chunk and expert (bit t = token t of the chunk
// picked the expert), built with LDS atomic OR (order-free, so the result is deterministic).
// Then, per expert, the exclusive prefix of the popcounts over the segment's chunks and the
// segment total.  A bit already set flags a duplicate expert within a token.
constexpr int kHistWaves = kSegMax < 16 ? kSegMax : 16, kHistThreads = 64 * kHistWaves;
constexpr int kHistRounds = (kSegMax + kHistWaves - 1) / kHistWaves;
__global__ __launch_bounds__(kHistThreads) void plan_hist(const int32_t* __restrict__ topk, PlanWs w) {
    extern __shared__ unsigned long long sbm[];   // [SEG][E]
    __shared__ int sst;
    const int seg = blockIdx.x;
    const int ch0 = seg * w.SEG, nch = min(w.SEG, w.NCH - ch0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = w.E, K = w.K;
    for (int i = tid; i < nch * E; i += kHistThreads) sbm[i] = 0ull;
    if (tid == 0) sst = 0;
    // this wave's chunks: the ids of its tokens' picks, all loads in flight together
    int ev[kHistRounds][kMaxK];
#pragma unroll
    for (int rd = 0; rd < kHistRounds; ++rd) {
        const int cl = wave + rd * kHistWaves;
        const int ch = ch0 + cl;
        const int r = ch / w.NC, c = ch % w.NC;
        const int s = c * kChunk + lane;
        const bool on = cl < nch && s < w.S;
        const int32_t* tp = on ? topk + ((size_t)r * w.S + s) * K : topk;
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) ev[rd][k] = on && k < K ? tp[k] : -1;
    }
    __syncthreads();
    int st = 0;
#pragma unroll
    for (int rd = 0; rd < kHistRounds; ++rd) {
        const int cl = wave + rd * kHistWaves;
        const int s = ((ch0 + cl) % w.NC) * kChunk + lane;
        if (cl >= nch || s >= w.S) continue;
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            if (k >= K) break;
            const int e = ev[rd][k];
            if ((unsigned)e >= (unsigned)E) {
                st |= MOONEP_ST_BAD_ID;
                continue;
            }
            const unsigned long long old = atomicOr(&sbm[cl * E + e], 1ull << lane);
            if ((old >> lane) & 1ull) st |= MOONEP_ST_DUP_ID;
        }
    }
    if (st) atomicOr(&sst, st);
    __syncthreads();
    // per expert: the segment's bitmaps read eight chunks at a time, then written out with the
    // running prefix
    for (int e = tid; e < E; e += kHistThreads) {
        int run = 0;
        for (int c0 = 0; c0 < nch; c0 += 8) {
            unsigned long long bv[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) bv[b] = c0 + b < nch ? sbm[(c0 + b) * E + e] : 0ull;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                if (c0 + b >= nch) break;
                const size_t o = (size_t)(ch0 + c0 + b) * E + e;
                w.bm[o] = bv[b];
                w.cnt[o] = run;
                run += __popcll(bv[b]);
            }
        }
        w.segtot[(size_t)seg * E + e] = run;
    }
    if (tid == 0) w.chunk_status[seg] = sst;
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

// Wave-wide sum, the same exchanges as wave_reduce.  Every lane must be active.
__device__ __forceinline__ int wave_sum(int v) {
    v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// Wave-wide unsigned minimum, the same exchanges as wave_reduce.
__device__ __forceinline__ unsigned wave_reduce_u32(unsigned v) {
    auto mn = [](unsigned a, unsigned b) { return a < b ? a : b; };
    v = mn(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
    v = mn(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
    v = mn(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
    v = mn(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
    return mn(mn((unsigned)__builtin_amdgcn_readlane((int)v, 0), (unsigned)__builtin_amdgcn_readlane((int)v, 16)),
              mn((unsigned)__builtin_amdgcn_readlane((int)v, 32), (unsigned)__builtin_amdgcn_readlane((int)v, 48)));
}

// lowest lane whose flag is set (flags wave-uniformly nonzero)
__device__ __forceinline__ int first_lane(bool f) {
    return __builtin_ctzll(__ballot(f));
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations, not for its global
// stores (which __syncthreads' fence would wait for; no phase of plan_decide reads what an earlier
// one stored to global memory).
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wave barrier for a data exchange between the lanes of one wave through LDS: this wave's LDS
// operations complete, and the compiler moves no memory access across it.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// Per-expert replica counters, packed: all replicas (bits 0-9), slot replicas (10-19),
// fallback replicas (20-29).  An expert has at most R - 1 < 1024 replicas.
constexpr int kCntAll = 1, kCntSlot = 1 << 10, kCntFb = 1 << 20;

constexpr int kDecideThreadsMax = 512;

struct DecideShared {
    int L[kMaxE];                 // rows routed to each expert
    int avail[kMaxE];             // rows not (yet) given to a replica; keep[] after the chain
    int ecnt[kMaxE];              // packed replica counters of each expert
    // plan entries (replicas) in creation order
    // (e, q, a, j): expert, rank, rows, creation index among rank q's entries (slot E+j if j < B)
    int4 ent[kMaxE];
    // (pre, k): rows of e given to earlier replicas of e; index among e's replicas | index among
    // those of its kind << 16
    int2 ent2[kMaxE];
    // the entries on each rank by creation index: (entry id, weight row, rows, expert)
    int4 rank_e[kMaxR][kMaxG];
    int rank_n[kMaxR];            // entries on each rank
    int homepre[kMaxE];           // rows kept by the experts of e's home group before e
    int nzpre[kMaxE];             // experts of e's home group before e that keep rows
    int hometot[kMaxR];           // rows kept by each rank's home group
    int nzbase[kMaxR + 1];        // experts that keep rows in the home groups before each rank
    int P[kMaxR], X[kMaxR], don[kMaxR], rec[kMaxR];
    int lpart[kDecideThreadsMax];  // partial expert loads (segments split over threads)
    int nent, status;
};

// Rows on rank q whose weight row is below w, i.e. cu_seqlens[q][w] (home rows in expert order,
// then the rank's replicas by weight row), from the home prefix and the rank's few replicas.
__device__ __forceinline__ int cu_at(const DecideShared& sh, int q, int w, int E, int G, int B) {
    const int h0 = q * G;
    int s = w <= h0 ? 0 : w >= h0 + G ? sh.hometot[q] : sh.homepre[w];
    const int n = sh.rank_n[q];
    for (int j = 0; j < n; ++j) {
        const int4 r = sh.rank_e[q][j];
        s += r.y < w ? r.z : 0;
    }
    return s;
}

constexpr int kDecideThreads = kDecideThreadsMax;

__global__ __launch_bounds__(kDecideThreads) void plan_decide(PlanWs w, uint32_t flags, int32_t* __restrict__ cu,
                                                              int32_t* __restrict__ stats) {
    extern __shared__ __attribute__((aligned(16))) char decide_smem[];
    DecideShared& sh = *reinterpret_cast<DecideShared*>(decide_smem);
    constexpr int NT = kDecideThreads, NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = w.R, E = w.E, B = w.B, G = w.G, C = w.C;
    const int ncu = E + B + 1;
    // expert loads L[e] = sum of the segment totals.  With E <= 512 the segments of an expert are
    // split over 512/E threads (strided), whose partial sums meet in LDS; the loads are only summed
    // here, so they are in flight together (the segment offsets are stored during the chain).
    int st = tid < w.NSEG ? w.chunk_status[tid] : 0;   // (more segments: below)
    const int P = E <= NT ? min(NT / E, 8) : 1;
    if (E <= NT) {
        const int e = tid % E, part = tid / E;
        if (part < P) {
            int l = 0;
            for (int s0 = part; s0 < w.NSEG; s0 += 32 * P) {
                int v[32];
#pragma unroll
                for (int b = 0; b < 32; ++b) v[b] = w.segtot[(size_t)min(s0 + b * P, w.NSEG - 1) * E + e];
#pragma unroll
                for (int b = 0; b < 32; ++b) l += s0 + b * P < w.NSEG ? v[b] : 0;
            }
            sh.lpart[tid] = l;
        }
    } else {
        for (int e = tid; e < E; e += NT) {
            int l = 0;
#pragma unroll 16
            for (int sg = 0; sg < w.NSEG; ++sg) l += w.segtot[(size_t)sg * E + e];
            sh.L[e] = l;
        }
    }
    for (int i = tid + NT; i < w.NSEG; i += NT) st |= w.chunk_status[i];
    if (tid == 0) {
        sh.status = 0;
        sh.nent = 0;
    }
    if (tid < R) sh.rank_n[tid] = 0;
    lds_sync();
    if (st) atomicOr(&sh.status, st);
    for (int e = tid; e < E; e += NT) {
        int l = 0;
        if (E <= NT) {
            for (int p = 0; p < P; ++p) l += sh.lpart[p * E + e];
            sh.L[e] = l;
        } else {
            l = sh.L[e];
        }
        sh.avail[e] = l;
        sh.ecnt[e] = 0;
    }
    lds_sync();

    // rank loads P[q] = rows wanting q's home group, X[q] = P[q] - C (one wave per rank, G <= 64)
    for (int q = wave; q < R; q += NW) {
        const int p = wave_sum(lane < G ? sh.L[q * G + lane] : 0);
        if (lane == 0) {
            sh.P[q] = p;
            sh.X[q] = p - C;
        }
    }
    lds_sync();

    // the duplicate chain, on wave 0; lane i holds the remaining rows of the donor's expert i
    if (wave == 0 && !(sh.status & kBad)) {
        // donors by excess desc, receivers by deficit desc, ties to the lower rank: lane q counts
        // the ranks of its kind ahead of it and writes its rank id there; the lanes then read each
        // other's entries, after a wave barrier (a data exchange between lanes through LDS)
        const int xq = lane < R ? sh.X[lane] : 0;
        {
            int pos = 0;
            for (int q = 0; q < R; ++q) {
                const int y = __builtin_amdgcn_readlane(xq, q);
                pos += xq > 0 ? (y > xq || (y == xq && q < lane)) : (y < xq || (y == xq && q < lane));
            }
            if (xq > 0) sh.don[pos] = lane;
            else if (xq < 0) sh.rec[pos] = lane;
        }
        wave_lds_sync();
        int fail = 0;
        int nent = 0;
        // The donor group d being shipped from: lane i holds expert d*G+i's remaining rows (av),
        // load (lv) and packed replica counters (cnt).  Every ship call of one donor iteration
        // ships from that donor, so the group stays in registers for the whole iteration.
        int av = 0, lv = 0, cnt = 0;
        auto take_group = [&](int d) {
            const int e = d * G + lane;
            av = lane < G ? sh.avail[e] : 0;
            lv = lane < G ? sh.L[e] : 0;
            cnt = lane < G ? sh.ecnt[e] : 0;
        };
        auto put_group = [&](int d) {
            if (lane < G) {
                sh.avail[d * G + lane] = av;
                sh.ecnt[d * G + lane] = cnt;
            }
        };
        // ship(d, t, amt): amt rows of donor group d's experts to rank t, best fit first.  Every
        // rank receives from one ship call only, so the entries this call makes on t are t's
        // entries j = 0, 1, ... in creation order; entry j is kept in lane j's registers and all
        // are written after the call.
        auto ship = [&](int d, int t, int amt) {
            int j = 0;
            int my_e = 0, my_a = 0, my_pre = 0, my_k = 0;
            while (amt > 0 && !fail) {
                // One unsigned minimum picks both ways: an expert that covers amt keys by its
                // rows (best fit: fewest rows, ties to the lower id); one that does not keys above
                // every covering key, by amt-1-av (most rows first, ties to the lower id).
                const unsigned key = lane >= G ? 0xFFFFFFFFu
                                     : av >= amt ? (unsigned)av
                                                 : 0x80000000u | (unsigned)(amt - 1 - av);
                const unsigned m = wave_reduce_u32(key);
                const int pick = first_lane(key == m);
                const int got = (m & 0x80000000u) ? amt - 1 - (int)(m & 0x7FFFFFFFu) : (int)m;
                const int a = got < amt ? got : amt;
                if (a <= 0 || nent + j >= E || j >= kMaxG) {
                    fail = a <= 0 ? MOONEP_ST_CAPACITY : MOONEP_ST_OVERFLOW;
                    break;
                }
                // the picked expert's counters and the rows it gave earlier replicas
                const int pc = __builtin_amdgcn_readlane(cnt, pick);
                const int pre = __builtin_amdgcn_readlane(lv - av, pick);
                const bool slot = j < B;
                const int kind = slot ? (pc >> 10) & 0x3FF : (pc >> 20) & 0x3FF;
                const int kcode = (pc & 0x3FF) | (kind << 16), ecode = d * G + pick;
                const int inc = kCntAll + (slot ? kCntSlot : kCntFb);
                const bool mine = lane == j, picked = lane == pick;
                my_e = mine ? ecode : my_e;
                my_a = mine ? a : my_a;
                my_pre = mine ? pre : my_pre;
                my_k = mine ? kcode : my_k;
                cnt += picked ? inc : 0;
                av -= picked ? a : 0;
                ++j;
                amt -= a;
            }
            if (lane < j) {
                const int i = nent + lane;
                sh.ent[i] = make_int4(my_e, t, my_a, lane);
                sh.ent2[i] = make_int2(my_pre, my_k);
                sh.rank_e[t][lane] = make_int4(i, lane < B ? E + lane : my_e, my_a, my_e);
            }
            if (lane == 0) sh.rank_n[t] = j;
            nent += j;
        };
        const int nd = __popcll(__ballot(xq > 0)), nr = __popcll(__ballot(xq < 0));
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
                take_group(d);
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
                put_group(d);
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
                take_group(d);
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
                put_group(d);
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
    } else if (wave % 4 != 0) {
        // meanwhile, on the waves that do not share wave 0's SIMD: each segment's offset per
        // expert (pairs of e in the earlier segments), for plan_dest; 32 segments' totals are
        // loaded before their offsets are stored
        constexpr int kHelpers = NT - NT / 4;
        const int hid = (wave - 1 - wave / 4) * 64 + lane;
        for (int e = hid; e < E; e += kHelpers) {
            int l = 0;
            for (int s0 = 0; s0 < w.NSEG; s0 += 32) {
                // unconditional loads (segments past the end re-read the last one), all in flight
                int v[32];
#pragma unroll
                for (int b = 0; b < 32; ++b) v[b] = w.segtot[(size_t)min(s0 + b, w.NSEG - 1) * E + e];
                const int nb = min(32, w.NSEG - s0);
#pragma unroll
                for (int b = 0; b < 32; ++b) {
                    if (b < nb) w.segpre[(size_t)(s0 + b) * E + e] = l;
                    l += b < nb ? v[b] : 0;
                }
            }
        }
    }
    lds_sync();

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
    lds_sync();
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
    lds_sync();
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
            const int4 r = sh.rank_e[q][jj];
            e = r.w;
            row0 = q * C + cu_at(sh, q, E + jj, E, G, B);
            rows = r.z;
        }
        w.slot_e[i] = e;
        w.slot_row0[i] = row0;
        w.slot_rows[i] = rows;
    }
    // zero row segment read by masked GEMM tile loads
    for (int i = tid; i < kZeroElems / 2; i += NT) reinterpret_cast<uint32_t*>(w.zeros)[i] = 0u;
    lds_sync();

    // per entry: its instance, reduce slot or fallback segment, GEMM group
    const int nhome = sh.nzbase[R];
    for (int i = tid; i < nent; i += NT) {
        const int4 en4 = sh.ent[i];
        const int2 en2 = sh.ent2[i];
        const int e = en4.x, q = en4.y, a = en4.z, jj = en4.w;
        const int k = en2.y & 0xFFFF, kk = en2.y >> 16;
        const int wr = jj < B ? E + jj : e;
        const int row0 = q * C + cu_at(sh, q, wr, E, G, B);
        const int stt = sh.avail[e] + en2.x;      // home rows first, then replicas in order
        int32_t* in = w.inst + ((size_t)e * kMaxR + 1 + k) * 3;
        in[0] = stt;
        in[1] = a;
        in[2] = row0 - stt;
        if (wr >= E) {
            w.red_slot[(size_t)e * kMaxR + kk] = q * B + jj;
        } else {
            w.fb_seg[(size_t)e * kMaxR + kk] = Segment{row0, a};
        }
        int32_t* en = w.entries + (size_t)i * 5;
        en[0] = e;
        en[1] = q;
        en[2] = a;
        en[3] = jj;
        en[4] = wr;
        w.groups[nhome + i] = Group{row0, a, wr < E ? wr : -1 - (q * B + jj), e};
    }
    // cu_seqlens: rows of rank q whose weight row is below p; one wave per rank, lanes over p, the
    // rank's few replicas (weight row, rows) taken from lanes of a register
    for (int q = wave; q < R; q += NW) {
        const int n = ok ? sh.rank_n[q] : 0;
        const int4 rl = lane < n ? sh.rank_e[q][lane] : make_int4(0, 0, 0, 0);
        const int lw = rl.y, la = rl.z;
        const int h0 = q * G, ht = sh.hometot[q];
        for (int p = lane; p < ncu; p += 64) {
            int c = p <= h0 ? 0 : p >= h0 + G ? ht : sh.homepre[p];
            for (int j = 0; j < n; ++j)
                c += __builtin_amdgcn_readlane(lw, j) < p ? __builtin_amdgcn_readlane(la, j) : 0;
            cu[(size_t)q * ncu + p] = ok ? c : 0;
        }
    }
    lds_sync();

    // statistics, on wave 0: sums over the entries, the experts and the ranks
    if (wave == 0) {
        int migr = 0, nsf = 0, fbrows = 0, nred = 0, maxl = 0;
        for (int i = lane; i < nent; i += 64) {
            const int4 en4 = sh.ent[i];
            const int a = en4.z;
            const bool slot = en4.w < B;
            migr += a;
            nsf += slot ? 1 : 1 << 16;       // slot replicas | fallback replicas << 16
            fbrows += slot ? 0 : a;
        }
        for (int e = lane; e < E; e += 64) {
            nred += ok && ((sh.ecnt[e] >> 10) & 0x3FF) > 0;
            maxl = max(maxl, sh.L[e]);
        }
        const int x = lane < R ? sh.X[lane] : 0, pr = lane < R ? sh.P[lane] : 0;
        migr = wave_sum(migr);
        nsf = wave_sum(nsf);
        fbrows = wave_sum(fbrows);
        nred = wave_sum(nred);
        maxl = wave_reduce<true>(maxl);
        const int bound = wave_sum(x > 0 ? x : 0);
        const int maxp = wave_reduce<true>(lane < R ? pr : INT_MIN);
        const int minp = wave_reduce<false>(lane < R ? pr : INT_MAX);
        const int maxper = ok ? wave_reduce<true>(lane < R ? sh.rank_n[lane] : 0) : 0;
        const int nd = __popcll(__ballot(x > 0)), nr = __popcll(__ballot(x < 0));
        const int nslot = nsf & 0xFFFF, nfb = nsf >> 16;
        int status = sh.status;
        if (ok && nfb > 0 && (flags & MOONEP_TRAINING)) status |= MOONEP_ST_TRAIN_FALLBACK;
        if (lane == 0) {
            const int v[MOONEP_NSTATS] = {status, nent, nslot, nfb, fbrows, migr, bound, maxl,
                                          maxp, minp, nd, nr, maxper, ok ? R * C : 0, 0, 0};
            for (int i = 0; i < MOONEP_NSTATS; ++i) stats[i] = v[i];
            w.hdr[HDR_STATUS] = status;
            w.hdr[HDR_NENTRIES] = nent;
            w.hdr[HDR_NGROUPS] = ok ? nhome + nent : 0;
            w.hdr[HDR_NSLOTREP] = nslot;
            w.hdr[HDR_NRED] = ok ? nred : 0;
        }
    }
}

// Final row of every (token, k) of one 64-token chunk, one lane per token.  The loads of up to
// eight k at a time (chunk prefix, bitmap, instance count and the first two instances) are
// issued together, then the instance holding the pair is looked up.
constexpr int kDestBatch = 8;
__global__ __launch_bounds__(64) void plan_dest(const int32_t* __restrict__ topk, PlanWs w,
                                                int32_t* __restrict__ dest) {
    const int ch = blockIdx.x;
    const int r = ch / w.NC, c = ch % w.NC, seg = ch / w.SEG;
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
            g[b] = v ? w.segpre[(size_t)seg * w.E + ee] + w.cnt[(size_t)ch * w.E + ee] +
                           __popcll(w.bm[(size_t)ch * w.E + ee] & low)
                     : -1;
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
    hipLaunchKernelGGL(plan_hist, dim3(w.NSEG), dim3(kHistThreads), (size_t)w.SEG * w.E * 8, s, topk, w);
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
