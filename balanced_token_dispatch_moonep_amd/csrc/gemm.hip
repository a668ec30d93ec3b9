// Grouped SwiGLU expert GEMM (forward and backward) on gfx950 matrix cores.
//
// Pages cited: [TC] thakicloud.com "The Busiest Rank Sets Your Step Time: Running
// MoonEP's Planning Code Ourselves"; [TD] twodots.gr "MoonEP balances AI experts in
// MoE models ...".
//
// The grouped GEMM reads the zero-copy receive buffer in place; the planner's groups
// (rank q, weight row w, cu_seqlens range) select the active rows and the weight row
// [TC, flowchart "Group GEMM" and Installation and integration; TD, memory contract].
// Home and fallback groups read the home weight row, slot groups the prefetched copy.
// Replica weight gradients go to the separate fp32 reduce buffer [TD, memory contract].
//
// Kernel design (MI355X / CDNA4):
//   * 256x256 output tile per workgroup, 4 waves in 2x2, each wave 128x128 = 4x4 tiles
//     of v_mfma_f32_32x32x16_bf16 (bf16 inputs, fp32 accumulation).  K step 64.
//   * Operands staged through LDS in a k-contiguous layout with a 16-byte row pad
//     (conflict-free 128-bit fragment reads), double-buffered: global loads of step
//     k+1 are in flight while the MFMAs of step k run; one barrier per step.
//   * Operands stored k-contiguous in HBM are copied as 16-byte rows; operands stored
//     m/n-contiguous (weights in the forward, both operands of dW) are loaded as 8x8
//     bf16 blocks and transposed in registers with v_perm_b32 before the LDS store.
//   * Persistent grid (one workgroup per CU).  Tiles are ordered group-major, then
//     n-tile, then m-tile, and each XCD (blockIdx % 8) takes a contiguous range of them,
//     so the tiles that share a weight panel or an activation panel run on the same XCD
//     at the same time and hit its L2.
//   * Epilogues are fused: SwiGLU (act = silu(gate) * up, with Gt|U saved) after the
//     gate/up GEMM; SwiGLU' (dGt, dU written over the saved Gt|U) after dA = dY W2^T;
//     fp32 accumulate into the home or reduce-buffer gradient for dW.
#include "common.h"

namespace moonep {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDK = BK + 8;                  // LDS row pitch (bf16 elements): 144 bytes
constexpr int TILE_ELEMS = BM * LDK;         // one operand, one stage
constexpr int GEMM_SMEM = 4 * TILE_ELEMS * 2;  // 2 stages x (A, B), bytes = 147456
constexpr int MAX_GROUPS = 2 * kMaxE;

enum Epi { EPI_SWIGLU_FWD = 0, EPI_STORE = 1, EPI_SWIGLU_BWD = 2, EPI_ACC_F32 = 3 };
enum BMode { B_NCONTIG = 0, B_KCONTIG = 1 };

struct GemmArgs {
    PlanWs w;
    const uint16_t* A;        // rows modes: activations [R*C, lda]; dW: [R*C, lda] read transposed
    int lda;
    const uint16_t* B;        // dW: [R*C, ldb] read transposed
    const uint16_t* Bhome;    // rows modes: weights, home rows [E, ...]
    const uint16_t* Bslot;    //             slot rows [R*B, ...]
    long long bstride;        // elements per weight row
    int ldb;
    int M, N, K;              // dW: output M x N; rows modes: N output cols, K reduction
    int I;                    // SwiGLU split
    uint16_t* out;            // EPI_STORE / EPI_SWIGLU_FWD (act): bf16 [R*C, ldo]
    int ldo;
    uint16_t* gu;             // SwiGLU: [R*C, 2I]
    float* dw_home;           // EPI_ACC_F32: [E, M, N]
    float* dw_slot;           // EPI_ACC_F32: [R*B, M, N]
    int ntiles_n;
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// k-contiguous operand: tile row r (0..255) at src + r*ld, columns k0..k0+63 already in src.
__device__ __forceinline__ void load_kc(uint4 (&v)[8], const uint16_t* src, int ld, int nvalid, int tid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = i * 256 + tid;
        const int r = c >> 3, kc = c & 7;
        v[i] = r < nvalid ? *reinterpret_cast<const uint4*>(src + (size_t)r * ld + kc * 8) : zero4();
    }
}
__device__ __forceinline__ void store_kc(const uint4 (&v)[8], uint16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = i * 256 + tid;
        const int r = c >> 3, kc = c & 7;
        *reinterpret_cast<uint4*>(lds + r * LDK + kc * 8) = v[i];
    }
}

// m/n-contiguous operand: this thread's 8x8 block = k rows kb*8..+7 (src points at row kb*8,
// column of the block), kvalid rows of the step are real.
__device__ __forceinline__ void load_t(uint4 (&v)[8], const uint16_t* src, int ld, int kvalid, bool ok) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = (ok && i < kvalid) ? *reinterpret_cast<const uint4*>(src + (size_t)i * ld) : zero4();
}
// transpose the 8x8 bf16 block in registers and store 8 k-contiguous 16-byte rows
__device__ __forceinline__ void store_t(const uint4 (&v)[8], uint16_t* lds, int tid) {
    const int kb = tid >> 5, mb = tid & 31;
    uint32_t in[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        in[i][0] = v[i].x;
        in[i][1] = v[i].y;
        in[i][2] = v[i].z;
        in[i][3] = v[i].w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint4 o;
        o.x = __builtin_amdgcn_perm(in[1][j >> 1], in[0][j >> 1], sel);
        o.y = __builtin_amdgcn_perm(in[3][j >> 1], in[2][j >> 1], sel);
        o.z = __builtin_amdgcn_perm(in[5][j >> 1], in[4][j >> 1], sel);
        o.w = __builtin_amdgcn_perm(in[7][j >> 1], in[6][j >> 1], sel);
        *reinterpret_cast<uint4*>(lds + (mb * 8 + j) * LDK + kb * 8) = o;
    }
}

// LDS column (tile n index) of wave-local MFMA column tile tj.
template <int EPI>
__device__ __forceinline__ int bcol(int wn, int tj) {
    if (EPI == EPI_SWIGLU_FWD) return tj < 2 ? wn * 64 + tj * 32 : 128 + wn * 64 + (tj - 2) * 32;
    return wn * 128 + tj * 32;
}

template <int EPI>
__device__ __forceinline__ void mma_step(f32x16_t (&acc)[4][4], const uint16_t* As, const uint16_t* Bs,
                                         int wm, int wn, int lane) {
    const int lr = lane & 31, lk = (lane >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            af[t] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 128 + t * 32 + lr) * LDK + kk * 16 + lk);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bfr[t] = *reinterpret_cast<const bf16x8_t*>(Bs + (bcol<EPI>(wn, t) + lr) * LDK + kk * 16 + lk);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
}

// Rows of a plan group, or 0 if the descriptor is out of range (never for a valid plan).
__device__ __forceinline__ int group_rows(const Group& g, const PlanWs& w) {
    const long long total = (long long)w.R * w.C;
    const bool ok = g.row0 >= 0 && g.rows >= 0 && (long long)g.row0 + g.rows <= total &&
                    g.wsel < w.E && (g.wsel >= 0 || -1 - g.wsel < w.R * w.B);
    return ok ? g.rows : 0;
}
__device__ __forceinline__ bool seg_ok(const Segment& s, const PlanWs& w) {
    return s.row0 >= 0 && s.rows >= 0 && (long long)s.row0 + s.rows <= (long long)w.R * w.C;
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f2bf16(float f) { return (uint16_t)f2bf(f); }
__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ---------------------------------------------------------------------------
// Epilogues.  The tile's accumulators are staged through LDS (each wave owns a
// 64 x 128 fp32 region, two halves per tile), then every lane handles 8 (or 4)
// consecutive columns so global stores are 16 bytes wide and row-contiguous.
// C layout of a 32x32 MFMA tile: lane l, reg r -> row (r/4)*8 + (l/32)*4 + r%4, col l%32.
// ---------------------------------------------------------------------------
constexpr int EPL = 132;   // fp32 pitch of a staged row (128 + 4 pad)

template <int h>
__device__ __forceinline__ void stage_half(const f32x16_t (&acc)[4][4], float* ep, int lane) {
    const int lc = lane & 31, lr4 = (lane >> 5) * 4;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                ep[(ii * 32 + (r >> 2) * 8 + lr4 + (r & 3)) * EPL + j * 32 + lc] = acc[2 * h + ii][j][r];
}

__device__ __forceinline__ uint4 pack8(const float (&v)[8]) {
    return make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
}
__device__ __forceinline__ void unpack8(uint4 u, float (&v)[8]) {
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}
__device__ __forceinline__ void read8(const float* p, float (&v)[8]) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}

template <int EPI, int h>
__device__ __forceinline__ void epilogue_rows_half(const GemmArgs& a, const f32x16_t (&acc)[4][4], uint16_t* smem,
                                                   int wm, int wn, int lane, int nt, int row0, int mvalid) {
    float* ep = reinterpret_cast<float*>(smem) + (wm * 2 + wn) * 64 * EPL;
    {
        stage_half<h>(acc, ep, lane);
        __syncthreads();
        const int rbase = wm * 128 + h * 64;   // tile-local row of the region's first row
        if (EPI == EPI_SWIGLU_FWD) {
            // region columns 0..63 = gate, 64..127 = up, for act columns nt*128 + wn*64 + c
            const int I = a.I;
            const int c = (lane & 7) * 8;
            const int col = nt * 128 + wn * 64 + c;
            for (int it = 0; it < 8; ++it) {
                const int rr = it * 8 + (lane >> 3);
                if (rbase + rr >= mvalid || col >= I) continue;
                float g[8], u[8], o[8];
                read8(ep + rr * EPL + c, g);
                read8(ep + rr * EPL + 64 + c, u);
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = g[i] * sigm(g[i]) * u[i];
                const size_t row = (size_t)(row0 + rbase + rr);
                *reinterpret_cast<uint4*>(a.out + row * a.ldo + col) = pack8(o);
                if (a.gu) {
                    *reinterpret_cast<uint4*>(a.gu + row * 2 * I + col) = pack8(g);
                    *reinterpret_cast<uint4*>(a.gu + row * 2 * I + I + col) = pack8(u);
                }
            }
        } else if (EPI == EPI_SWIGLU_BWD) {
            const int I = a.I;
            const int c = (lane & 15) * 8;
            const int col = nt * BN + wn * 128 + c;
            for (int it = 0; it < 16; ++it) {
                const int rr = it * 4 + (lane >> 4);
                if (rbase + rr >= mvalid || col >= I) continue;
                const size_t row = (size_t)(row0 + rbase + rr);
                uint4* pg = reinterpret_cast<uint4*>(a.gu + row * 2 * I + col);
                uint4* pu = reinterpret_cast<uint4*>(a.gu + row * 2 * I + I + col);
                float da[8], g[8], u[8], dg[8], du[8];
                read8(ep + rr * EPL + c, da);
                unpack8(*pg, g);
                unpack8(*pu, u);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float sg = sigm(g[i]);
                    dg[i] = da[i] * u[i] * sg * (1.0f + g[i] * (1.0f - sg));
                    du[i] = da[i] * g[i] * sg;
                }
                *pg = pack8(dg);
                *pu = pack8(du);
            }
        } else {
            const int c = (lane & 15) * 8;
            const int col = nt * BN + wn * 128 + c;
            for (int it = 0; it < 16; ++it) {
                const int rr = it * 4 + (lane >> 4);
                if (rbase + rr >= mvalid || col >= a.N) continue;
                float v[8];
                read8(ep + rr * EPL + c, v);
                *reinterpret_cast<uint4*>(a.out + (size_t)(row0 + rbase + rr) * a.ldo + col) = pack8(v);
            }
        }
        __syncthreads();
    }
}

template <int EPI>
__device__ __forceinline__ void epilogue_rows(const GemmArgs& a, const f32x16_t (&acc)[4][4], uint16_t* smem,
                                              int wm, int wn, int lane, int nt, int row0, int mvalid) {
    epilogue_rows_half<EPI, 0>(a, acc, smem, wm, wn, lane, nt, row0, mvalid);
    epilogue_rows_half<EPI, 1>(a, acc, smem, wm, wn, lane, nt, row0, mvalid);
}

template <int h>
__device__ __forceinline__ void epilogue_dw_half(const GemmArgs& a, const f32x16_t (&acc)[4][4], uint16_t* smem,
                                            int wm, int wn, int lane, float* out, int m0, int n0) {
    float* ep = reinterpret_cast<float*>(smem) + (wm * 2 + wn) * 64 * EPL;
    {
        stage_half<h>(acc, ep, lane);
        __syncthreads();
        const int c = (lane & 31) * 4;
        const int col = n0 + wn * 128 + c;
        for (int it = 0; it < 32; ++it) {
            const int rr = it * 2 + (lane >> 5);
            const int row = m0 + wm * 128 + h * 64 + rr;
            if (row >= a.M || col >= a.N) continue;
            const float4 v = *reinterpret_cast<const float4*>(ep + rr * EPL + c);
            float4* p = reinterpret_cast<float4*>(out + (size_t)row * a.N + col);
            float4 o = *p;
            o.x += v.x;
            o.y += v.y;
            o.z += v.z;
            o.w += v.w;
            *p = o;
        }
        __syncthreads();
    }
}

__device__ __forceinline__ void epilogue_dw(const GemmArgs& a, const f32x16_t (&acc)[4][4], uint16_t* smem,
                                            int wm, int wn, int lane, float* out, int m0, int n0) {
    epilogue_dw_half<0>(a, acc, smem, wm, wn, lane, out, m0, n0);
    epilogue_dw_half<1>(a, acc, smem, wm, wn, lane, out, m0, n0);
}

// ---------------------------------------------------------------------------
// Row-grouped GEMM: C[rows, N] = A[rows, K] * B_w[K, N] per plan group.
// ---------------------------------------------------------------------------
template <int EPI, int BMODE>
__global__ __launch_bounds__(256, 1) void gemm_rows_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    __shared__ int s_pref[MAX_GROUPS + 1];
    __shared__ int s_part[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const Group* groups = a.w.groups;
    const int ng = min(max(a.w.hdr[HDR_NGROUPS], 0), min(2 * a.w.E, MAX_GROUPS));

    // m-tiles per group -> prefix in LDS (each thread scans a contiguous slice)
    {
        const int per = (ng + 255) / 256;
        const int lo = tid * per;
        int sum = 0;
        for (int g = lo; g < lo + per && g < ng; ++g) sum += (group_rows(groups[g], a.w) + BM - 1) / BM;
        s_part[tid] = sum;
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int i = 0; i < 256; ++i) {
                const int v = s_part[i];
                s_part[i] = run;
                run += v;
            }
        }
        __syncthreads();
        int run = s_part[tid];
        for (int g = lo; g < lo + per && g < ng; ++g) {
            s_pref[g] = run;
            run += (group_rows(groups[g], a.w) + BM - 1) / BM;
        }
        if (tid == 255) s_pref[ng] = run;   // lo + per covers ng for the last thread
        __syncthreads();
        if (tid == 0 && ng == 0) s_pref[0] = 0;
        __syncthreads();
    }
    const int NT = a.ntiles_n;
    const int total = s_pref[ng] * NT;
    const int nxcd = 8;
    const int xcd = blockIdx.x % nxcd, li = blockIdx.x / nxcd, per_wg = gridDim.x / nxcd;
    const int chunk = (total + nxcd - 1) / nxcd;
    const int t_lo = xcd * chunk, t_hi = min(total, t_lo + chunk);

    uint16_t* As0 = smem;
    uint16_t* Bs0 = smem + TILE_ELEMS;
    uint16_t* As1 = smem + 2 * TILE_ELEMS;
    uint16_t* Bs1 = smem + 3 * TILE_ELEMS;

    for (int t = t_lo + li; t < t_hi; t += per_wg) {
        // decode tile -> group, n-tile, m-tile (binary search over the prefix)
        int lo = 0, hi = ng - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pref[mid] * NT <= t) lo = mid; else hi = mid - 1;
        }
        const int g = lo;
        const Group gr = groups[g];
        const int mtiles = s_pref[g + 1] - s_pref[g];
        const int local = t - s_pref[g] * NT;
        const int nt = local / mtiles, mt = local % mtiles;
        const int row0 = gr.row0 + mt * BM;
        const int mvalid = min(BM, group_rows(gr, a.w) - mt * BM);
        const uint16_t* W = gr.wsel >= 0 ? a.Bhome + (size_t)gr.wsel * a.bstride
                                         : a.Bslot + (size_t)(-1 - gr.wsel) * a.bstride;
        const uint16_t* Arow = a.A + (size_t)row0 * a.lda;

        // per-thread B addressing
        const uint16_t* Bsrc;
        bool bok = true;
        int bvalid = BN;
        if (BMODE == B_NCONTIG) {
            const int c = (tid & 31) * 8;      // tile column of this thread's 8x8 block
            int gcol;
            if (EPI == EPI_SWIGLU_FWD) {
                const int cc = nt * 128 + (c & 127);
                bok = cc < a.I;
                gcol = c < 128 ? cc : a.I + cc;
            } else {
                gcol = nt * BN + c;
                bok = gcol < a.N;
            }
            Bsrc = W + (size_t)((tid >> 5) * 8) * a.ldb + (bok ? gcol : 0);
        } else {
            Bsrc = W + (size_t)(nt * BN) * a.ldb;
            bvalid = min(BN, a.N - nt * BN);
        }

        f32x16_t acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        const int nsteps = a.K / BK;
        uint4 va[8], vb[8];
        load_kc(va, Arow, a.lda, mvalid, tid);
        if (BMODE == B_NCONTIG) load_t(vb, Bsrc, a.ldb, BK, bok);
        else load_kc(vb, Bsrc, a.ldb, bvalid, tid);
        store_kc(va, As0, tid);
        if (BMODE == B_NCONTIG) store_t(vb, Bs0, tid);
        else store_kc(vb, Bs0, tid);
        __syncthreads();
        for (int s = 0; s < nsteps; ++s) {
            const bool more = s + 1 < nsteps;
            if (more) {
                const int k0 = (s + 1) * BK;
                load_kc(va, Arow + k0, a.lda, mvalid, tid);
                if (BMODE == B_NCONTIG) load_t(vb, Bsrc + (size_t)k0 * a.ldb, a.ldb, BK, bok);
                else load_kc(vb, Bsrc + k0, a.ldb, bvalid, tid);
            }
            const uint16_t* Ac = (s & 1) ? As1 : As0;
            const uint16_t* Bc = (s & 1) ? Bs1 : Bs0;
            mma_step<EPI>(acc, Ac, Bc, wm, wn, lane);
            if (more) {
                uint16_t* An = (s & 1) ? As0 : As1;
                uint16_t* Bn = (s & 1) ? Bs0 : Bs1;
                store_kc(va, An, tid);
                if (BMODE == B_NCONTIG) store_t(vb, Bn, tid);
                else store_kc(vb, Bn, tid);
            }
            __syncthreads();
        }

        epilogue_rows<EPI>(a, acc, smem, wm, wn, lane, nt, row0, mvalid);
    }
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM: dW[M, N] += A^T B over the target's row segments, where
// A = [rows, M] and B = [rows, N] are both read row-major and transposed in registers.
// Targets: t < E home expert t (home rows + its fallback replicas), else slot t - E.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void gemm_dw_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const PlanWs& w = a.w;
    const int MT = (a.M + BM - 1) / BM, NT = a.ntiles_n;
    const int per_target = MT * NT;
    const int ntargets = w.E + w.R * w.B;
    const int total = ntargets * per_target;
    const int nxcd = 8;
    const int xcd = blockIdx.x % nxcd, li = blockIdx.x / nxcd, per_wg = gridDim.x / nxcd;
    const int chunk = (total + nxcd - 1) / nxcd;
    const int t_lo = xcd * chunk, t_hi = min(total, t_lo + chunk);

    uint16_t* As0 = smem;
    uint16_t* Bs0 = smem + TILE_ELEMS;
    uint16_t* As1 = smem + 2 * TILE_ELEMS;
    uint16_t* Bs1 = smem + 3 * TILE_ELEMS;

    for (int t = t_lo + li; t < t_hi; t += per_wg) {
        const int target = t / per_target;
        const int local = t % per_target;
        const int nt = local / MT, mt = local % MT;
        // row segments of this target: home rows then fallback replicas (home expert), or the slot's rows
        float* out;
        Segment first{0, 0};
        const Segment* extra = nullptr;   // further segments (fallback replicas), read from the plan
        int nseg = 0;
        if (target < w.E) {
            first = w.home_seg[target];
            extra = w.fb_seg + (size_t)target * kMaxR;
            if (!seg_ok(first, w)) first.rows = 0;
            nseg = (first.rows > 0 ? 1 : 0) + min(max(w.fb_n[target], 0), kMaxR - 1);
            if (first.rows == 0) {
                first = extra[0];
                ++extra;
            }
            out = a.dw_home + (size_t)target * a.M * a.N;
        } else {
            const int sl = target - w.E;
            if (w.slot_e[sl] < 0) continue;
            first = Segment{w.slot_row0[sl], w.slot_rows[sl]};
            if (!seg_ok(first, w)) continue;
            nseg = 1;
            out = a.dw_slot + (size_t)sl * a.M * a.N;
        }
        auto seg_at = [&](int i) -> Segment {
            const Segment sg = i == 0 ? first : extra[i - 1];
            return seg_ok(sg, w) ? sg : Segment{0, 0};
        };
        int nsteps = 0;
        for (int i = 0; i < nseg; ++i) nsteps += (seg_at(i).rows + BK - 1) / BK;
        if (nsteps == 0) continue;

        const int m0 = mt * BM, n0 = nt * BN;
        const int cblk = (tid & 31) * 8;
        const bool aok = m0 + cblk < a.M, bok = n0 + cblk < a.N;
        const int kb8 = (tid >> 5) * 8;

        f32x16_t acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // step iterator over segments
        int si = 0, sk = 0;   // segment index, row offset inside it
        uint4 va[8], vb[8];
        Segment cur = first;
        auto load_step = [&](int koff) {
            const Segment sg = cur;
            const int kvalid = min(BK, sg.rows - koff) - kb8;
            const size_t r0 = (size_t)(sg.row0 + koff + kb8);
            load_t(va, a.A + r0 * a.lda + (aok ? m0 + cblk : 0), a.lda, kvalid, aok);
            load_t(vb, a.B + r0 * a.ldb + (bok ? n0 + cblk : 0), a.ldb, kvalid, bok);
        };
        auto advance = [&]() {
            sk += BK;
            if (sk >= cur.rows) {
                ++si;
                sk = 0;
                if (si < nseg) cur = seg_at(si);
            }
        };
        load_step(sk);
        advance();
        store_t(va, As0, tid);
        store_t(vb, Bs0, tid);
        __syncthreads();
        for (int s = 0; s < nsteps; ++s) {
            const bool more = s + 1 < nsteps;
            if (more) {
                load_step(sk);
                advance();
            }
            mma_step<EPI_ACC_F32>(acc, (s & 1) ? As1 : As0, (s & 1) ? Bs1 : Bs0, wm, wn, lane);
            if (more) {
                store_t(va, (s & 1) ? As0 : As1, tid);
                store_t(vb, (s & 1) ? Bs0 : Bs1, tid);
            }
            __syncthreads();
        }

        epilogue_dw(a, acc, smem, wm, wn, lane, out, m0, n0);
    }
}

static int g_num_cu = 0;
static int num_cus() {
    if (g_num_cu <= 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_num_cu = n;
    }
    return g_num_cu;
}

template <typename K>
static bool set_smem(K kernel) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_SMEM) == hipSuccess;
}

static int launch_rows(int epi, int bmode, const GemmArgs& a, hipStream_t s) {
    const int grid = (num_cus() / 8) * 8;
#define MOONEP_ROWS(E_, B_)                                                         \
    do {                                                                            \
        static bool ok = set_smem(gemm_rows_kernel<E_, B_>);                        \
        if (!ok) return MOONEP_EHIP;                                                \
        hipLaunchKernelGGL((gemm_rows_kernel<E_, B_>), dim3(grid), dim3(256), GEMM_SMEM, s, a); \
    } while (0)
    if (epi == EPI_SWIGLU_FWD && bmode == B_NCONTIG) MOONEP_ROWS(EPI_SWIGLU_FWD, B_NCONTIG);
    else if (epi == EPI_STORE && bmode == B_NCONTIG) MOONEP_ROWS(EPI_STORE, B_NCONTIG);
    else if (epi == EPI_SWIGLU_BWD && bmode == B_KCONTIG) MOONEP_ROWS(EPI_SWIGLU_BWD, B_KCONTIG);
    else if (epi == EPI_STORE && bmode == B_KCONTIG) MOONEP_ROWS(EPI_STORE, B_KCONTIG);
    else return MOONEP_ENOTSUP;
#undef MOONEP_ROWS
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

static int launch_dw(const GemmArgs& a, hipStream_t s) {
    static bool ok = set_smem(gemm_dw_kernel);
    if (!ok) return MOONEP_EHIP;
    const int grid = (num_cus() / 8) * 8;
    hipLaunchKernelGGL(gemm_dw_kernel, dim3(grid), dim3(256), GEMM_SMEM, s, a);
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

static int check_ffn_dims(const moonep_dims_t* d) {
    int rc = check_dims(d, true);
    if (rc != MOONEP_OK) return rc;
    if (d->flags & MOONEP_F32_ROWS) return MOONEP_ENOTSUP;   // the expert GEMM is bf16
    if (d->H % BK != 0 || d->I % BK != 0) return MOONEP_ENOTSUP;
    return MOONEP_OK;
}

}  // namespace moonep

using namespace moonep;

extern "C" int moonep_grouped_ffn(const moonep_dims_t* dims, const void* plan_ws, const int32_t* cu_seqlens,
                                  const void* recv, const void* w13_home, const void* w2_home,
                                  const void* w13_slot, const void* w2_slot, void* gu_save, void* act,
                                  void* y, void* stream) {
    int rc = check_ffn_dims(dims);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(plan_ws);
    MOONEP_CHECK_PTR(cu_seqlens);
    MOONEP_CHECK_PTR(recv);
    MOONEP_CHECK_PTR(w13_home);
    MOONEP_CHECK_PTR(w2_home);
    MOONEP_CHECK_PTR(act);
    MOONEP_CHECK_PTR(y);
    if (dims->B > 0) {
        MOONEP_CHECK_PTR(w13_slot);
        MOONEP_CHECK_PTR(w2_slot);
    }
    if (gu_save && !aligned16(gu_save)) return MOONEP_EALIGN;
    const int H = dims->H, I = dims->I;
    hipStream_t s = static_cast<hipStream_t>(stream);
    GemmArgs a{};
    plan_ws_layout(dims, const_cast<void*>(plan_ws), &a.w);
    // [Gt U] = X W13, act = silu(Gt) * U
    a.A = static_cast<const uint16_t*>(recv);
    a.lda = H;
    a.Bhome = static_cast<const uint16_t*>(w13_home);
    a.Bslot = static_cast<const uint16_t*>(w13_slot);
    a.bstride = (long long)H * 2 * I;
    a.ldb = 2 * I;
    a.N = 2 * I;
    a.K = H;
    a.I = I;
    a.out = static_cast<uint16_t*>(act);
    a.ldo = I;
    a.gu = static_cast<uint16_t*>(gu_save);
    a.ntiles_n = (I + 127) / 128;
    rc = launch_rows(EPI_SWIGLU_FWD, B_NCONTIG, a, s);
    if (rc != MOONEP_OK) return rc;
    // y = act W2
    a.A = static_cast<const uint16_t*>(act);
    a.lda = I;
    a.Bhome = static_cast<const uint16_t*>(w2_home);
    a.Bslot = static_cast<const uint16_t*>(w2_slot);
    a.bstride = (long long)I * H;
    a.ldb = H;
    a.N = H;
    a.K = I;
    a.out = static_cast<uint16_t*>(y);
    a.ldo = H;
    a.gu = nullptr;
    a.ntiles_n = (H + BN - 1) / BN;
    return launch_rows(EPI_STORE, B_NCONTIG, a, s);
}

extern "C" int moonep_grouped_ffn_backward(const moonep_dims_t* dims, const void* plan_ws,
                                           const int32_t* cu_seqlens, const void* recv, const void* gu_save,
                                           const void* act, const void* dy, const void* w13_home,
                                           const void* w2_home, const void* w13_slot, const void* w2_slot,
                                           void* drecv, float* dw13_home, float* dw2_home, float* dw13_red,
                                           float* dw2_red, void* stream) {
    int rc = check_ffn_dims(dims);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(plan_ws);
    MOONEP_CHECK_PTR(cu_seqlens);
    MOONEP_CHECK_PTR(recv);
    MOONEP_CHECK_PTR(gu_save);
    MOONEP_CHECK_PTR(act);
    MOONEP_CHECK_PTR(dy);
    MOONEP_CHECK_PTR(w13_home);
    MOONEP_CHECK_PTR(w2_home);
    MOONEP_CHECK_PTR(drecv);
    MOONEP_CHECK_PTR(dw13_home);
    MOONEP_CHECK_PTR(dw2_home);
    if (dims->B > 0) {
        MOONEP_CHECK_PTR(w13_slot);
        MOONEP_CHECK_PTR(w2_slot);
        MOONEP_CHECK_PTR(dw13_red);
        MOONEP_CHECK_PTR(dw2_red);
    }
    const int H = dims->H, I = dims->I;
    hipStream_t s = static_cast<hipStream_t>(stream);
    GemmArgs a{};
    plan_ws_layout(dims, const_cast<void*>(plan_ws), &a.w);
    uint16_t* gu = static_cast<uint16_t*>(const_cast<void*>(gu_save));
    // dA = dY W2^T (B = W2 [I, H] is k-contiguous), fused SwiGLU' written over Gt|U
    a.A = static_cast<const uint16_t*>(dy);
    a.lda = H;
    a.Bhome = static_cast<const uint16_t*>(w2_home);
    a.Bslot = static_cast<const uint16_t*>(w2_slot);
    a.bstride = (long long)I * H;
    a.ldb = H;
    a.N = I;
    a.K = H;
    a.I = I;
    a.gu = gu;
    a.ntiles_n = (I + BN - 1) / BN;
    rc = launch_rows(EPI_SWIGLU_BWD, B_KCONTIG, a, s);
    if (rc != MOONEP_OK) return rc;
    // dX = [dGt dU] W13^T (B = W13 [H, 2I] is k-contiguous)
    a.A = gu;
    a.lda = 2 * I;
    a.Bhome = static_cast<const uint16_t*>(w13_home);
    a.Bslot = static_cast<const uint16_t*>(w13_slot);
    a.bstride = (long long)H * 2 * I;
    a.ldb = 2 * I;
    a.N = H;
    a.K = 2 * I;
    a.out = static_cast<uint16_t*>(drecv);
    a.ldo = H;
    a.gu = nullptr;
    a.ntiles_n = (H + BN - 1) / BN;
    rc = launch_rows(EPI_STORE, B_KCONTIG, a, s);
    if (rc != MOONEP_OK) return rc;
    // dW2 = A^T dY  ([I, H])
    GemmArgs d{};
    d.w = a.w;
    d.A = static_cast<const uint16_t*>(act);
    d.lda = I;
    d.B = static_cast<const uint16_t*>(dy);
    d.ldb = H;
    d.M = I;
    d.N = H;
    d.dw_home = dw2_home;
    d.dw_slot = dw2_red;
    d.ntiles_n = (H + BN - 1) / BN;
    rc = launch_dw(d, s);
    if (rc != MOONEP_OK) return rc;
    // dW13 = X^T [dGt dU]  ([H, 2I])
    d.A = static_cast<const uint16_t*>(recv);
    d.lda = H;
    d.B = gu;
    d.ldb = 2 * I;
    d.M = H;
    d.N = 2 * I;
    d.dw_home = dw13_home;
    d.dw_slot = dw13_red;
    d.ntiles_n = (2 * I + BN - 1) / BN;
    return launch_dw(d, s);
}
