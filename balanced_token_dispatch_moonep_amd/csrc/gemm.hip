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
//   * 256x256 output tile per workgroup, 8 waves in 2x4 (two per SIMD), each wave
//     128x64 = 4x2 tiles of v_mfma_f32_32x32x16_bf16 (bf16 inputs, fp32 accumulation).
//     Compile-time alternatives: a 4-wave 2x2 layout of 128x128 per wave for the row kernels;
//     256x128 weight-gradient tiles on two 4-wave workgroups per CU.
//   * Operand tiles go HBM -> LDS with global_load_lds_dwordx4 (16 bytes per lane, no
//     register staging), addressed as a wave-uniform base in scalar registers plus a 32-bit
//     per-lane offset.  Row kernels: 64-k stages in five 32 KiB buffers, one operand
//     triple-buffered (loaded two stages ahead), the other double-buffered.  Weight-gradient
//     kernel: a ring of four 32-k stages loaded three steps ahead.  One explicit vmcnt wait
//     and one barrier per stage.  The steady-state stages take their "does a later stage
//     exist" conditions as compile-time flags (the last stages are peeled off), so they carry
//     no branch around their copies and waits.
//   * LDS tiles are XOR-swizzled in 16-byte chunks so fragment reads are bank-conflict
//     free.  k-contiguous operands (activations, backward weights) are read with
//     ds_read_b128; m/n-contiguous operands (forward weights, both dW operands) stay
//     m/n-contiguous in LDS and are read with ds_read_b64_tr_b16, which hands each lane
//     4 consecutive k of one column -- two of them make one MFMA fragment.
//   * Persistent grid (one workgroup per CU).  Row kernels: tiles are ordered group-major,
//     then n-tile, then m-tile, and each XCD (blockIdx % 8) takes a contiguous range of them,
//     handed out in order from a per-XCD counter, so tiles sharing a weight or activation
//     panel run on the same XCD together.  Activation rows past a group's end (row-tile
//     padding: about 12% of the rows at R8 E256 S4096 K8 with maxvio 4) load zeros through the
//     range check of a buffer resource,
//     so their MFMAs run on zero operands, which draw less power (measured: the row kernels
//     ran 1-4% faster than with copies of the last valid row); weight columns outside a tile
//     clamp to the last valid one.  Weight-gradient kernel: tiles are
//     handed out dynamically, largest target first, and the loop is software-pipelined by one
//     tile (the next tile's first copies go out before this tile's stores); rows past a
//     segment's end load from a zero block kept in the plan workspace.
//   * Epilogues are fused and staged through LDS for 16-byte stores: SwiGLU (act =
//     silu(gate) * up, Gt|U saved) after the gate/up GEMM; SwiGLU' (dGt, dU written over
//     the saved Gt|U, which arrives by LDS DMA ahead of each quarter) after dA = dY W2^T;
//     fp32 store or accumulate into the home or reduce-buffer gradient for dW.
#include <type_traits>

#include "common.h"

namespace moonep {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int BM = 256, BN = 256, BK = 32, NSTAGE = 4;
constexpr int OP_BYTES = 256 * BK * 2;             // one operand tile of one stage: 16 KiB
constexpr int STAGE_BYTES = 2 * OP_BYTES;
constexpr int GEMM_SMEM = NSTAGE * STAGE_BYTES;    // 128 KiB
// Row kernels: K step 64, so every k-contiguous row segment a DMA lane group fetches is one full
// 128-byte line.
constexpr int BK2 = 64;
constexpr int OP2_BYTES = 256 * BK2 * 2;          // 32 KiB
// One operand gets three buffers, the other two: five operand buffers of 32 KiB fill the 160 KiB
// of LDS.  Which operand gets the third buffer is chosen per kernel by measurement (the SwiGLU
// kernels: the activations; the plain-store kernels: the weights).
constexpr int ROWS_SMEM = 5 * OP2_BYTES;          // 160 KiB
constexpr int MAX_GROUPS = 2 * kMaxE;
static_assert(4 * 32 * 132 * 4 <= GEMM_SMEM, "epilogue staging must fit in the stage ring");
static_assert(8 * 32 * 68 * 4 <= 4 * 32768 && 4 * 32 * 132 * 4 <= 4 * 32768,
              "row-kernel epilogue staging must end below the fifth operand buffer");
static_assert(8 * 32 * 68 * 4 <= 3 * 32768 && 4 * 32 * 132 * 4 <= 3 * 32768,
              "dA epilogue: staging below the fourth operand buffer (Gt|U copies use the last two)");

enum Epi { EPI_SWIGLU_FWD = 0, EPI_STORE = 1, EPI_SWIGLU_BWD = 2, EPI_ACC_F32 = 3 };
enum Mode { ROWS_BN = 0, ROWS_BK = 1 };   // weights n-contiguous ([K, N]) or k-contiguous ([N, K])

struct GemmArgs {
    PlanWs w;
    const uint16_t* A;        // rows modes: activations [R*C, lda]; dW: [R*C, lda] (m-contiguous)
    int lda;
    const uint16_t* B;        // dW: [R*C, ldb] (n-contiguous)
    const uint16_t* Bhome;    // rows modes: weights, home rows [E, ...]
    const uint16_t* Bslot;    //             slot rows [R*B, ...]
    long long bstride;        // elements per weight row
    int ldb;
    int M, N, K;              // dW: output M x N; rows modes: N output columns, K reduction
    int I;                    // SwiGLU split
    uint16_t* out;            // EPI_STORE / EPI_SWIGLU_FWD (act): bf16 [R*C, ldo]
    int ldo;
    uint16_t* gu;             // SwiGLU: [R*C, 2I]
    float* dw_home;           // EPI_ACC_F32: [E, M, N]
    float* dw_slot;           // EPI_ACC_F32: [R*B, M, N]
    int ntiles_n;
    int* counter;             // tile counters, one per XCD, zero at launch
    int accum;                // dW: add into the outputs (1) or write them (0)
    int dw_fn, dw_bm, dw_bn;  // dW: XCD x takes the tile block (x / dw_fn, x % dw_fn) of dw_bm x dw_bn
};

// ---------------------------------------------------------------------------
// synchronisation and LDS tile layout
// ---------------------------------------------------------------------------
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// Workgroup barrier without the memory fence of __syncthreads (which would wait for every
// in-flight LDS DMA); LDS DMA completion is waited for explicitly with wait_vm.
__device__ __forceinline__ void block_sync() {
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}
__device__ __forceinline__ void wave_sync() {
    compiler_fence();
    __builtin_amdgcn_wave_barrier();
    compiler_fence();
}
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait until every LDS access of this wave has completed
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// m/n-contiguous tile [32 k][256 mn]: 16-byte chunk (k, c), c = mn/8 in 0..31
__device__ __forceinline__ int mn_pos(int k, int c) { return k * 32 + (c ^ ((k & 3) << 2)); }
// k-contiguous tile [256 rows][64 k]: 16-byte chunk (r, c), c = k/8 in 0..7; sixteen consecutive
// rows reading the same chunk hit sixteen different 16-byte bank groups
__device__ __forceinline__ int kc8_pos(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// HBM -> LDS copy of 16 bytes per lane: lane l's bytes land at lds + 16*l (lds is wave-uniform).
// Issued as inline asm so the compiler does not track it as an LDS write (it would otherwise
// drain every in-flight copy before each transposing LDS read); completion is awaited with
// wait_vm() and a barrier before the data is read.  The instruction has no register outputs.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved: nothing else in these kernels uses it
__device__ __forceinline__ void dma16(const uint16_t* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}
// The same copy from a wave-uniform base (scalar registers) plus a per-lane 32-bit byte offset:
// the address arithmetic stays on the scalar unit (one base per stage), not on 64-bit vector adds.
__device__ __forceinline__ void dma16s(const uint16_t* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}
// The same copy through a buffer resource (base and byte limit in four scalar registers): a lane
// whose offset lies past the limit gets zeros (the range check of buffer loads).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16b(u32x4_t rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds)
                 : "memory", "m0");
}
// Raw buffer resource over [base, base + 0xFFFFFFF0): offsets of padding rows are set to the limit,
// and the range check (per dword, offset >= limit) returns zeros for them.  Every valid copy ends
// below it: check_ffn_dims keeps rows * K below 2^31 elements with K a multiple of 64, so a
// row's 16-byte chunks end at or below 2^32 - 128 bytes from the operand's start.
constexpr uint32_t kZeroOff = 0xFFFFFFF0u;
__device__ __forceinline__ u32x4_t rsrc_of(const void* base) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    u32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)p);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xFFFFu);
    r.z = kZeroOff;
    r.w = 0x00020000u;   // 32-bit data format, no swizzle, no stride
    return r;
}
#pragma clang diagnostic pop
// Next ticket of a tile counter.  An atomic increment rather than an add: the compiler rewrites
// an atomic add into a wave-reduced form that reads the result back at once, i.e. it waits there
// for every memory operation the wave has in flight; the increment's result is awaited only
// where it is used.
__device__ __forceinline__ int take_ticket(int* c) {
    return (int)atomicInc(reinterpret_cast<unsigned*>(c), 0xFFFFFFFFu);
}
// Scalar (wave-uniform) load of data that no kernel of this launch writes: the address must be
// the same for every lane; read through the constant address space, so it becomes a scalar load.
__device__ __forceinline__ int sload(const int32_t* p) {
    return *(const __attribute__((address_space(4))) int32_t*)(p);
}
// LDS byte address of a pointer into dynamic shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((lds_void_t*)(p));
}

// MFMA fragment (32 rows/cols x 16 k) from a k-contiguous 64-k tile: one 16-byte read per lane
__device__ __forceinline__ bf16x8_t frag_kc8(const char* T, int rb, int kk, int lane) {
    const int r = rb + (lane & 31), c = kk * 2 + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(T + kc8_pos(r, c) * 16);
}
// same fragment from an m/n-contiguous tile of CH 16-byte chunks per k-row: lane l gets column
// mb + l%32, k = 8*(l/32) + 0..7, as two transposing reads of 4 k each (lanes of a 16-lane group
// address a 4 k x 16 col block)
template <int CH = 32>
__device__ __forceinline__ bf16x8_t frag_mn(const char* T, int mb, int kk, int lane) {
    const int G = lane >> 4, i = lane & 15;
    const int col = mb + 16 * (G & 1) + 4 * (i & 3);
    const int k = kk * 16 + 8 * (G >> 1) + (i >> 2);
    const char* p = T + (k * CH + ((col >> 3) ^ ((k & 3) << 2))) * 16 + (col & 7) * 2;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * CH * 16));
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

// Wave layout of a 256x256 tile: 2 x WN waves; wave (wm, wn) owns rows wm*128 .. +128 and
// TN = 8/WN column blocks of 32.  WN = 2: 4 waves of 128x128 (one per SIMD); WN = 4: 8 waves of
// 128x64 (two per SIMD, so one wave's MFMAs cover the other's memory waits).
template <int WN>
struct WL {
    static constexpr int WAVES = 2 * WN;
    static constexpr int NTHR = 64 * WAVES;
    static constexpr int TN = 8 / WN;                  // 32-column blocks per wave
    static constexpr int PARTS = 16 / WAVES;           // DMA loads per operand, step and wave
    static constexpr int PER_STEP = 2 * PARTS;         // DMA loads per step and wave
    static constexpr int EPL = TN * 32 + 4;            // fp32 pitch of a staged epilogue row
};

// LDS column (tile n index) of wave-local MFMA column block tj.
template <int EPI, int WN>
__device__ __forceinline__ int bcol(int wn, int tj) {
    constexpr int TN = WL<WN>::TN;
    if (EPI == EPI_SWIGLU_FWD) {   // tile columns [0,128) gate, [128,256) up; a wave gets both halves
        constexpr int half = TN / 2;
        return tj < half ? wn * (128 / WN) + tj * 32 : 128 + wn * (128 / WN) + (tj - half) * 32;
    }
    return wn * (256 / WN) + tj * 32;
}

// MFMA operand fragments of one 16-k slice of a stage: 4 row blocks of A, TN column blocks of B.
template <int TN>
struct Frags {
    bf16x8_t a[4], b[TN];
};

// Weight-gradient tiles: 256 (M) x TBN (N), waves of 128 x 64 in 2 x TBN/64.  TBN = 256: one
// workgroup of 8 waves per CU, a ring of four 32-k stages.  TBN = 128: two workgroups of 4 waves
// per CU (each wave has its own vmcnt, so one workgroup's output stores do not hold up the
// other's copies), a ring of three stages each.
template <int TBN>
struct DWT {
    static constexpr int WAVES = TBN / 32;
    static constexpr int NTHR = 64 * WAVES;
    static constexpr int WNN = TBN / 64;          // waves along N
    static constexpr int TN = 2;                  // 32-column blocks per wave
    static constexpr int NST = TBN == 256 ? 4 : 3;
    static constexpr int OPA = 256 * BK * 2;      // A tile of one stage: [32 k][256 m]
    static constexpr int OPB = TBN * BK * 2;      // B tile of one stage: [32 k][TBN n]
    static constexpr int STAGE = OPA + OPB;
    static constexpr int PA = 16 / WAVES;         // 1 KiB copies of A per wave and step
    static constexpr int PB = (TBN / 16) / WAVES; // of B (PB <= PA)
    static constexpr int PER = PA + PB;
    static constexpr int BCH = TBN / 8;           // 16-byte chunks per k-row of the B tile
    static constexpr int EPL = TN * 32 + 4;       // fp32 pitch of a staged epilogue row
    // epilogue staging: the ring's last buffer onwards (the next tile's first NST-1 steps are
    // in the others while this tile's results are stored)
    static constexpr int STG = (NST - 1) * STAGE;
    static constexpr int SMEM = NST * STAGE > STG + WAVES * 16 * EPL * 4 ? NST * STAGE
                                                                          : STG + WAVES * 16 * EPL * 4;
};
static_assert(DWT<256>::SMEM <= ROWS_SMEM - 4096, "one 8-wave weight-gradient workgroup per CU");
static_assert(2 * (DWT<128>::SMEM + 2048) <= ROWS_SMEM, "two 4-wave weight-gradient workgroups per CU");

// Fragments of one 16-k slice of a weight-gradient step (both operands m/n-contiguous).
template <int TBN>
__device__ __forceinline__ void dw_load_frags(Frags<2>& f, const char* st, int kk, int wm, int wn, int lane) {
    using T = DWT<TBN>;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.a[t] = frag_mn<32>(st, wm * 128 + t * 32, kk, lane);
#pragma unroll
    for (int t = 0; t < 2; ++t) f.b[t] = frag_mn<T::BCH>(st + T::OPA, wn * 64 + t * 32, kk, lane);
}

template <int TN>
__device__ __forceinline__ void mma_row(f32x16_t (&acc)[4][TN], const Frags<TN>& f, int i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}
template <int TN>
__device__ __forceinline__ void mma_frags(f32x16_t (&acc)[4][TN], const Frags<TN>& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) mma_row<TN>(acc, f, i);
}

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }

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

template <int TN>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[4][TN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// Weight-gradient main loop over nst K-steps of 32 (two 16-k slices each), split in two so a
// persistent workgroup can issue the next tile's first copies before the current tile's stores.
// issue(s, buf, part) enqueues this wave's DMA loads of step s (copy `part` of A, p < PA, and of
// B if p < PB) into a ring of NST buffers.  dw_prologue issues steps 0..NST-2.
template <int TBN, typename Issue>
__device__ __forceinline__ void dw_prologue(int nst, Issue&& issue) {
    using T = DWT<TBN>;
#pragma unroll
    for (int s = 0; s < T::NST - 1; ++s)
        if (s < nst)
#pragma unroll
            for (int p = 0; p < T::PA; ++p) issue(s, s, p);
}

// Fragments are double-buffered in registers: the reads of the next slice are issued before the
// MFMAs of the current one; the step barrier sits between a step's two slices so the MFMAs already
// issued keep the matrix cores busy across it; and the DMA loads of step s+NST-1 are spread between
// the MFMAs of the second slice, so no burst of memory instructions stalls the wave's in-order
// issue while the matrix pipe drains.
template <int TBN, typename Issue, typename IssueFast, typename FastRun>
__device__ __forceinline__ void dw_main(f32x16_t (&acc)[4][2], char* smem, int nst, int wm, int wn, int lane,
                                        Issue&& issue, IssueFast&& issue_fast, FastRun&& fast_run) {
    using T = DWT<TBN>;
    constexpr int NST = T::NST, PER = T::PER;
    if (nst > 0) {
        // step 0 landed (vmcnt retires in issue order: all but the last n issued are done);
        // the following steps of the prologue (if any) may still be in flight
        if constexpr (NST == 4) {
            if (nst >= 3) wait_vm<2 * PER>();
            else if (nst == 2) wait_vm<PER>();
            else wait_vm<0>();
        } else {
            if (nst >= 2) wait_vm<PER>();
            else wait_vm<0>();
        }
        block_sync();
        Frags<2> f0, f1;
        dw_load_frags<TBN>(f0, smem, 0, wm, wn, lane);
        // One step.  FAST: a step s in 2 .. nst-NST (step s+NST-1 exists) whose step s+NST-1 is
        // full and does not end its segment; the conditions are then compile-time, so these steps
        // carry no branch around their waits and copies.  (Steps 0 and 1 run the general way:
        // starting the fast run at step 0 measured the same.)
        auto step = [&](int s, auto fast_c) {
            constexpr bool fast = decltype(fast_c)::value;
            const char* st = smem + ((unsigned)s % NST) * T::STAGE;
            dw_load_frags<TBN>(f1, st, 1, wm, wn, lane);
            mma_frags<2>(acc, f0);
            // Settle the slice-1 reads only after all slice-0 MFMAs are issued (the scheduling
            // barrier keeps the compiler from hoisting the wait above them, which would expose the
            // reads' latency); settling them here keeps the compiler from making the next MFMAs
            // wait on the reads issued after the step barrier.
            __builtin_amdgcn_sched_barrier(0);
            wait_lgkm0();
            if (fast || s + 1 < nst) {
                // step s+1 must have landed; with four stages step s+2 may still be in flight
                if constexpr (NST == 4) {
                    if (fast || s + 2 < nst) wait_vm<PER>();
                    else wait_vm<0>();
                } else {
                    wait_vm<0>();
                }
                block_sync();
                dw_load_frags<TBN>(f0, smem + ((unsigned)(s + 1) % NST) * T::STAGE, 0, wm, wn, lane);
            }
            // every wave is past step s-1, so its buffer takes step s+NST-1
            const bool more = fast || s + NST - 1 < nst;
            const int nb = (unsigned)(s + NST - 1) % NST;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mma_row<2>(acc, f1, i);
                if (more && i % (4 / T::PA) == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (fast) issue_fast(s + NST - 1, nb, i / (4 / T::PA));
                    else issue(s + NST - 1, nb, i / (4 / T::PA));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        int s = 0;
        for (; s < nst && s < 2; ++s) step(s, std::false_type{});
        // the run of full steps that the cursor's segment still holds (all of a one-segment
        // target's steps but its last), then everything else the general way
        if (s + NST - 1 < nst) {
            const int e = s + max(0, min(nst - (NST - 1) - s, fast_run()));
            for (; s < e; ++s) step(s, std::true_type{});
        }
        for (; s + NST - 1 < nst; ++s) step(s, std::false_type{});
        for (; s < nst; ++s) step(s, std::false_type{});
    }
    block_sync();     // every wave is done with the ring before the next tile's copies reuse it
}

// Fragments of one 16-k slice (kk = 0..3) of a 64-k row-kernel stage.
template <bool B_KC, int EPI, int WN>
__device__ __forceinline__ void load_frags64(Frags<WL<WN>::TN>& f, const char* As, const char* Bs, int kk, int wm,
                                             int wn, int lane) {
#pragma unroll
    for (int t = 0; t < 4; ++t) f.a[t] = frag_kc8(As, wm * 128 + t * 32, kk, lane);
#pragma unroll
    for (int t = 0; t < WL<WN>::TN; ++t)
        f.b[t] = B_KC ? frag_kc8(Bs, bcol<EPI, WN>(wn, t), kk, lane) : frag_mn(Bs, bcol<EPI, WN>(wn, t), kk, lane);
}

// Main loop of the row kernels over nst 64-k stages.  A has RA buffers, B has RB (3 and 2, or 2
// and 3 with DEEP_B; buffers of A at [0, RA), of B at [RA, RA+RB) in units of 32 KiB).  During stage s
// the wave issues, after the barrier that retired stage s-1's buffers, the double-buffered
// operand's stage s+1 (slice 0) and then the triple-buffered operand's stage s+2 (slice 1);
// issue(op, u, buf, part) loads operand op (0 = A, 1 = B) of stage u into buffer buf.  At the
// end of stage s only the triple-buffered operand's stage s+2 may be newer than stage s+1.
// Fragments are double-buffered across the four 16-k slices, and the barrier sits before the
// last slice's MFMAs so they cover the first reads of the next stage.
template <bool B_KC, int EPI, int WN, bool DEEP_B, typename Issue>
__device__ __forceinline__ void pipeline64(f32x16_t (&acc)[4][WL<WN>::TN], char* smem, int nst, int wm, int wn,
                                           int lane, Issue&& issue) {
    using L = WL<WN>;
    constexpr int P2 = 2 * L::PARTS;      // loads per operand, stage and wave
    constexpr int RA = DEEP_B ? 2 : 3, RB = DEEP_B ? 3 : 2;
    constexpr int D2 = RA == 2 ? 0 : 1;   // double-buffered operand
    constexpr int D3 = 1 - D2;            // triple-buffered operand
    constexpr int N3 = D3 == 0 ? RA : RB;
    auto buf_of = [&](int op, int u) { return op == 0 ? u % RA : RA + u % RB; };
#pragma unroll
    for (int p = 0; p < P2; ++p) issue(0, 0, buf_of(0, 0), p);
#pragma unroll
    for (int p = 0; p < P2; ++p) issue(1, 0, buf_of(1, 0), p);
    if (nst > 1) {
#pragma unroll
        for (int p = 0; p < P2; ++p) issue(D3, 1, buf_of(D3, 1), p);
        wait_vm<P2>();
    } else {
        wait_vm<0>();
    }
    block_sync();
    Frags<L::TN> f0, f1;
    load_frags64<B_KC, EPI, WN>(f0, smem, smem + RA * OP2_BYTES, 0, wm, wn, lane);
    // One stage; MORE: stage s+1 exists, MORE3: stage s+2 exists.  Compile-time flags, so the
    // steady-state loop below carries no branch around its copies and waits.
    auto stage = [&](int s, auto more_c, auto more3_c) {
        constexpr bool more = decltype(more_c)::value, more3 = decltype(more3_c)::value;
        const char* As = smem + (s % RA) * OP2_BYTES;
        const char* Bs = smem + (RA + s % RB) * OP2_BYTES;
        // slice 0: the double-buffered operand of stage s+1
        load_frags64<B_KC, EPI, WN>(f1, As, Bs, 1, wm, wn, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mma_row<L::TN>(acc, f0, i);
            if constexpr (more)
                if (i % (4 / P2 > 0 ? 4 / P2 : 1) == 0)
#pragma unroll
                    for (int p = 0; p < (P2 > 4 ? P2 / 4 : 1); ++p) {
                        const int part = P2 > 4 ? i * (P2 / 4) + p : i / (4 / P2);
                        __builtin_amdgcn_sched_barrier(0);
                        issue(D2, s + 1, buf_of(D2, s + 1), part);
                        __builtin_amdgcn_sched_barrier(0);
                    }
        }
        // slice 1: the triple-buffered operand of stage s+2
        load_frags64<B_KC, EPI, WN>(f0, As, Bs, 2, wm, wn, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mma_row<L::TN>(acc, f1, i);
            if constexpr (more3)
                if (i % (4 / P2 > 0 ? 4 / P2 : 1) == 0)
#pragma unroll
                    for (int p = 0; p < (P2 > 4 ? P2 / 4 : 1); ++p) {
                        const int part = P2 > 4 ? i * (P2 / 4) + p : i / (4 / P2);
                        __builtin_amdgcn_sched_barrier(0);
                        issue(D3, s + 2, buf_of(D3, s + 2), part);
                        __builtin_amdgcn_sched_barrier(0);
                    }
        }
        // slice 2
        load_frags64<B_KC, EPI, WN>(f1, As, Bs, 3, wm, wn, lane);
        mma_frags<L::TN>(acc, f0);
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm0();
        if constexpr (more) {
            if constexpr (more3) wait_vm<P2>();     // stage s+1 has landed (stage s+2's deep operand may not)
            else wait_vm<0>();
            block_sync();
            load_frags64<B_KC, EPI, WN>(f0, smem + ((s + 1) % RA) * OP2_BYTES,
                                        smem + (RA + (s + 1) % RB) * OP2_BYTES, 0, wm, wn, lane);
        }
        // slice 3
        mma_frags<L::TN>(acc, f1);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    int s = 0;
    for (; s + 2 < nst; ++s) stage(s, T_{}, T_{});
    if (s + 1 < nst) stage(s++, T_{}, F_{});
    if (s < nst) stage(s, F_{}, F_{});
    (void)N3;
    block_sync();     // every wave is done with the buffers before the epilogue reuses them
}

// m-tile prefix of the groups (tile_pref[g] = 256-row tiles of groups before g), for the row
// kernels: one wave, 64 groups at a time, wave-wide inclusive scan with a running carry
__global__ __launch_bounds__(64) void tile_prefix_kernel(PlanWs w) {
    const int lane = threadIdx.x;
    const int ng = min(max(w.hdr[HDR_NGROUPS], 0), 2 * w.E);
    int run = 0;
    for (int g0 = 0; g0 < ng; g0 += 64) {
        const int g = g0 + lane;
        const int v = g < ng ? (group_rows(w.groups[g], w) + BM - 1) / BM : 0;
        int x = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (g < ng) w.tile_pref[g] = run + x - v;
        run += __shfl(x, 63);
    }
    if (lane == 0) w.tile_pref[ng] = run;
}

// ---------------------------------------------------------------------------
// Epilogues: each wave stages a 32-row quarter of its accumulators (fp32) in its own LDS
// region, then every lane handles 8 (or 4) consecutive columns of a row so global accesses
// are 16 bytes wide.  C layout of a 32x32 MFMA tile: lane l, reg r -> row (r/4)*8 + (l/32)*4
// + r%4, column l%32.
// ---------------------------------------------------------------------------
template <int q, int TN, int EPLD>
__device__ __forceinline__ void stage_quarter(const f32x16_t (&acc)[4][TN], float* ep, int lane) {
    const int lc = lane & 31, lr4 = (lane >> 5) * 4;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) ep[((r >> 2) * 8 + lr4 + (r & 3)) * EPLD + j * 32 + lc] = acc[q][j][r];
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

// dA epilogue: DMA of quarter q's saved Gt|U into the wave's LDS region (its share of the two
// operand buffers the epilogue does not use): chunk (it, gate/up) of lane l lands at region + (2 it + u) KiB +
// 16 l, holding the (row, columns) that lane reads in the epilogue; rows and columns outside the
// tile clamp to the last valid one.  Copied rather than loaded so that it can be issued ahead of
// the previous quarter's stores without holding registers: vmcnt retires in order, so a load
// issued after those stores would wait for them.
template <int WN, int q>
__device__ __forceinline__ void prefetch_gu(const GemmArgs& a, int wm, int wn, int lane, int nt, int row0,
                                            int mvalid, uint32_t region) {
    constexpr int TN = WL<WN>::TN;
    constexpr int LPR = 4 * TN, RPI = 64 / LPR, IT = 32 / RPI;
    const int I = a.I;
    const int lcol = min(nt * BN + wn * (256 / WN) + (lane % LPR) * 8, I - 8);
    const int rbase = wm * 128 + q * 32;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const size_t row = (size_t)(row0 + min(rbase + it * RPI + lane / LPR, mvalid - 1));
        dma16(a.gu + row * 2 * I + lcol, region + (2 * it) * 1024);
        dma16(a.gu + row * 2 * I + I + lcol, region + (2 * it + 1) * 1024);
    }
}

template <int EPI, int WN, int q>
__device__ __forceinline__ void epi_rows_quarter(const GemmArgs& a, const f32x16_t (&acc)[4][WL<WN>::TN], float* ep,
                                                 int wm, int wn, int lane, int nt, int row0, int mvalid,
                                                 const char* gl = nullptr, uint32_t gu_lds = 0,
                                                 bool gfull = false) {
    constexpr int TN = WL<WN>::TN, EPLD = WL<WN>::EPL;
    stage_quarter<q, TN, EPLD>(acc, ep, lane);
    wave_sync();
    const int rbase = wm * 128 + q * 32;   // tile-local row of the quarter's first row
    if (EPI == EPI_SWIGLU_FWD) {
        // staged columns [0, 16 TN) = gate, [16 TN, 32 TN) = up, for act columns
        // nt*128 + wn*(128/WN) + c; 2 TN lanes per row, 8 columns each
        constexpr int LPR = 2 * TN, RPI = 64 / LPR;
        const int I = a.I;
        const int c = (lane % LPR) * 8;
        const int col = nt * 128 + wn * (128 / WN) + c;
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
            const int rr = it * RPI + lane / LPR;
            if (rbase + rr < mvalid && col < I) {
                float g[8], u[8], o[8];
                read8(ep + rr * EPLD + c, g);
                read8(ep + rr * EPLD + 16 * TN + c, u);
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = g[i] * sigm(g[i]) * u[i];
                const size_t row = (size_t)(row0 + rbase + rr);
                *reinterpret_cast<uint4*>(a.out + row * a.ldo + col) = pack8(o);
                if (a.gu) {
                    *reinterpret_cast<uint4*>(a.gu + row * 2 * I + col) = pack8(g);
                    *reinterpret_cast<uint4*>(a.gu + row * 2 * I + I + col) = pack8(u);
                }
            }
        }
    } else if (EPI == EPI_SWIGLU_BWD) {
        constexpr int LPR = 4 * TN, RPI = 64 / LPR, IT = 32 / RPI;
        const int I = a.I;
        const int c = (lane % LPR) * 8;
        const int col = nt * BN + wn * (256 / WN) + c;
        // this quarter's Gt|U has landed in the wave's LDS region: in a full tile only the
        // previous quarter's 2 IT stores were issued after its copy
        if (q > 0 && gfull) wait_vm<2 * IT>();
        else wait_vm<0>();
        uint4 gv[IT], uv[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            gv[it] = *reinterpret_cast<const uint4*>(gl + (2 * it) * 1024 + lane * 16);
            uv[it] = *reinterpret_cast<const uint4*>(gl + (2 * it + 1) * 1024 + lane * 16);
        }
        wait_lgkm0();   // the region is free again: the next quarter's copy goes out before the stores
        if constexpr (q < 3) prefetch_gu<WN, q + 1>(a, wm, wn, lane, nt, row0, mvalid, gu_lds);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int rr = it * RPI + lane / LPR;
            if (rbase + rr < mvalid && col < I) {
                const size_t row = (size_t)(row0 + rbase + rr);
                float da[8], g[8], u[8], dg[8], du[8];
                read8(ep + rr * EPLD + c, da);
                unpack8(gv[it], g);
                unpack8(uv[it], u);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float sg = sigm(g[i]);
                    dg[i] = da[i] * u[i] * sg * (1.0f + g[i] * (1.0f - sg));
                    du[i] = da[i] * g[i] * sg;
                }
                *reinterpret_cast<uint4*>(a.gu + row * 2 * I + col) = pack8(dg);
                *reinterpret_cast<uint4*>(a.gu + row * 2 * I + I + col) = pack8(du);
            }
        }
    } else {
        constexpr int LPR = 4 * TN, RPI = 64 / LPR, IT = 32 / RPI;
        const int c = (lane % LPR) * 8;
        const int col = nt * BN + wn * (256 / WN) + c;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int rr = it * RPI + lane / LPR;
            if (rbase + rr < mvalid && col < a.N) {
                float v[8];
                read8(ep + rr * EPLD + c, v);
                *reinterpret_cast<uint4*>(a.out + (size_t)(row0 + rbase + rr) * a.ldo + col) = pack8(v);
            }
        }
    }
    wave_sync();
}

// Rows 16h..16h+15 of row block q of a wave's accumulators -> LDS staging [16][EPLD] floats.
template <int q, int h, int TN, int EPLD>
__device__ __forceinline__ void stage_half(const f32x16_t (&acc)[4][TN], float* ep, int lane) {
    const int lc = lane & 31, lr4 = (lane >> 5) * 4;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; ++r)
            ep[(((r >> 2) & 1) * 8 + lr4 + (r & 3)) * EPLD + j * 32 + lc] = acc[q][j][r];
}

// Weight-gradient epilogue for rows 16h..16h+15 of row block q: float32 stores, or += with
// MOONEP_GRAD_ACCUM.  FULL: the tile lies inside [M, N], so every store is issued unmasked and
// the caller can count them.
template <int q, int h, bool FULL>
__device__ __forceinline__ void epi_dw_part(const GemmArgs& a, const f32x16_t (&acc)[4][2], float* ep,
                                            int wm, int wn, int lane, float* out, int m0, int n0) {
    constexpr int TN = 2, EPLD = TN * 32 + 4;
    constexpr int LPR = 8 * TN, RPI = 64 / LPR, IT = 16 / RPI;   // float4 chunks
    stage_half<q, h, TN, EPLD>(acc, ep, lane);
    wave_sync();
    const int c = (lane % LPR) * 4;
    const int col = n0 + wn * 64 + c;
    const int rb = m0 + wm * 128 + q * 32 + h * 16;
    if (!a.accum) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int rr = it * RPI + lane / LPR;
            const int row = rb + rr;
            if (FULL || (row < a.M && col < a.N))   // streamed out: non-temporal (measured 0.7% faster)
                st_nt(*reinterpret_cast<const float4*>(ep + rr * EPLD + c),
                      reinterpret_cast<float4*>(out + (size_t)row * a.N + col));
        }
        wave_sync();
        return;
    }
    // all loads first (clamped to in-bounds addresses), then add and store
    float4 old[IT];
    const int lcol = min(col, a.N - 4);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int rr = it * RPI + lane / LPR;
        const int row = min(rb + rr, a.M - 1);
        old[it] = *reinterpret_cast<const float4*>(out + (size_t)row * a.N + lcol);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int rr = it * RPI + lane / LPR;
        const int row = rb + rr;
        if (FULL || (row < a.M && col < a.N)) {
            const float4 v = *reinterpret_cast<const float4*>(ep + rr * EPLD + c);
            float4 o = old[it];
            o.x += v.x;
            o.y += v.y;
            o.z += v.z;
            o.w += v.w;
            st_nt(o, reinterpret_cast<float4*>(out + (size_t)row * a.N + col));
        }
    }
    wave_sync();
}

template <bool FULL>
__device__ __forceinline__ void epi_dw(const GemmArgs& a, const f32x16_t (&acc)[4][2], float* ep, int wm,
                                       int wn, int lane, float* out, int m0, int n0) {
    epi_dw_part<0, 0, FULL>(a, acc, ep, wm, wn, lane, out, m0, n0);
    epi_dw_part<0, 1, FULL>(a, acc, ep, wm, wn, lane, out, m0, n0);
    epi_dw_part<1, 0, FULL>(a, acc, ep, wm, wn, lane, out, m0, n0);
    epi_dw_part<1, 1, FULL>(a, acc, ep, wm, wn, lane, out, m0, n0);
    epi_dw_part<2, 0, FULL>(a, acc, ep, wm, wn, lane, out, m0, n0);
    epi_dw_part<2, 1, FULL>(a, acc, ep, wm, wn, lane, out, m0, n0);
    epi_dw_part<3, 0, FULL>(a, acc, ep, wm, wn, lane, out, m0, n0);
    epi_dw_part<3, 1, FULL>(a, acc, ep, wm, wn, lane, out, m0, n0);
}

// ---------------------------------------------------------------------------
// Row-grouped GEMM: C[rows, N] = A[rows, K] * B_w[K, N] for every plan group.
// ---------------------------------------------------------------------------
template <int MODE, int EPI, int WN>
__global__ __launch_bounds__(128 * WN, 1) void gemm_rows_kernel(GemmArgs a) {
    using L = WL<WN>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const Group* groups = a.w.groups;
    const int ng = min(max(a.w.hdr[HDR_NGROUPS], 0), min(2 * a.w.E, MAX_GROUPS));
    const int32_t* tp = a.w.tile_pref;    // m-tile prefix of the groups (tile_prefix_kernel)
    const int NT = a.ntiles_n;
    const int total = tp[ng] * NT;
    const int nxcd = 8;
    const int xcd = blockIdx.x % nxcd;
    const int chunk = (total + nxcd - 1) / nxcd;
    const int t_lo = xcd * chunk, t_hi = min(total, t_lo + chunk);
    float* ep = reinterpret_cast<float*>(smem) + wave * 32 * L::EPL;
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_addr(smem) + wave * 2 * L::PARTS * 1024);

    // The tiles of this XCD's range are handed out in order from a per-XCD counter, so the tiles
    // in flight on an XCD stay neighbours (sharing A rows and weight columns in its L2) even when
    // tiles take different times.  Tile ids pass through two words at the start of the fifth
    // operand buffer, alternating: between a tile's last barrier and the next tile's first one no
    // copy targets that buffer (the first copies go to the first stage's buffers and the deep
    // operand's second stage), and the epilogue staging ends below it.  The dA epilogue's Gt|U
    // copies do land there, but each is awaited before that epilogue's last barrier, and a word
    // is read only after thread 0 rewrites it.  All 160 KiB of LDS are dynamic, so no static LDS
    // is left for them.
    int* const s_t = reinterpret_cast<int*>(smem + 4 * OP2_BYTES);
    int fs = 0;
    auto publish = [&](int v) {
        if (tid == 0) s_t[fs] = v;
        wait_lgkm0();
        block_sync();
        const int r = __builtin_amdgcn_readfirstlane(s_t[fs]);
        fs ^= 1;
        return r;
    };
    int* const qc = a.counter + xcd;
    int nxt = 0;
    if (tid == 0) nxt = take_ticket(qc);
    for (int t = t_lo + publish(nxt); t < t_hi; t = t_lo + publish(nxt)) {
        if (tid == 0) nxt = take_ticket(qc);   // the next tile, read after this tile's main loop
        // the tile's group, by binary search over the tile prefix; scalar loads (the search is
        // wave-uniform), which do not wait for the previous tile's stores and stay in the scalar
        // cache after the first tile
        int lo = 0, hi = ng - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sload(tp + mid) * NT <= t) lo = mid; else hi = mid - 1;
        }
        const int g = lo;
        const Group gr{sload(&groups[g].row0), sload(&groups[g].rows), sload(&groups[g].wsel),
                       sload(&groups[g].expert)};
        const int tpg = sload(tp + g);
        const int mtiles = sload(tp + g + 1) - tpg;
        const int local = t - tpg * NT;
        const int nt = local / mtiles, mt = local % mtiles;
        const int row0 = gr.row0 + mt * BM;
        const int mvalid = min(BM, group_rows(gr, a.w) - mt * BM);
        const uint16_t* W = gr.wsel >= 0 ? a.Bhome + (size_t)gr.wsel * a.bstride
                                         : a.Bslot + (size_t)(-1 - gr.wsel) * a.bstride;

        // per-lane sources of this wave's DMA loads (2*PARTS per operand and stage), as byte
        // offsets from the stage's operand base; activation rows past the group's end get an
        // offset beyond the buffer resource's limit (zeros), weight columns outside the tile clamp
        // to the last valid one (their products only reach outputs the epilogue does not store)
        constexpr int P2 = 2 * L::PARTS;
        uint32_t ao[P2], bo[P2];
#pragma unroll
        for (int i = 0; i < P2; ++i) {
            const int p = (wave * P2 + i) * 64 + lane;
            {   // A: k-contiguous activations [rows, K]; rows past the group's end read zeros
                const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
                ao[i] = r < mvalid ? 2u * (uint32_t)((row0 + r) * a.lda + c * 8) : kZeroOff;
            }
            if (MODE == ROWS_BK) {   // weights [N, K]
                const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
                bo[i] = 2u * (uint32_t)(min(nt * BN + r, a.N - 1) * a.ldb + c * 8);
            } else {                 // weights [K, N]
                const int k = p >> 5, c = (p & 31) ^ ((k & 3) << 2);
                int col;
                if (EPI == EPI_SWIGLU_FWD) {
                    const int cc = min(nt * 128 + (c & 15) * 8, a.I - 8);
                    col = c < 16 ? cc : a.I + cc;
                } else {
                    col = min(nt * BN + c * 8, a.N - 8);
                }
                bo[i] = 2u * (uint32_t)(k * a.ldb + col);
            }
        }
        const int bstep = MODE == ROWS_BK ? BK2 : BK2 * a.ldb;
        const uint16_t* A0 = a.A;

        f32x16_t acc[4][L::TN];
        zero_acc<L::TN>(acc);
        pipeline64<MODE == ROWS_BK, EPI, WN, EPI == EPI_STORE>(acc, smem, a.K / BK2, wm, wn, lane,
                                             [&](int op, int s, int buf, int i) {
            const uint32_t l = lds_wave + buf * OP2_BYTES + i * 1024;
            // activations through a buffer resource per stage (zeros for padding rows); weights
            // from a scalar stage base + per-lane offset, except in the dX kernel (k-contiguous
            // weights, plain store), which measured faster with per-lane 64-bit addresses
            if (op == 0) {
                dma16b(rsrc_of(A0 + s * BK2), ao[i], l);
            } else if constexpr (MODE == ROWS_BK && EPI == EPI_STORE) {
                dma16(W + (bo[i] / 2 + s * bstep), l);
            } else {
                dma16s(W + (size_t)s * bstep, bo[i], l);
            }
        });
        // the next tile's ticket is read here, while no stores are in flight: vmcnt retires in
        // order, so awaiting it after the epilogue would wait for all of the epilogue's stores
        // (every wave reads it, so none carries it as outstanding into the next tile)
        nxt = __builtin_amdgcn_readfirstlane(nxt);
        // dA: the saved Gt|U goes through the last two operand buffers (64 KiB split over the
        // waves), which the epilogue staging does not reach; quarter 0's copy goes out now
        constexpr int GU_WAVE = 2 * OP2_BYTES / L::WAVES;
        static_assert(GU_WAVE == 2 * 1024 * (32 / (64 / (4 * L::TN))),
                      "a wave's Gt|U copies of one quarter fill its share of the two buffers");
        const char* gl = smem + 3 * OP2_BYTES + wave * GU_WAVE;
        const uint32_t gu_lds = __builtin_amdgcn_readfirstlane(lds_addr(gl));
        const bool gfull = mvalid >= BM && nt * BN + BN <= a.I;
        if constexpr (EPI == EPI_SWIGLU_BWD) prefetch_gu<WN, 0>(a, wm, wn, lane, nt, row0, mvalid, gu_lds);
        epi_rows_quarter<EPI, WN, 0>(a, acc, ep, wm, wn, lane, nt, row0, mvalid, gl, gu_lds, gfull);
        epi_rows_quarter<EPI, WN, 1>(a, acc, ep, wm, wn, lane, nt, row0, mvalid, gl, gu_lds, gfull);
        epi_rows_quarter<EPI, WN, 2>(a, acc, ep, wm, wn, lane, nt, row0, mvalid, gl, gu_lds, gfull);
        epi_rows_quarter<EPI, WN, 3>(a, acc, ep, wm, wn, lane, nt, row0, mvalid, gl, gu_lds, gfull);
        block_sync();   // the ring is reused by the next tile's loads
    }
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM: dW[M, N] = A^T B (or += with MOONEP_GRAD_ACCUM) over the target's row
// segments, where A = [rows, M] and B = [rows, N] are read m/n-contiguous.  Targets: t < E is
// home expert t (its home rows plus its fallback replicas, in plan order), t >= E is prefetch
// slot t - E.  Targets are taken in descending row order.
//
// Tile order.  Each target's MT x NT tile grid is cut into eight blocks of dw_bm x dw_bn tiles
// (the split with the fewest panels per block), one per XCD (workgroup b runs on XCD b mod 8).
// The XCD's workgroups take its blocks, target after target, from the XCD's own counter
// (n-tiles fastest inside a block), so the tiles in flight on an XCD share a few A panels and
// dw_bn B panels in its L2.  A tile at position (i, j) of its block runs the full K steps of a
// one-segment target rotated by 3(i + j) steps (its last, possibly partial, step stays last),
// so tiles that share a panel read a slab some steps apart and the later reader can find it in
// L2 instead of waiting on the same miss.  Against one global largest-first order this
// measured dW13 8% and dW2 5% faster; a block without the rotation gained about 3.6% on dW13
// and nothing on dW2, m-tiles fastest 2.5% and 1% less, and rotations of 1 to 5 steps per
// position measured within 1-2% of each other.
// ---------------------------------------------------------------------------
// WHICH (2 or 13) only separates the two weight-gradient launches' kernel names in traces.
//
// The persistent loop is software-pipelined by one tile: after tile i's main loop, the workgroup
// sets up tile i+1 (its id was fetched during tile i) and issues its first three steps, then
// stages and stores tile i's result, so tile i+1's first copies are in flight during the
// epilogue.  Every wave then waits for all of its stores before tile i+1's main loop.  Letting
// the stores drain behind tile i+1's first steps instead measured no faster, and variants that
// issued all of them without pacing measured 1-2% slower; the compiled epilogue also waits for
// the previous slice's stores before each slice (a side effect of the accumulate path's loads),
// and wave 0 for all of its operations after the tile counter's atomic add.
template <int TBN, int WHICH>
__global__ __launch_bounds__(DWT<TBN>::NTHR, TBN == 128 ? 2 : 1) void gemm_dw_kernel(GemmArgs a) {
    using T = DWT<TBN>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    __shared__ Segment s_seg[2][kMaxR + 1];
    __shared__ int s_tile[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WNN, wn = wave % T::WNN;
    const PlanWs& w = a.w;
    const int MT = (a.M + BM - 1) / BM, NT = a.ntiles_n;
    const int xcd = blockIdx.x % 8;
    const int bm = a.dw_bm, bn = a.dw_bn;
    const int bx = xcd / a.dw_fn, by = xcd % a.dw_fn;
    const int per_target = bm * bn;                      // tiles of one target on this XCD
    const int total = (w.E + w.R * w.B) * per_target;
    int* const counter = a.counter + xcd;
    float* ep = reinterpret_cast<float*>(smem + T::STG) + wave * 16 * T::EPL;
    // this wave's 1 KiB DMA slots of the A and B tiles of a stage
    const uint32_t lds_a = __builtin_amdgcn_readfirstlane(lds_addr(smem) + wave * T::PA * 1024);
    const uint32_t lds_b = __builtin_amdgcn_readfirstlane(lds_addr(smem) + T::OPA + wave * T::PB * 1024);

    // Tile ids pass through s_tile, alternating between its two words, so a wave still reading
    // one word is never overtaken by thread 0 writing the next id into it.
    int fs = 0;
    auto publish = [&](int v) {     // thread 0's value -> every thread
        if (tid == 0) s_tile[fs] = v;
        wait_lgkm0();
        block_sync();
        const int r = s_tile[fs];
        fs ^= 1;
        return r;
    };
    auto fetch = [&]() {            // next tile id from the XCD's counter
        int v = 0;
        if (tid == 0) v = atomicAdd(counter, 1);
        return publish(v);
    };
    // Descriptor of this XCD's tile t; its row segments go to s_seg[par].  Returns false for a
    // tile with nothing to do (past the grid's edge, an unused slot, or no rows in accumulate
    // mode).  Target t < E is home expert t (its home rows, then its fallback replicas in plan
    // order); t >= E is prefetch slot t - E.
    int nseg = 0, nst = 0, m0 = 0, n0 = 0, rot = 0;
    float* out = nullptr;
    auto setup = [&](int t, int par) {
        const int target = w.dw_order[t / per_target];
        const int local = t % per_target;
        const int j = local % bn, i = local / bn;        // n-tiles fastest
        const int mt = bx * bm + i, nt = by * bn + j;
        if (mt >= MT || nt >= NT) return false;
        rot = 3 * (i + j);
        if (target < w.E) {
            const Segment hs = w.home_seg[target];
            const int nfb = min(max(w.fb_n[target], 0), kMaxR - 1);
            const bool has_home = seg_ok(hs, w) && hs.rows > 0;
            nseg = (has_home ? 1 : 0) + nfb;
            if (tid == 0 && has_home) s_seg[par][0] = hs;
            if (tid >= 1 && tid <= nfb) {
                const Segment f = w.fb_seg[(size_t)target * kMaxR + tid - 1];
                s_seg[par][(has_home ? 1 : 0) + tid - 1] = seg_ok(f, w) ? f : Segment{0, 0};
            }
            out = a.dw_home + (size_t)target * a.M * a.N;
        } else {
            const int sl = target - w.E;
            if (w.slot_e[sl] < 0) return false;
            const Segment f{w.slot_row0[sl], w.slot_rows[sl]};
            if (!seg_ok(f, w)) return false;
            if (tid == 0) s_seg[par][0] = f;
            nseg = 1;
            out = a.dw_slot + (size_t)sl * a.M * a.N;
        }
        wait_lgkm0();
        block_sync();
        nst = 0;
        for (int i = 0; i < nseg; ++i) nst += (s_seg[par][i].rows + BK - 1) / BK;
        m0 = mt * BM;
        n0 = nt * TBN;
        // (an expert without rows gets a zero gradient when the outputs are written)
        return nst > 0 || !a.accum;
    };

    // DMA issue state of the tile whose steps are being issued: per-lane byte offsets of each
    // load (k-row kk of the step, a 16-byte column chunk) from the step's first row, and a cursor
    // over the segments; columns outside the tile clamp to the last valid chunk (their products
    // only reach outputs the epilogue does not store), rows past a segment's end load zeros.
    // The cursor counts rows in issue order (ikoff); a one-segment target's first rspan rows
    // (its full steps before the last) are read rotated by roff rows: row phys(ikoff).
    uint32_t ao[T::PA], bo[T::PB];
    int ipar = 0, iseg = 0, ikoff = 0, roff = 0, rspan = 0;
    Segment icur{0, 0};
    auto phys = [&](int k) {
        const int p = k + roff;
        return k >= rspan ? k : (p >= rspan ? p - rspan : p);
    };
    auto start_issue = [&](int par) {
#pragma unroll
        for (int i = 0; i < T::PA; ++i) {
            const int p = (wave * T::PA + i) * 64 + lane;
            const int k = p >> 5, c = (p & 31) ^ ((k & 3) << 2);
            ao[i] = 2u * (uint32_t)(k * a.lda + min(m0 + c * 8, a.M - 8));
        }
#pragma unroll
        for (int i = 0; i < T::PB; ++i) {
            const int p = (wave * T::PB + i) * 64 + lane;
            const int k = p / T::BCH, c = (p % T::BCH) ^ ((k & 3) << 2);
            bo[i] = 2u * (uint32_t)(k * a.ldb + min(n0 + c * 8, a.N - 8));
        }
        ipar = par;
        iseg = 0;
        ikoff = 0;
        while (iseg < nseg && s_seg[par][iseg].rows <= 0) ++iseg;   // (never for a valid plan)
        icur = iseg < nseg ? s_seg[par][iseg] : Segment{0, 0};
        roff = 0;
        rspan = 0;
        if (nseg == 1) {
            const int full = (icur.rows - 1) / BK;   // steps before the last
            if (full > 1) {
                roff = (rot % full) * BK;
                rspan = full * BK;
            }
        }
    };
    auto issue = [&](int, int buf, int i) {
        const uint32_t la = __builtin_amdgcn_readfirstlane(lds_a + buf * T::STAGE + i * 1024);
        const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_b + buf * T::STAGE + i * 1024);
        const int row = __builtin_amdgcn_readfirstlane(icur.row0 + phys(ikoff));
        const int left = __builtin_amdgcn_readfirstlane(icur.rows - ikoff);
        const uint16_t* ga = a.A + (size_t)row * a.lda;
        const uint16_t* gb = a.B + (size_t)row * a.ldb;
        if (__builtin_expect(left >= BK, 1)) {   // all but a segment's last step: fall-through path
            dma16s(ga, ao[i], la);
            if (i < T::PB) dma16s(gb, bo[i], lb);
        } else {    // rows past the segment's end load zeros; k-row of the lane's copy as in start_issue
            const bool va = (((wave * T::PA + i) * 64 + lane) >> 5) < left;
            dma16(va ? ga + ao[i] / 2 : w.zeros, la);
            if (i < T::PB) {
                const bool vb = ((wave * T::PB + i) * 64 + lane) / T::BCH < left;
                dma16(vb ? gb + bo[i] / 2 : w.zeros, lb);
            }
        }
        if (i == T::PA - 1) {    // step issued: advance the cursor
            ikoff += BK;
            if (__builtin_expect(ikoff >= icur.rows, 0)) {
                // next segment with rows: an empty one (a descriptor a valid plan never makes)
                // holds no step of nst, so the cursor must not spend one on it
                ikoff = 0;
                ++iseg;
                while (iseg < nseg && s_seg[ipar][iseg].rows <= 0) ++iseg;
                if (iseg < nseg) icur = s_seg[ipar][iseg];
            }
        }
    };
    // A full step that does not end its segment (more than BK rows left): no branches.
    auto issue_fast = [&](int, int buf, int i) {
        const int row = __builtin_amdgcn_readfirstlane(icur.row0 + phys(ikoff));
        dma16s(a.A + (size_t)row * a.lda, ao[i], __builtin_amdgcn_readfirstlane(lds_a + buf * T::STAGE + i * 1024));
        if (i < T::PB)
            dma16s(a.B + (size_t)row * a.ldb, bo[i], __builtin_amdgcn_readfirstlane(lds_b + buf * T::STAGE + i * 1024));
        if (i == T::PA - 1) ikoff += BK;
    };
    // how many steps issue_fast may issue in a row from the cursor
    auto fast_run = [&]() { return __builtin_amdgcn_readfirstlane((icur.rows - ikoff - 1) / BK); };

    // first tile
    int par = 0;
    int t = fetch();
    bool have = false;
    while (t < total && !(have = setup(t, 0))) t = fetch();
    if (have) {
        start_issue(0);
        dw_prologue<TBN>(nst, issue);
    }
    while (have) {
        int nxt = 0;
        if (tid == 0) nxt = atomicAdd(counter, 1);     // consumed after the main loop (an atomic
                                                       // add on purpose: see the loop's header)
        f32x16_t acc[4][2];
        zero_acc<2>(acc);
        dw_main<TBN>(acc, smem, nst, wm, wn, lane, issue, issue_fast, fast_run);
        // this tile's output, kept while the next tile is set up
        float* const cout = out;
        const int cm0 = m0, cn0 = n0;
        // next tile: descriptor, then its first three steps
        int tn = publish(nxt);
        bool next = false;
        while (tn < total && !(next = setup(tn, par ^ 1))) tn = fetch();
        if (next) {
            start_issue(par ^ 1);
            dw_prologue<TBN>(nst, issue);
        }
        // this tile's stores (unmasked for an interior tile), all retired before the next tile
        const bool full = cm0 + BM <= a.M && cn0 + TBN <= a.N;
        if (full) epi_dw<true>(a, acc, ep, wm, wn, lane, cout, cm0, cn0);
        else epi_dw<false>(a, acc, ep, wm, wn, lane, cout, cm0, cn0);
        wait_vm<0>();
        have = next;
        par ^= 1;
    }
}

__global__ void reset_counters_kernel(int* c, int n) {
    if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
}

// Before a weight-gradient launch: reset its tile counter and order the dW targets (home experts
// with their fallback replicas, then slots) by rows, descending, ties to the lower index, so the
// kernel hands out the largest first (longest-processing-time order).  The order only schedules
// tiles: every target's result is the same in any order.
constexpr int kOrderThreads = 512;
__global__ __launch_bounds__(kOrderThreads) void dw_prepare_kernel(PlanWs w, int* counter) {
    extern __shared__ unsigned long long okey[];   // [E + R*B]
    const int tid = threadIdx.x;
    const int ntarget = w.E + w.R * w.B;
    if (tid < 8) counter[tid] = 0;
    for (int t = tid; t < ntarget; t += kOrderThreads) {
        int rows = 0;
        if (t < w.E) {
            const Segment hs = w.home_seg[t];
            rows = seg_ok(hs, w) ? hs.rows : 0;
            const int nfb = min(max(w.fb_n[t], 0), kMaxR - 1);
            for (int i = 0; i < nfb; ++i) {
                const Segment f = w.fb_seg[(size_t)t * kMaxR + i];
                rows += seg_ok(f, w) ? f.rows : 0;
            }
        } else if (w.slot_e[t - w.E] >= 0) {
            rows = max(w.slot_rows[t - w.E], 0);
        }
        okey[t] = ((unsigned long long)(unsigned)rows << 32) | (unsigned)(~t);
    }
    __syncthreads();
    for (int t = tid; t < ntarget; t += kOrderThreads) {
        const unsigned long long k = okey[t];
        int rank = 0;
#pragma unroll 8
        for (int u = 0; u < ntarget; ++u) rank += okey[u] > k;
        w.dw_order[rank] = t;
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
static bool set_smem(K kernel, int bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
}

// waves along N of each kernel (2: 4 waves of 128x128; 4: 8 waves of 128x64)
#ifndef MOONEP_WN_ROWS
#define MOONEP_WN_ROWS 4
#endif
// weight-gradient tile width: 256 (one 8-wave workgroup per CU) or 128 (two 4-wave workgroups)
#ifndef MOONEP_DW_TBN
#define MOONEP_DW_TBN 256
#endif
constexpr int DW_TBN = MOONEP_DW_TBN;
static_assert(DW_TBN == 256 || DW_TBN == 128, "weight-gradient tile width");

// Resets the eight per-XCD tile counters, then runs a row kernel.
static int launch_rows(int epi, int mode, const GemmArgs& a0, hipStream_t s) {
    const int grid = (num_cus() / 8) * 8;
    constexpr int WN = MOONEP_WN_ROWS;
    GemmArgs a = a0;
    a.counter = a.w.counters + 8;
    hipLaunchKernelGGL(reset_counters_kernel, dim3(1), dim3(64), 0, s, a.counter, 8);
    MOONEP_LAUNCH_CHECK();
#define MOONEP_ROWS(M_, E_)                                                                            \
    do {                                                                                               \
        static bool ok = set_smem(gemm_rows_kernel<M_, E_, WN>, ROWS_SMEM);                            \
        if (!ok) return MOONEP_EHIP;                                                                   \
        hipLaunchKernelGGL((gemm_rows_kernel<M_, E_, WN>), dim3(grid), dim3(128 * WN), ROWS_SMEM, s, a); \
    } while (0)
    if (epi == EPI_SWIGLU_FWD && mode == ROWS_BN) MOONEP_ROWS(ROWS_BN, EPI_SWIGLU_FWD);
    else if (epi == EPI_STORE && mode == ROWS_BN) MOONEP_ROWS(ROWS_BN, EPI_STORE);
    else if (epi == EPI_SWIGLU_BWD && mode == ROWS_BK) MOONEP_ROWS(ROWS_BK, EPI_SWIGLU_BWD);
    else if (epi == EPI_STORE && mode == ROWS_BK) MOONEP_ROWS(ROWS_BK, EPI_STORE);
    else return MOONEP_ENOTSUP;
#undef MOONEP_ROWS
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

// Resets the launch's eight per-XCD tile counters and orders the targets, then runs the
// weight-gradient kernel with each target's tile grid cut into eight blocks (fm x 8/fm of them;
// the split with the fewest panels per block, dw_bm + dw_bn).
template <int WHICH>
static int launch_dw(const GemmArgs& a0, hipStream_t s) {
    GemmArgs a = a0;
    const int MT = (a.M + BM - 1) / BM, NT = a.ntiles_n;
    a.dw_fn = 8;
    a.dw_bm = MT;
    a.dw_bn = (NT + 7) / 8;
    for (int fm = 2; fm <= 8; fm *= 2) {
        const int bm = (MT + fm - 1) / fm, bn = (NT + 8 / fm - 1) / (8 / fm);
        if (bm + bn < a.dw_bm + a.dw_bn) {
            a.dw_fn = 8 / fm;
            a.dw_bm = bm;
            a.dw_bn = bn;
        }
    }
    constexpr int smem = DWT<DW_TBN>::SMEM;
    static bool ok = set_smem(gemm_dw_kernel<DW_TBN, WHICH>, smem);
    if (!ok) return MOONEP_EHIP;
    const size_t okey_bytes = (size_t)(a.w.E + a.w.R * a.w.B) * sizeof(unsigned long long);
    static bool ok_order = set_smem(dw_prepare_kernel, (int)((kMaxE + kMaxR * kMaxB) * sizeof(unsigned long long)));
    if (!ok_order) return MOONEP_EHIP;
    hipLaunchKernelGGL(dw_prepare_kernel, dim3(1), dim3(kOrderThreads), okey_bytes, s, a.w, a.counter);
    MOONEP_LAUNCH_CHECK();
    const int grid = (num_cus() / 8) * 8 * (DW_TBN == 128 ? 2 : 1);
    hipLaunchKernelGGL((gemm_dw_kernel<DW_TBN, WHICH>), dim3(grid), dim3(DWT<DW_TBN>::NTHR), smem, s, a);
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

// Phases of one call selected by flags: the call's bits that are set, or all of them.
static uint32_t phases(const moonep_dims_t* d, uint32_t mine) {
    const uint32_t p = d->flags & mine;
    return p ? p : mine;
}

static int check_ffn_dims(const moonep_dims_t* d) {
    int rc = check_dims(d, true);
    if (rc != MOONEP_OK) return rc;
    if (d->flags & MOONEP_F32_ROWS) return MOONEP_ENOTSUP;   // the expert GEMM is bf16
    if (d->H % 64 != 0 || d->I % 64 != 0) return MOONEP_ENOTSUP;
    // the row kernels address operands with 32-bit element offsets
    if ((long long)d->R * d->S * d->K * std::max(d->H, 2 * d->I) >= (1ll << 31)) return MOONEP_ENOTSUP;
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
    const uint32_t ph = phases(dims, kFwdPhases);
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(64), 0, s, a.w);
    MOONEP_LAUNCH_CHECK();
    if (ph & MOONEP_PHASE_GATE_UP) {
        rc = launch_rows(EPI_SWIGLU_FWD, ROWS_BN, a, s);
        if (rc != MOONEP_OK) return rc;
    }
    if (!(ph & MOONEP_PHASE_DOWN)) return MOONEP_OK;
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
    return launch_rows(EPI_STORE, ROWS_BN, a, s);
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
    const uint32_t ph = phases(dims, kBwdPhases);
    if (ph & (MOONEP_PHASE_DACT | MOONEP_PHASE_DX)) {
        hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(64), 0, s, a.w);
        MOONEP_LAUNCH_CHECK();
    }
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
    if (ph & MOONEP_PHASE_DACT) {
        rc = launch_rows(EPI_SWIGLU_BWD, ROWS_BK, a, s);
        if (rc != MOONEP_OK) return rc;
    }
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
    if (ph & MOONEP_PHASE_DX) {
        rc = launch_rows(EPI_STORE, ROWS_BK, a, s);
        if (rc != MOONEP_OK) return rc;
    }
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
    d.ntiles_n = (H + DW_TBN - 1) / DW_TBN;
    d.counter = a.w.counters + 16;
    d.accum = (dims->flags & MOONEP_GRAD_ACCUM) ? 1 : 0;
    if (ph & MOONEP_PHASE_DW2) {
        rc = launch_dw<2>(d, s);
        if (rc != MOONEP_OK) return rc;
    }
    // dW13 = X^T [dGt dU]  ([H, 2I])
    d.A = static_cast<const uint16_t*>(recv);
    d.lda = H;
    d.B = gu;
    d.ldb = 2 * I;
    d.M = H;
    d.N = 2 * I;
    d.dw_home = dw13_home;
    d.dw_slot = dw13_red;
    d.ntiles_n = (2 * I + DW_TBN - 1) / DW_TBN;
    d.counter = a.w.counters + 24;
    return (ph & MOONEP_PHASE_DW13) ? launch_dw<13>(d, s) : MOONEP_OK;
}
