// Internal declarations shared by the libmoonep HIP sources: argument checks,
// the layout of the opaque plan workspace, and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/moonep.h"

namespace moonep {

constexpr int kChunk = 64;           // tokens per planning chunk (one wave, one 64-bit bitmap)
constexpr int kMaxR = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxG = 64;            // home experts per rank
constexpr int kMaxB = 64;
constexpr int kMaxK = 16;
// chunks per planning histogram segment, at most (fewer segments: less for plan_decide to sum;
// more: more workgroups for plan_hist)
#ifndef MOONEP_PLAN_SEG
#define MOONEP_PLAN_SEG 8
#endif
constexpr int kSegMax = MOONEP_PLAN_SEG;
constexpr int kZeroElems = 512;      // zero bf16 elements kept in the plan workspace
constexpr uint32_t kFwdPhases = MOONEP_PHASE_GATE_UP | MOONEP_PHASE_DOWN;
constexpr uint32_t kBwdPhases = MOONEP_PHASE_DACT | MOONEP_PHASE_DX | MOONEP_PHASE_DW2 | MOONEP_PHASE_DW13;
constexpr uint32_t kPhaseBits = kFwdPhases | kBwdPhases;

// Header words of the plan workspace.
enum HdrWord {
    HDR_STATUS = 0,
    HDR_NENTRIES = 1,
    HDR_NGROUPS = 2,
    HDR_NSLOTREP = 3,   // replicas holding a prefetch slot
    HDR_NRED = 4,       // experts with at least one slot replica
    HDR_WORDS = 64
};

// Group descriptor (one GEMM group = one (rank, weight row) with rows > 0).
struct Group {
    int32_t row0;    // first absolute row in the [R*C] receive buffer
    int32_t rows;
    int32_t wsel;    // >= 0: home weight row (home or fallback); < 0: -1 - (q*B + j) slot
    int32_t expert;  // expert whose weights the group uses
};

// dW target: one home expert (its home rows + fallback replicas) or one slot replica.
struct Segment {
    int32_t row0;
    int32_t rows;
};

// Plan workspace layout.  Every array is rewritten by each moonep_plan call before it is read.
struct PlanWs {
    int R, E, B, S, K, G, C, NC, NCH;
    int SEG, NSEG;         // chunks per histogram segment (consecutive in (rank, token) order), segments
    int32_t* hdr;          // [HDR_WORDS]
    uint64_t* bm;          // [NCH][E]   bit t of bm[ch][e]: token t of chunk ch picked e
    int32_t* cnt;          // [NCH][E]   pairs of e in the earlier chunks of ch's segment
    int32_t* segtot;       // [NSEG][E]  pairs of e in each segment
    int32_t* segpre;       // [NSEG][E]  pairs of e in the earlier segments
    int32_t* chunk_status; // [NSEG]     invalid / duplicate ids seen in each segment
    int32_t* keep;         // [E]
    int32_t* ninst;        // [E]
    int32_t* inst;         // [E][kMaxR][3]  (start g, rows, dest offset = q*C + cu - start)
    int32_t* entries;      // [E][5]  (e, q, a, j, w) in creation order
    Group* groups;         // [2E]
    int32_t* slot_e;       // [R*B] expert held by slot (q, j), -1 if unused
    int32_t* slot_row0;    // [R*B] first row of the slot group, rows in slot_rows
    int32_t* slot_rows;    // [R*B]
    int32_t* red_n;        // [E] slot replicas of expert e
    int32_t* red_slot;     // [E][kMaxR] their slot ids q*B+j in creation order
    int32_t* fb_n;         // [E] fallback replicas of expert e
    Segment* fb_seg;       // [E][kMaxR]
    Segment* home_seg;     // [E]
    int32_t* counters;     // [64] tile counters of dynamically scheduled kernels
    int32_t* dw_order;     // [E + R*B] dW targets by rows, descending (ties: lower id); written
                           // before each weight-gradient launch
    uint16_t* zeros;       // [kZeroElems] zero bf16 row segment (source of masked GEMM tile loads)
    int32_t* tile_pref;    // [2E + 1] prefix over the groups of their 256-row GEMM tiles
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Computes the layout; when base is NULL only the total size is meaningful.
inline size_t plan_ws_layout(const moonep_dims_t* d, void* base, PlanWs* ws) {
    PlanWs w{};
    w.R = d->R; w.E = d->E; w.B = d->B; w.S = d->S; w.K = d->K;
    w.G = d->E / d->R; w.C = d->S * d->K;
    w.NC = (d->S + kChunk - 1) / kChunk;
    w.NCH = w.R * w.NC;
    // a segment's bitmaps fill at most 64 KiB of LDS
    w.SEG = std::max(1, std::min(kSegMax, 8192 / w.E));
    w.NSEG = (w.NCH + w.SEG - 1) / w.SEG;
    size_t off = 0;
    char* b = static_cast<char*>(base);
    auto take = [&](size_t bytes) -> void* {
        void* p = b ? b + off : nullptr;
        off = align_up(off + bytes, 256);
        return p;
    };
    const size_t E = w.E, R = w.R, NCH = w.NCH, RB = (size_t)w.R * (w.B > 0 ? w.B : 1);
    w.hdr = (int32_t*)take(HDR_WORDS * 4);
    w.bm = (uint64_t*)take(NCH * E * 8);
    w.cnt = (int32_t*)take(NCH * E * 4);
    w.segtot = (int32_t*)take((size_t)w.NSEG * E * 4);
    w.segpre = (int32_t*)take((size_t)w.NSEG * E * 4);
    w.chunk_status = (int32_t*)take((size_t)w.NSEG * 4);
    w.keep = (int32_t*)take(E * 4);
    w.ninst = (int32_t*)take(E * 4);
    w.inst = (int32_t*)take(E * kMaxR * 3 * 4);
    w.entries = (int32_t*)take(E * 5 * 4);
    w.groups = (Group*)take(2 * E * sizeof(Group));
    w.slot_e = (int32_t*)take(RB * 4);
    w.slot_row0 = (int32_t*)take(RB * 4);
    w.slot_rows = (int32_t*)take(RB * 4);
    w.red_n = (int32_t*)take(E * 4);
    w.red_slot = (int32_t*)take(E * kMaxR * 4);
    w.fb_n = (int32_t*)take(E * 4);
    w.fb_seg = (Segment*)take(E * kMaxR * sizeof(Segment));
    w.home_seg = (Segment*)take(E * sizeof(Segment));
    w.counters = (int32_t*)take(64 * 4);
    w.dw_order = (int32_t*)take((E + RB) * 4);
    w.zeros = (uint16_t*)take(kZeroElems * 2);
    w.tile_pref = (int32_t*)take((2 * E + 1) * 4);
    (void)R;
    if (ws) *ws = w;
    return off;
}

// Host-side validation of dims; returns MOONEP_OK or a negative code.
inline int check_dims(const moonep_dims_t* d, bool need_ffn) {
    if (!d) return MOONEP_EINVAL;
    if (d->R < 1 || d->R > kMaxR) return MOONEP_EINVAL;
    if (d->E < d->R || d->E > kMaxE || d->E % d->R != 0) return MOONEP_EINVAL;
    if (d->E / d->R > kMaxG) return MOONEP_EINVAL;
    if (d->B < 0 || d->B > kMaxB) return MOONEP_EINVAL;
    if (d->S < 1 || d->K < 1 || d->K > kMaxK || d->K > d->E) return MOONEP_EINVAL;
    if ((int64_t)d->R * d->S * d->K > (int64_t)1 << 30) return MOONEP_EINVAL;
    if (d->H < 8 || d->H % 8 != 0) return MOONEP_EINVAL;
    if (d->flags & ~(MOONEP_TRAINING | MOONEP_F32_ROWS | MOONEP_GRAD_ACCUM | MOONEP_PLAN_LOWMIG | kPhaseBits))
        return MOONEP_EINVAL;
    if (need_ffn && (d->I < 8 || d->I % 8 != 0)) return MOONEP_EINVAL;
    return MOONEP_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MOONEP_CHECK_PTR(p)                         \
    do {                                            \
        if (!(p)) return MOONEP_EINVAL;             \
        if (!::moonep::aligned16(p)) return MOONEP_EALIGN; \
    } while (0)

#define MOONEP_LAUNCH_CHECK()                                   \
    do {                                                        \
        if (hipGetLastError() != hipSuccess) return MOONEP_EHIP; \
    } while (0)

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// two floats -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2_t v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte loads/stores with the non-temporal hint (streamed once, keep out of the way in L2)
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint4 v, uint4* p) {
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ float4 ld_nt(const float4* p) {
    const uint4 v = ld_nt(reinterpret_cast<const uint4*>(p));
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ void st_nt(float4 v, float4* p) {
    st_nt(make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)),
          reinterpret_cast<uint4*>(p));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace moonep
