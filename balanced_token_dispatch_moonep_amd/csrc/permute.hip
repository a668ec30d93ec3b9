// Fused zero-copy permute (dispatch) and unpermute (combine).
//
// Pages cited: [TC] thakicloud.com "The Busiest Rank Sets Your Step Time: Running
// MoonEP's Planning Code Ourselves"; [AL] agentlenshq.com "MoonshotAI/MoonEP";
// [TD] twodots.gr "MoonEP balances AI experts in MoE models ...".
//
// Dispatch writes each (token, k) row straight into its final expert-grouped row of
// the static [R, S*K, H] receive buffer, at the row the planner computed on the send
// side; there is no receive-then-sort copy and the grouped GEMM reads the buffer in
// place [TC, "What the technique is"; AL, How it works; TD, architecture].  Combine
// gathers the K expert outputs of a token back into token order [TC, flowchart].
//
// Both are HBM-bound row copies.  One wave owns one token: each lane moves 16-byte
// vectors, so every load or store instruction of the wave covers 1 KiB of one row
// (fully coalesced).  The token's source row is read once and written K times
// (dispatch); the K rows of a token are gathered one after another, a chunk of the row
// at a time, into float32 accumulators (combine).
#include "common.h"

namespace moonep {

constexpr int kWavesPerBlock = 4;
// Vectors (16 bytes) per lane that one batch of a row moves; chosen by measurement on MI355X at
// H = 7168 (896 vectors per bf16 row).
#ifndef MOONEP_DISPATCH_VB
#define MOONEP_DISPATCH_VB 2
#endif
#ifndef MOONEP_DISPATCH_SCALED_VB
#define MOONEP_DISPATCH_SCALED_VB 2
#endif
#ifndef MOONEP_COMBINE_VB
#define MOONEP_COMBINE_VB 7
#endif

template <bool F32, bool SCALE>
__device__ __forceinline__ uint4 scale_vec(uint4 v, float g) {
    if constexpr (!SCALE) {
        return v;
    } else if constexpr (F32) {
        return make_uint4(__float_as_uint(__uint_as_float(v.x) * g), __float_as_uint(__uint_as_float(v.y) * g),
                          __float_as_uint(__uint_as_float(v.z) * g), __float_as_uint(__uint_as_float(v.w) * g));
    } else {
        return make_uint4(pack_bf16(bf16_lo(v.x) * g, bf16_hi(v.x) * g), pack_bf16(bf16_lo(v.y) * g, bf16_hi(v.y) * g),
                          pack_bf16(bf16_lo(v.z) * g, bf16_hi(v.z) * g), pack_bf16(bf16_lo(v.w) * g, bf16_hi(v.w) * g));
    }
}

// recv[dest[p]] = scale(src[token(p)]); one wave per token, 16-byte vectors per lane.
// A batch of VB vectors per lane of the source row is read once (non-temporal) and written to
// the token's K destination rows with ordinary stores (measured faster than non-temporal ones
// for this scatter of 1 KiB wave segments).  KT > 0 (the scaled form at K = 8): compile-time
// K, and the token's K destinations and scales are read once, before its row, which keeps the
// scale loads out of the store loop; the unscaled form reads its destinations in the loop
// (measured faster).
// IDENT: dest[p] = p (rows land in arrival order: the first copy of the staged baseline).
// FULL: the row is a whole number of batches (64 VB vectors), so no vector needs a bounds check.
template <bool F32, bool SCALE, int KT, int VB, bool IDENT = false, bool FULL = false>
__global__ __launch_bounds__(256) void dispatch_kernel(const int32_t* __restrict__ dest,
                                                       const uint4* __restrict__ src,
                                                       const float* __restrict__ scale,
                                                       uint4* __restrict__ recv, int ntok, int Krt,
                                                       int rowvec, long long nrows) {
    constexpr int KA = KT > 0 ? KT : 1;
    const int K = KT > 0 ? KT : Krt;
    const int tok = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (tok >= ntok) return;
    const int32_t* dp = dest + (size_t)tok * K;
    const float* gp = SCALE ? scale + (size_t)tok * K : nullptr;
    const uint4* s = src + (size_t)tok * rowvec;
    int dk[KA];
    float gk[KA];
    if constexpr (KT > 0) {
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            dk[k] = IDENT ? tok * KT + k : dp[k];
            gk[k] = SCALE ? gp[k] : 1.0f;
        }
    }
    for (int v0 = 0; v0 < rowvec; v0 += 64 * VB) {
        uint4 x[VB];
#pragma unroll
        for (int u = 0; u < VB; ++u) {
            const int v = v0 + u * 64 + lane;
            if (FULL || v < rowvec) x[u] = ld_nt(s + v);
        }
        auto put = [&](int d, float g) {
            if ((unsigned long long)(long long)d >= (unsigned long long)nrows) return;
            uint4* o = recv + (size_t)d * rowvec;
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int v = v0 + u * 64 + lane;
                if (FULL || v < rowvec) o[v] = scale_vec<F32, SCALE>(x[u], g);
            }
        };
        if constexpr (KT > 0) {
#pragma unroll
            for (int k = 0; k < KT; ++k) put(dk[k], gk[k]);
        } else {
            for (int k = 0; k < K; ++k) put(IDENT ? tok * K + k : dp[k], SCALE ? gp[k] : 1.0f);
        }
    }
}

template <bool F32>
__device__ __forceinline__ void acc_vec(float* a, uint4 v, float g) {
    if constexpr (F32) {
        a[0] += g * __uint_as_float(v.x);
        a[1] += g * __uint_as_float(v.y);
        a[2] += g * __uint_as_float(v.z);
        a[3] += g * __uint_as_float(v.w);
    } else {
        a[0] += g * bf16_lo(v.x);
        a[1] += g * bf16_hi(v.x);
        a[2] += g * bf16_lo(v.y);
        a[3] += g * bf16_hi(v.y);
        a[4] += g * bf16_lo(v.z);
        a[5] += g * bf16_hi(v.z);
        a[6] += g * bf16_lo(v.w);
        a[7] += g * bf16_hi(v.w);
    }
}

// out[token] = sum_k g_k * y[dest[p_k]] (k order, float32); one wave per token.
// The output row is produced in chunks of VB vectors per lane; for a chunk the K source rows
// are read one after another, VB KiB of one row at a time (measured faster than keeping all K
// rows' loads in flight, which spreads each wave over K places of HBM at once).
// IDENT: dest[p] = p (rows read in arrival order: the reduction of the staged baseline).
// FULL: as for dispatch_kernel.
template <bool F32, bool GATES, int VB, bool IDENT = false, bool FULL = false>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ dest,
                                                      const uint4* __restrict__ y,
                                                      const float* __restrict__ gates,
                                                      uint4* __restrict__ out, int ntok, int K,
                                                      int rowvec, long long nrows) {
    constexpr int NE = F32 ? 4 : 8;
    const int tok = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (tok >= ntok) return;
    const int32_t* dp = dest + (size_t)tok * K;
    const float* gp = GATES ? gates + (size_t)tok * K : nullptr;
    uint4* o = out + (size_t)tok * rowvec;
    for (int v0 = 0; v0 < rowvec; v0 += 64 * VB) {
        float acc[VB][NE];
#pragma unroll
        for (int u = 0; u < VB; ++u)
#pragma unroll
            for (int i = 0; i < NE; ++i) acc[u][i] = 0.0f;
#pragma unroll 1
        for (int k = 0; k < K; ++k) {
            const int d = IDENT ? tok * K + k : dp[k];
            if ((unsigned long long)(long long)d >= (unsigned long long)nrows) continue;
            const float g = GATES ? gp[k] : 1.0f;
            const uint4* yr = y + (size_t)d * rowvec;
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int v = v0 + u * 64 + lane;
                if (FULL || v < rowvec) acc_vec<F32>(acc[u], ld_nt(yr + v), g);
            }
        }
#pragma unroll
        for (int u = 0; u < VB; ++u) {
            const int v = v0 + u * 64 + lane;
            if (!FULL && v >= rowvec) continue;
            uint4 r;
            if constexpr (F32) {
                r = make_uint4(__float_as_uint(acc[u][0]), __float_as_uint(acc[u][1]), __float_as_uint(acc[u][2]),
                               __float_as_uint(acc[u][3]));
            } else {
                r = make_uint4(pack_bf16(acc[u][0], acc[u][1]), pack_bf16(acc[u][2], acc[u][3]),
                               pack_bf16(acc[u][4], acc[u][5]), pack_bf16(acc[u][6], acc[u][7]));
            }
            st_nt(r, o + v);
        }
    }
}

template <bool F32, bool SCALE, bool IDENT = false>
static void launch_dispatch(int K, dim3 grid, hipStream_t s, const int32_t* dest, const uint4* src,
                            const float* scale, uint4* recv, int ntok, int rowvec, long long nrows) {
    constexpr int VB = SCALE ? MOONEP_DISPATCH_SCALED_VB : MOONEP_DISPATCH_VB;
    const bool full = rowvec % (64 * VB) == 0;   // (measured neutral here; fewer instructions)
    if constexpr (SCALE) {
        if (K == 8) {
            if (full) hipLaunchKernelGGL((dispatch_kernel<F32, SCALE, 8, VB, IDENT, true>), grid, dim3(256), 0, s, dest, src, scale, recv, ntok, K, rowvec, nrows);
            else hipLaunchKernelGGL((dispatch_kernel<F32, SCALE, 8, VB, IDENT, false>), grid, dim3(256), 0, s, dest, src, scale, recv, ntok, K, rowvec, nrows);
            return;
        }
    }
    if (full) hipLaunchKernelGGL((dispatch_kernel<F32, SCALE, 0, VB, IDENT, true>), grid, dim3(256), 0, s, dest, src, scale, recv, ntok, K, rowvec, nrows);
    else hipLaunchKernelGGL((dispatch_kernel<F32, SCALE, 0, VB, IDENT, false>), grid, dim3(256), 0, s, dest, src, scale, recv, ntok, K, rowvec, nrows);
}

template <bool F32, bool GATES, bool IDENT = false>
static void launch_combine(int K, dim3 grid, hipStream_t s, const int32_t* dest, const uint4* y,
                           const float* gates, uint4* out, int ntok, int rowvec, long long nrows) {
    // the full-row form measured 2% faster with gates and 2% slower with unit weights
    if (GATES && rowvec % (64 * MOONEP_COMBINE_VB) == 0)
        hipLaunchKernelGGL((combine_kernel<F32, GATES, MOONEP_COMBINE_VB, IDENT, true>), grid, dim3(256), 0, s, dest, y, gates, out, ntok, K, rowvec, nrows);
    else
        hipLaunchKernelGGL((combine_kernel<F32, GATES, MOONEP_COMBINE_VB, IDENT, false>), grid, dim3(256), 0, s, dest, y, gates, out, ntok, K, rowvec, nrows);
}

// The sort-copy of the staged baseline, one wave per row p, 16-byte vectors per lane:
// GATHER: out[p] = in[dest[p]]; otherwise out[dest[p]] = in[p].
template <bool GATHER>
__global__ __launch_bounds__(256) void permute_rows_kernel(const int32_t* __restrict__ dest,
                                                           const uint4* __restrict__ in, uint4* __restrict__ out,
                                                           long long nrows, int rowvec) {
    const long long p = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (p >= nrows) return;
    const int d = dest[p];
    if ((unsigned long long)(long long)d >= (unsigned long long)nrows) return;
    const uint4* src = in + (size_t)(GATHER ? d : p) * rowvec;
    uint4* dst = out + (size_t)(GATHER ? p : d) * rowvec;
    for (int v0 = 0; v0 < rowvec; v0 += 64 * 4) {
        uint4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < rowvec) x[u] = ld_nt(src + v);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < rowvec) st_nt(x[u], dst + v);
        }
    }
}

}  // namespace moonep

using namespace moonep;

extern "C" int moonep_dispatch(const moonep_dims_t* dims, const int32_t* dest, const void* src,
                               const float* row_scale, void* recv, void* stream) {
    const int rc = check_dims(dims, false);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(dest);
    MOONEP_CHECK_PTR(src);
    MOONEP_CHECK_PTR(recv);
    if (row_scale && !aligned16(row_scale)) return MOONEP_EALIGN;
    const bool f32 = (dims->flags & MOONEP_F32_ROWS) != 0;
    const int ntok = dims->R * dims->S;
    const int rowvec = dims->H * (f32 ? 4 : 2) / 16;
    const long long nrows = (long long)ntok * dims->K;
    const dim3 grid((ntok + kWavesPerBlock - 1) / kWavesPerBlock);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* sv = static_cast<const uint4*>(src);
    uint4* rv = static_cast<uint4*>(recv);
    if (f32) {
        if (row_scale) launch_dispatch<true, true>(dims->K, grid, s, dest, sv, row_scale, rv, ntok, rowvec, nrows);
        else launch_dispatch<true, false>(dims->K, grid, s, dest, sv, row_scale, rv, ntok, rowvec, nrows);
    } else {
        if (row_scale) launch_dispatch<false, true>(dims->K, grid, s, dest, sv, row_scale, rv, ntok, rowvec, nrows);
        else launch_dispatch<false, false>(dims->K, grid, s, dest, sv, row_scale, rv, ntok, rowvec, nrows);
    }
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

extern "C" int moonep_combine(const moonep_dims_t* dims, const int32_t* dest, const void* y,
                              const float* gates, void* out, void* stream) {
    const int rc = check_dims(dims, false);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(dest);
    MOONEP_CHECK_PTR(y);
    MOONEP_CHECK_PTR(out);
    if (gates && !aligned16(gates)) return MOONEP_EALIGN;
    const bool f32 = (dims->flags & MOONEP_F32_ROWS) != 0;
    const int ntok = dims->R * dims->S;
    const int rowvec = dims->H * (f32 ? 4 : 2) / 16;
    const long long nrows = (long long)ntok * dims->K;
    const dim3 grid((ntok + kWavesPerBlock - 1) / kWavesPerBlock);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* yv = static_cast<const uint4*>(y);
    uint4* ov = static_cast<uint4*>(out);
    if (f32) {
        if (gates) launch_combine<true, true>(dims->K, grid, s, dest, yv, gates, ov, ntok, rowvec, nrows);
        else launch_combine<true, false>(dims->K, grid, s, dest, yv, gates, ov, ntok, rowvec, nrows);
    } else {
        if (gates) launch_combine<false, true>(dims->K, grid, s, dest, yv, gates, ov, ntok, rowvec, nrows);
        else launch_combine<false, false>(dims->K, grid, s, dest, yv, gates, ov, ntok, rowvec, nrows);
    }
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

extern "C" int moonep_dispatch_staged(const moonep_dims_t* dims, const int32_t* dest, const void* src,
                                      const float* row_scale, void* stage, void* recv, void* stream) {
    const int rc = check_dims(dims, false);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(dest);
    MOONEP_CHECK_PTR(src);
    MOONEP_CHECK_PTR(stage);
    MOONEP_CHECK_PTR(recv);
    if (row_scale && !aligned16(row_scale)) return MOONEP_EALIGN;
    const bool f32 = (dims->flags & MOONEP_F32_ROWS) != 0;
    const int ntok = dims->R * dims->S;
    const int rowvec = dims->H * (f32 ? 4 : 2) / 16;
    const long long nrows = (long long)ntok * dims->K;
    const dim3 grid((ntok + kWavesPerBlock - 1) / kWavesPerBlock);
    const dim3 rgrid((unsigned)((nrows + kWavesPerBlock - 1) / kWavesPerBlock));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* sv = static_cast<const uint4*>(src);
    uint4* tv = static_cast<uint4*>(stage);
    // 1. arrival order: stage[(r, s, k)] = scale(src[r, s])
    if (f32) {
        if (row_scale) launch_dispatch<true, true, true>(dims->K, grid, s, dest, sv, row_scale, tv, ntok, rowvec, nrows);
        else launch_dispatch<true, false, true>(dims->K, grid, s, dest, sv, row_scale, tv, ntok, rowvec, nrows);
    } else {
        if (row_scale) launch_dispatch<false, true, true>(dims->K, grid, s, dest, sv, row_scale, tv, ntok, rowvec, nrows);
        else launch_dispatch<false, false, true>(dims->K, grid, s, dest, sv, row_scale, tv, ntok, rowvec, nrows);
    }
    MOONEP_LAUNCH_CHECK();
    // 2. the sort into expert order: recv[dest[p]] = stage[p]
    hipLaunchKernelGGL((permute_rows_kernel<false>), rgrid, dim3(256), 0, s, dest, tv, static_cast<uint4*>(recv),
                       nrows, rowvec);
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

extern "C" int moonep_combine_staged(const moonep_dims_t* dims, const int32_t* dest, const void* y,
                                     const float* gates, void* stage, void* out, void* stream) {
    const int rc = check_dims(dims, false);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(dest);
    MOONEP_CHECK_PTR(y);
    MOONEP_CHECK_PTR(stage);
    MOONEP_CHECK_PTR(out);
    if (gates && !aligned16(gates)) return MOONEP_EALIGN;
    const bool f32 = (dims->flags & MOONEP_F32_ROWS) != 0;
    const int ntok = dims->R * dims->S;
    const int rowvec = dims->H * (f32 ? 4 : 2) / 16;
    const long long nrows = (long long)ntok * dims->K;
    const dim3 grid((ntok + kWavesPerBlock - 1) / kWavesPerBlock);
    const dim3 rgrid((unsigned)((nrows + kWavesPerBlock - 1) / kWavesPerBlock));
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint4* tv = static_cast<uint4*>(stage);
    // 1. back to arrival order: stage[p] = y[dest[p]]
    hipLaunchKernelGGL((permute_rows_kernel<true>), rgrid, dim3(256), 0, s, dest, static_cast<const uint4*>(y), tv,
                       nrows, rowvec);
    MOONEP_LAUNCH_CHECK();
    // 2. reduction over k in arrival order (same arithmetic as moonep_combine)
    uint4* ov = static_cast<uint4*>(out);
    if (f32) {
        if (gates) launch_combine<true, true, true>(dims->K, grid, s, dest, tv, gates, ov, ntok, rowvec, nrows);
        else launch_combine<true, false, true>(dims->K, grid, s, dest, tv, gates, ov, ntok, rowvec, nrows);
    } else {
        if (gates) launch_combine<false, true, true>(dims->K, grid, s, dest, tv, gates, ov, ntok, rowvec, nrows);
        else launch_combine<false, false, true>(dims->K, grid, s, dest, tv, gates, ov, ntok, rowvec, nrows);
    }
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}
