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
// (dispatch); K rows are gathered with all loads of a vector batch in flight before
// the float32 accumulation (combine).
#include "common.h"

namespace moonep {

constexpr int kWavesPerBlock = 4;

template <bool F32, bool SCALE>
__device__ __forceinline__ uint4 scale_vec(uint4 v, float g) {
    if (!SCALE) return v;
    uint4 o;
    if (F32) {
        o.x = __float_as_uint(__uint_as_float(v.x) * g);
        o.y = __float_as_uint(__uint_as_float(v.y) * g);
        o.z = __float_as_uint(__uint_as_float(v.z) * g);
        o.w = __float_as_uint(__uint_as_float(v.w) * g);
    } else {
        o.x = pack_bf16(bf16_lo(v.x) * g, bf16_hi(v.x) * g);
        o.y = pack_bf16(bf16_lo(v.y) * g, bf16_hi(v.y) * g);
        o.z = pack_bf16(bf16_lo(v.z) * g, bf16_hi(v.z) * g);
        o.w = pack_bf16(bf16_lo(v.w) * g, bf16_hi(v.w) * g);
    }
    return o;
}

// recv[dest[p]] = scale(src[token(p)]); one wave per token, 16-byte vectors per lane.
// IDENT: dest[p] = p (rows land in arrival order: the first copy of the staged baseline).
template <bool F32, bool SCALE, int VB, bool IDENT = false>
__global__ __launch_bounds__(256) void dispatch_kernel(const int32_t* __restrict__ dest,
                                                       const uint4* __restrict__ src,
                                                       const float* __restrict__ scale,
                                                       uint4* __restrict__ recv, int ntok, int K,
                                                       int rowvec, long long nrows) {
    const int tok = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (tok >= ntok) return;
    const int32_t* dp = dest + (size_t)tok * K;
    const float* gp = SCALE ? scale + (size_t)tok * K : nullptr;
    const uint4* s = src + (size_t)tok * rowvec;
    for (int v0 = 0; v0 < rowvec; v0 += 64 * VB) {
        uint4 x[VB];
#pragma unroll
        for (int u = 0; u < VB; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v < rowvec) x[u] = ld_nt(s + v);
        }
        for (int k = 0; k < K; ++k) {
            const int d = IDENT ? tok * K + k : dp[k];
            if ((unsigned long long)(long long)d >= (unsigned long long)nrows) continue;
            const float g = SCALE ? gp[k] : 1.0f;
            uint4* o = recv + (size_t)d * rowvec;
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                const int v = v0 + u * 64 + lane;
                if (v < rowvec) st_nt(scale_vec<F32, SCALE>(x[u], g), o + v);
            }
        }
    }
}

template <bool F32>
__device__ __forceinline__ void acc_vec(float* a, uint4 v, float g) {
    if (F32) {
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
// KT > 0: compile-time K (all K loads of a vector batch issued before accumulating).
// IDENT: dest[p] = p (rows read in arrival order: the reduction of the staged baseline).
template <bool F32, bool GATES, int KT, int VB, bool IDENT = false>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ dest,
                                                      const uint4* __restrict__ y,
                                                      const float* __restrict__ gates,
                                                      uint4* __restrict__ out, int ntok, int Krt,
                                                      int rowvec, long long nrows) {
    constexpr int NE = F32 ? 4 : 8;
    const int K = KT > 0 ? KT : Krt;
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
        if (KT > 0) {
            uint4 x[KT > 0 ? KT : 1][VB];
#pragma unroll
            for (int k = 0; k < (KT > 0 ? KT : 1); ++k) {
                const int d = IDENT ? tok * K + k : dp[k];
                const bool ok = (unsigned long long)(long long)d < (unsigned long long)nrows;
                const uint4* yr = y + (size_t)(ok ? d : 0) * rowvec;
#pragma unroll
                for (int u = 0; u < VB; ++u) {
                    const int v = v0 + u * 64 + lane;
                    x[k][u] = (ok && v < rowvec) ? ld_nt(yr + v) : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int k = 0; k < (KT > 0 ? KT : 1); ++k) {
                const float g = GATES ? gp[k] : 1.0f;
#pragma unroll
                for (int u = 0; u < VB; ++u) acc_vec<F32>(acc[u], x[k][u], g);
            }
        } else {
            for (int k = 0; k < K; ++k) {
                const int d = IDENT ? tok * K + k : dp[k];
                if ((unsigned long long)(long long)d >= (unsigned long long)nrows) continue;
                const float g = GATES ? gp[k] : 1.0f;
                const uint4* yr = y + (size_t)d * rowvec;
#pragma unroll
                for (int u = 0; u < VB; ++u) {
                    const int v = v0 + u * 64 + lane;
                    if (v < rowvec) acc_vec<F32>(acc[u], ld_nt(yr + v), g);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < VB; ++u) {
            const int v = v0 + u * 64 + lane;
            if (v >= rowvec) continue;
            uint4 r;
            if (F32) {
                r.x = __float_as_uint(acc[u][0]);
                r.y = __float_as_uint(acc[u][1]);
                r.z = __float_as_uint(acc[u][2]);
                r.w = __float_as_uint(acc[u][3]);
            } else {
                r.x = pack_bf16(acc[u][0], acc[u][1]);
                r.y = pack_bf16(acc[u][2], acc[u][3]);
                r.z = pack_bf16(acc[u][4], acc[u][5]);
                r.w = pack_bf16(acc[u][6], acc[u][7]);
            }
            st_nt(r, o + v);
        }
    }
}

template <bool F32, bool GATES, bool IDENT = false>
static void launch_combine(int K, dim3 grid, hipStream_t s, const int32_t* dest, const uint4* y,
                           const float* gates, uint4* out, int ntok, int rowvec, long long nrows) {
    switch (K) {
        case 8:
            hipLaunchKernelGGL((combine_kernel<F32, GATES, 8, 2, IDENT>), grid, dim3(256), 0, s, dest, y, gates, out, ntok, K, rowvec, nrows);
            break;
        case 4:
            hipLaunchKernelGGL((combine_kernel<F32, GATES, 4, 4, IDENT>), grid, dim3(256), 0, s, dest, y, gates, out, ntok, K, rowvec, nrows);
            break;
        case 2:
            hipLaunchKernelGGL((combine_kernel<F32, GATES, 2, 4, IDENT>), grid, dim3(256), 0, s, dest, y, gates, out, ntok, K, rowvec, nrows);
            break;
        case 1:
            hipLaunchKernelGGL((combine_kernel<F32, GATES, 1, 4, IDENT>), grid, dim3(256), 0, s, dest, y, gates, out, ntok, K, rowvec, nrows);
            break;
        default:
            hipLaunchKernelGGL((combine_kernel<F32, GATES, 0, 2, IDENT>), grid, dim3(256), 0, s, dest, y, gates, out, ntok, K, rowvec, nrows);
    }
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
        if (row_scale)
            hipLaunchKernelGGL((dispatch_kernel<true, true, 4>), grid, dim3(256), 0, s, dest, sv, row_scale, rv, ntok, dims->K, rowvec, nrows);
        else
            hipLaunchKernelGGL((dispatch_kernel<true, false, 4>), grid, dim3(256), 0, s, dest, sv, row_scale, rv, ntok, dims->K, rowvec, nrows);
    } else {
        if (row_scale)
            hipLaunchKernelGGL((dispatch_kernel<false, true, 4>), grid, dim3(256), 0, s, dest, sv, row_scale, rv, ntok, dims->K, rowvec, nrows);
        else
            hipLaunchKernelGGL((dispatch_kernel<false, false, 4>), grid, dim3(256), 0, s, dest, sv, row_scale, rv, ntok, dims->K, rowvec, nrows);
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
        if (row_scale)
            hipLaunchKernelGGL((dispatch_kernel<true, true, 4, true>), grid, dim3(256), 0, s, dest, sv, row_scale, tv, ntok, dims->K, rowvec, nrows);
        else
            hipLaunchKernelGGL((dispatch_kernel<true, false, 4, true>), grid, dim3(256), 0, s, dest, sv, row_scale, tv, ntok, dims->K, rowvec, nrows);
    } else {
        if (row_scale)
            hipLaunchKernelGGL((dispatch_kernel<false, true, 4, true>), grid, dim3(256), 0, s, dest, sv, row_scale, tv, ntok, dims->K, rowvec, nrows);
        else
            hipLaunchKernelGGL((dispatch_kernel<false, false, 4, true>), grid, dim3(256), 0, s, dest, sv, row_scale, tv, ntok, dims->K, rowvec, nrows);
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
