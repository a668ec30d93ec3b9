// Weight prefetch into replica slots, and reduce_grad.
//
// Pages cited: [TC] thakicloud.com "The Busiest Rank Sets Your Step Time: Running
// MoonEP's Planning Code Ourselves"; [TD] twodots.gr "MoonEP balances AI experts in
// MoE models ..."; [AT] aitrending.vip "Moonshot AI Open-Sources MoonEP ...".
//
// Prefetch copies a replicated expert's home weights into the prefetch slot that the
// plan gave it on the serving rank, before the expert GEMM [TC, flowchart "Weight
// prefetch"; TD, memory contract].  reduce_grad adds every slot replica's fp32
// gradient into the home expert's gradient, in replica creation order, and clears the
// slot for the next micro-batch [TD, memory contract; AT, Technical Details].
// Both are HBM-bound streams of 16-byte vectors; which slots are live is read from the
// plan workspace on the device, so the host never waits for the plan.
#include "common.h"

namespace moonep {

constexpr int kCopyBlocks = 128;    // workgroups per slot (per tensor)

__global__ __launch_bounds__(256) void prefetch_kernel(PlanWs w, const uint4* __restrict__ w13,
                                                       const uint4* __restrict__ w2,
                                                       uint4* __restrict__ s13, uint4* __restrict__ s2,
                                                       long long n13, long long n2) {
    const int slot = blockIdx.y;
    const int e = w.slot_e[slot];
    if (e < 0 || e >= w.E) return;
    const bool first = blockIdx.z == 0;
    const long long n = first ? n13 : n2;
    const uint4* src = (first ? w13 : w2) + (size_t)e * n;
    uint4* dst = (first ? s13 : s2) + (size_t)slot * n;
    const long long per = (n + kCopyBlocks - 1) / kCopyBlocks;
    const long long lo = per * blockIdx.x;
    const long long hi = lo + per < n ? lo + per : n;
    constexpr int U = 4;
    for (long long i = lo + threadIdx.x; i < hi; i += 256 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long j = i + (long long)u * 256;
            if (j < hi) v[u] = ld_nt(src + j);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long j = i + (long long)u * 256;
            if (j < hi) st_nt(v[u], dst + j);
        }
    }
}

#ifndef MOONEP_REDUCE_U
#define MOONEP_REDUCE_U 4
#endif

__global__ __launch_bounds__(256) void reduce_grad_kernel(PlanWs w, float4* __restrict__ d13,
                                                          float4* __restrict__ d2,
                                                          float4* __restrict__ r13,
                                                          float4* __restrict__ r2, long long n13,
                                                          long long n2) {
    const int e = blockIdx.y;
    const int nred = min(w.red_n[e], kMaxR);
    if (nred <= 0) return;
    const bool first = blockIdx.z == 0;
    const long long n = first ? n13 : n2;
    float4* home = (first ? d13 : d2) + (size_t)e * n;
    float4* red = first ? r13 : r2;
    const int32_t* slots = w.red_slot + (size_t)e * kMaxR;
    const long long per = (n + kCopyBlocks - 1) / kCopyBlocks;
    const long long lo = per * blockIdx.x;
    const long long hi = lo + per < n ? lo + per : n;
    // U vectors per thread per pass, all loads of a replica issued before its adds (replicas are
    // added in creation order, so every element sees the same sequence of float32 additions)
    constexpr int U = MOONEP_REDUCE_U;
    for (long long i0 = lo + threadIdx.x; i0 < hi; i0 += 256 * U) {
        float4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * 256 < hi) a[u] = home[i0 + u * 256];
        for (int r = 0; r < nred; ++r) {
            const int sl = slots[r];
            if (sl < 0 || sl >= w.R * w.B) continue;
            float4* rb = red + (size_t)sl * n + i0;
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (i0 + u * 256 < hi) v[u] = ld_nt(rb + u * 256);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (i0 + u * 256 >= hi) continue;
                a[u].x += v[u].x;
                a[u].y += v[u].y;
                a[u].z += v[u].z;
                a[u].w += v[u].w;
                st_nt(make_float4(0.f, 0.f, 0.f, 0.f), rb + u * 256);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * 256 < hi) home[i0 + u * 256] = a[u];
    }
}

}  // namespace moonep

using namespace moonep;

extern "C" int moonep_prefetch(const moonep_dims_t* dims, const void* plan_ws, const void* w13_home,
                               const void* w2_home, void* w13_slot, void* w2_slot, void* stream) {
    const int rc = check_dims(dims, true);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(plan_ws);
    MOONEP_CHECK_PTR(w13_home);
    MOONEP_CHECK_PTR(w2_home);
    if (dims->B == 0) return MOONEP_OK;
    MOONEP_CHECK_PTR(w13_slot);
    MOONEP_CHECK_PTR(w2_slot);
    PlanWs w;
    plan_ws_layout(dims, const_cast<void*>(plan_ws), &w);
    const long long n13 = (long long)dims->H * 2 * dims->I * 2 / 16;
    const long long n2 = (long long)dims->I * dims->H * 2 / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(prefetch_kernel, dim3(kCopyBlocks, dims->R * dims->B, 2), dim3(256), 0, s, w,
                       static_cast<const uint4*>(w13_home), static_cast<const uint4*>(w2_home),
                       static_cast<uint4*>(w13_slot), static_cast<uint4*>(w2_slot), n13, n2);
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}

extern "C" int moonep_reduce_grad(const moonep_dims_t* dims, const void* plan_ws, float* dw13_home,
                                  float* dw2_home, float* dw13_red, float* dw2_red, void* stream) {
    const int rc = check_dims(dims, true);
    if (rc != MOONEP_OK) return rc;
    MOONEP_CHECK_PTR(plan_ws);
    MOONEP_CHECK_PTR(dw13_home);
    MOONEP_CHECK_PTR(dw2_home);
    if (dims->B == 0) return MOONEP_OK;
    MOONEP_CHECK_PTR(dw13_red);
    MOONEP_CHECK_PTR(dw2_red);
    PlanWs w;
    plan_ws_layout(dims, const_cast<void*>(plan_ws), &w);
    const long long n13 = (long long)dims->H * 2 * dims->I / 4;
    const long long n2 = (long long)dims->I * dims->H / 4;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(reduce_grad_kernel, dim3(kCopyBlocks, dims->E, 2), dim3(256), 0, s, w,
                       reinterpret_cast<float4*>(dw13_home), reinterpret_cast<float4*>(dw2_home),
                       reinterpret_cast<float4*>(dw13_red), reinterpret_cast<float4*>(dw2_red), n13, n2);
    MOONEP_LAUNCH_CHECK();
    return MOONEP_OK;
}
