// Router: sigmoid scores, noaux_tc-corrected group-limited top-k, weights, and
// the batch union (worklist) of the selected experts.
//
// Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
// DeepSeek-V3-style sigmoid router with noaux_tc correction,
// routed_scaling_factor and a shared expert; batch-union MoE.  The
// group-score rule (top-2 sum), the use of the corrected score for selection
// only and the tie-breaking (lower index) are this library's reading.
//
// Kernel 1 (router_gemv): one workgroup per expert row; every thread issues all
// of its 16-byte loads of the row before using them, then the row is dotted
// with the tokens, four at a time with their loads issued together, and
// s = sigmoid(W_r[e] . x_t) is written.
// Kernel 2 (route_select): one workgroup running route_select_block (see
// route.h): each wave routes its tokens with wave-wide arg-max rounds, then
// the expert-ascending worklist comes from a rank sort in LDS.
#include "route.h"

namespace moedec {

namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvMaxF4 = MOEDEC_MAX_DIM / 4 / kGemvThreads;   // float4 per thread at most
constexpr int kGemvTB = 4;                                        // tokens whose x loads go out together
constexpr int kSelThreads = 512;                                   // 8 waves (1024 would spill)

// NF float4 of the row per thread; tokens in batches of kGemvTB whose x loads
// all go out before any is used (the row's loads went out first of all).
template <int NF>
__global__ __launch_bounds__(kGemvThreads) void router_gemv_kernel(const float* __restrict__ x,
                                                                   const float* __restrict__ W, int T, int H,
                                                                   int E, float* __restrict__ scores) {
    __shared__ float red[MOEDEC_MAX_TOKENS][kGemvThreads / kWave];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const float4* w4 = reinterpret_cast<const float4*>(W + (size_t)e * H);
    const int n4 = H >> 2;
    float4 wr[NF];
#pragma unroll
    for (int k = 0; k < NF; ++k) wr[k] = w4[min((int)threadIdx.x + k * kGemvThreads, n4 - 1)];
#pragma unroll
    for (int k = 0; k < NF; ++k)          // columns past the row's end count as zero
        if ((int)threadIdx.x + k * kGemvThreads >= n4) wr[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t0 = 0; t0 < T; t0 += kGemvTB) {
        float4 xv[kGemvTB][NF];
#pragma unroll
        for (int b = 0; b < kGemvTB; ++b) {
            const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)min(t0 + b, T - 1) * H);
#pragma unroll
            for (int k = 0; k < NF; ++k) xv[b][k] = x4[min((int)threadIdx.x + k * kGemvThreads, n4 - 1)];
        }
#pragma unroll
        for (int b = 0; b < kGemvTB; ++b) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < NF; ++k)
                acc += (wr[k].x * xv[b][k].x + wr[k].y * xv[b][k].y) + (wr[k].z * xv[b][k].z + wr[k].w * xv[b][k].w);
            acc = group_sum<kWave>(acc);
            if (lane == 0 && t0 + b < T) red[t0 + b][wave] = acc;
        }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < T; t += kGemvThreads) {
        const float z = (red[t][0] + red[t][1]) + (red[t][2] + red[t][3]);
        scores[(size_t)t * E + e] = 1.0f / (1.0f + expf(-z));
    }
}

template <bool kTopP>
__global__ __launch_bounds__(kSelThreads) void route_select_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int T, int E, int n_group, int topk_group,
    int top_k, int n_shared, float rsf, float top_p, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ wl_n_active, int32_t* __restrict__ wl_expert_id, int32_t* __restrict__ wl_seg,
    int32_t* __restrict__ wl_assign) {
    __shared__ RouteLdsT<MOEDEC_MAX_TOKENS, MOEDEC_MAX_EXPERTS, kSelThreads / kWave> r;
    route_select_block<MOEDEC_MAX_TOKENS, MOEDEC_MAX_EXPERTS, kSelThreads / kWave, false, kTopP>(
        scores, bias, T, E, n_group, topk_group, top_k, n_shared, rsf, top_p, r);
    // outputs
    for (int i = threadIdx.x; i < T * top_k; i += blockDim.x) {
        topk_idx[i] = r.sel[i];
        topk_w[i] = r.selw[i];
    }
    if (wl_n_active == nullptr) return;
    const int n = r.n_active;
    const int A = r.n_assign;                          // = seg[n]
    if (threadIdx.x == 0) *wl_n_active = n;
    for (int j = threadIdx.x; j <= n; j += blockDim.x) {
        if (j < n) wl_expert_id[j] = r.eid[j];
        wl_seg[j] = r.seg[j];
    }
    for (int a = threadIdx.x; a < A; a += blockDim.x) wl_assign[a] = r.assign[a];
}

}  // namespace

hipError_t launch_route(const float* x, const float* router_w, const float* bias, int T, int H, int E,
                        int n_group, int topk_group, int top_k, int n_shared, float rsf, float top_p,
                        float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                        hipStream_t st) {
    const int per = (H / 4 + kGemvThreads - 1) / kGemvThreads;
    if (per <= 2)
        hipLaunchKernelGGL(router_gemv_kernel<2>, dim3(E), dim3(kGemvThreads), 0, st, x, router_w, T, H, E, scores);
    else if (per <= 4)
        hipLaunchKernelGGL(router_gemv_kernel<4>, dim3(E), dim3(kGemvThreads), 0, st, x, router_w, T, H, E, scores);
    else if (per <= 6)
        hipLaunchKernelGGL(router_gemv_kernel<6>, dim3(E), dim3(kGemvThreads), 0, st, x, router_w, T, H, E, scores);
    else if (per <= 8)
        hipLaunchKernelGGL(router_gemv_kernel<8>, dim3(E), dim3(kGemvThreads), 0, st, x, router_w, T, H, E, scores);
    else
        hipLaunchKernelGGL(router_gemv_kernel<kGemvMaxF4>, dim3(E), dim3(kGemvThreads), 0, st, x, router_w, T, H, E,
                           scores);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    auto k = top_p < 1.f ? route_select_kernel<true> : route_select_kernel<false>;
    hipLaunchKernelGGL(k, dim3(1), dim3(kSelThreads), 0, st, scores, bias, T, E, n_group,
                       topk_group, top_k, n_shared, rsf, top_p, topk_idx, topk_w, wl ? wl->n_active : nullptr,
                       wl ? wl->expert_id : nullptr, wl ? wl->seg : nullptr, wl ? wl->assign : nullptr);
    return hipGetLastError();
}

}  // namespace moedec
