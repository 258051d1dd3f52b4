// Between stacked MoE layers: residual add and weightless RMSNorm.  The pages
// describe a single MoE layer; this pre-norm residual form is the reading used
// to chain layers (x <- x + MoE(rmsnorm(x))).  One workgroup per token; rows
// of aligned float4s hold the row in registers between the sum and the scale.
#include "common.h"

namespace moedec {

namespace {

constexpr int kNormThreads = 256;

__device__ __forceinline__ float block_sum(float ss) {
    __shared__ float red[kNormThreads / kWave];
    ss = group_sum<kWave>(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Rows of 16-byte-aligned float4s: each thread issues all of its loads (NV
// float4 of x, and of y) before using any, so a row costs one memory latency.
template <int NV>
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_vec(float* __restrict__ x, const float* __restrict__ y,
                                                                     float* __restrict__ xn, int H, float eps) {
    const int t = blockIdx.x, n4 = H >> 2;
    float4* xt = reinterpret_cast<float4*>(x + (size_t)t * H);
    const float4* yt = y ? reinterpret_cast<const float4*>(y + (size_t)t * H) : nullptr;
    float4 v[NV], u[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = xt[min((int)threadIdx.x + k * kNormThreads, n4 - 1)];
    if (yt) {
#pragma unroll
        for (int k = 0; k < NV; ++k) u[k] = yt[min((int)threadIdx.x + k * kNormThreads, n4 - 1)];
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = threadIdx.x + k * kNormThreads;
        if (yt) {
            v[k].x += u[k].x;
            v[k].y += u[k].y;
            v[k].z += u[k].z;
            v[k].w += u[k].w;
            if (i < n4) xt[i] = v[k];
        }
        if (i < n4) ss += (v[k].x * v[k].x + v[k].y * v[k].y) + (v[k].z * v[k].z + v[k].w * v[k].w);
    }
    const float inv = 1.0f / sqrtf(block_sum(ss) / (float)H + eps);
    float4* xo = reinterpret_cast<float4*>(xn + (size_t)t * H);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = threadIdx.x + k * kNormThreads;
        if (i < n4) xo[i] = make_float4(v[k].x * inv, v[k].y * inv, v[k].z * inv, v[k].w * inv);
    }
}

// Any row length or alignment.
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(float* __restrict__ x,
                                                                        const float* __restrict__ y,
                                                                        float* __restrict__ xn, int H, float eps) {
    const int t = blockIdx.x;
    float* xt = x + (size_t)t * H;
    const float* yt = y ? y + (size_t)t * H : nullptr;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += kNormThreads) {
        float v = xt[i];
        if (yt) {
            v += yt[i];
            xt[i] = v;
        }
        ss += v * v;
    }
    const float inv = 1.0f / sqrtf(block_sum(ss) / (float)H + eps);
    for (int i = threadIdx.x; i < H; i += kNormThreads) xn[(size_t)t * H + i] = xt[i] * inv;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_residual_rmsnorm(float* x, const float* y, float* xn, int T, int H, float eps, hipStream_t st) {
    const int per = (H / 4 + kNormThreads - 1) / kNormThreads;
    const bool vec = H % 4 == 0 && aligned16(x) && aligned16(xn) && (!y || aligned16(y)) && per <= 16;
    if (!vec)
        hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3(T), dim3(kNormThreads), 0, st, x, y, xn, H, eps);
    else if (per <= 2)
        hipLaunchKernelGGL(residual_rmsnorm_vec<2>, dim3(T), dim3(kNormThreads), 0, st, x, y, xn, H, eps);
    else if (per <= 4)
        hipLaunchKernelGGL(residual_rmsnorm_vec<4>, dim3(T), dim3(kNormThreads), 0, st, x, y, xn, H, eps);
    else if (per <= 8)
        hipLaunchKernelGGL(residual_rmsnorm_vec<8>, dim3(T), dim3(kNormThreads), 0, st, x, y, xn, H, eps);
    else
        hipLaunchKernelGGL(residual_rmsnorm_vec<16>, dim3(T), dim3(kNormThreads), 0, st, x, y, xn, H, eps);
    return hipGetLastError();
}

}  // namespace moedec
