// Between stacked MoE layers: residual add and weightless RMSNorm.  The pages
// describe a single MoE layer; this pre-norm residual form is the reading used
// to chain layers (x <- x + MoE(rmsnorm(x))).  One workgroup per token.
#include "common.h"

namespace moedec {

namespace {

constexpr int kNormThreads = 256;

__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(float* __restrict__ x,
                                                                        const float* __restrict__ y,
                                                                        float* __restrict__ xn, int H, float eps) {
    __shared__ float red[kNormThreads / kWave];
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
    ss = group_sum<kWave>(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
    for (int i = threadIdx.x; i < H; i += kNormThreads) xn[(size_t)t * H + i] = xt[i] * inv;
}

}  // namespace

hipError_t launch_residual_rmsnorm(float* x, const float* y, float* xn, int T, int H, float eps, hipStream_t st) {
    hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3(T), dim3(kNormThreads), 0, st, x, y, xn, H, eps);
    return hipGetLastError();
}

}  // namespace moedec
