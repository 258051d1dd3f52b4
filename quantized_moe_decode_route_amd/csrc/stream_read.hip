// A plain 128-bit streaming read (measurement aid): the achievable HBM read
// rate that the weight streams of the MoE kernels are compared against.  Each
// workgroup reads one contiguous stretch of the buffer; its threads read
// consecutive 16-byte words (a wave covers 1 KB per load), U loads in flight
// per thread before any is used.
#include "common.h"
#include "moedec_bench.h"

#define MOEDEC_API extern "C" __attribute__((visibility("default")))

namespace moedec {
namespace {

constexpr uint32_t kNever = 0x9E3779B9u;   // a fold value the sink records (practically never)

template <int U>
__global__ void stream_read_kernel(const uint4* __restrict__ p, int64_t n16, int64_t per_wg,
                                   uint32_t* __restrict__ sink) {
    const int64_t b0 = (int64_t)blockIdx.x * per_wg;
    const int64_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
    const int64_t step = (int64_t)blockDim.x * U;
    uint32_t acc = 0;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += step) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = i + (int64_t)u * blockDim.x;
            v[u] = k < b1 ? p[k] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == kNever) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace
}  // namespace moedec

MOEDEC_API int moe_bench_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int grid, int threads,
                                     int unroll, void* stream) {
    using namespace moedec;
    if (!buf || !sink || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15)) return MOEDEC_ERR_INVALID_ARG;
    if (grid < 1 || grid > 65536 || (threads != 256 && threads != 512 && threads != 1024)) return MOEDEC_ERR_INVALID_ARG;
    const int64_t n16 = bytes / 16;
    const int64_t per_wg = (n16 + grid - 1) / grid;
    const uint4* p = static_cast<const uint4*>(buf);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (unroll) {
        case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(threads), 0, st, p, n16, per_wg, sink); break;
        case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(threads), 0, st, p, n16, per_wg, sink); break;
        case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(grid), dim3(threads), 0, st, p, n16, per_wg, sink); break;
        default: return MOEDEC_ERR_INVALID_ARG;
    }
    return hipGetLastError() == hipSuccess ? MOEDEC_OK : MOEDEC_ERR_DEVICE;
}
