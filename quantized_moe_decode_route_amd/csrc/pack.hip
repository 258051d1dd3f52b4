// Packing of int8 / int4 / int2 codes into bytes and back.
//
// ideipro.ru article "Энтузиаст запустил GLM-5.2 на ноутбуке с 25 ГБ RAM": the
// packed formats were checked bit for bit; Show HN page "धीमे कंप्यूटर पर GLM
// 5.2 चलाना", section "implemented features": int8, packed int4, packed int2.
// Field j of byte k holds column k*(8/bits)+j in bits j*bits.., two's complement.
// One thread per output byte (pack) or input byte (unpack); grid-stride.
#include "common.h"

namespace moedec {

namespace {

template <int BITS>
__global__ void pack_kernel(const int8_t* __restrict__ codes, uint8_t* __restrict__ packed, int64_t n_bytes) {
    constexpr int F = 8 / BITS;
    constexpr uint32_t M = (1u << BITS) - 1u;
    for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < n_bytes;
         b += (int64_t)gridDim.x * blockDim.x) {
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < F; ++j) v |= ((uint32_t)(uint8_t)codes[b * F + j] & M) << (j * BITS);
        packed[b] = (uint8_t)v;
    }
}

template <int BITS>
__global__ void unpack_kernel(const uint8_t* __restrict__ packed, int8_t* __restrict__ codes, int64_t n_bytes) {
    constexpr int F = 8 / BITS;
    for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < n_bytes;
         b += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t v = packed[b];
#pragma unroll
        for (int j = 0; j < F; ++j) {
            // move field j to the top of a 32-bit word, then arithmetic-shift it down
            const int32_t f = (int32_t)(v << (32 - BITS - j * BITS)) >> (32 - BITS);
            codes[b * F + j] = (int8_t)f;
        }
    }
}

dim3 grid_for(int64_t n) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return dim3((unsigned)blocks);
}

}  // namespace

hipError_t launch_pack(int bits, const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len,
                       hipStream_t st) {
    const int64_t n_bytes = rows * (row_len * bits / 8);
    if (n_bytes == 0) return hipSuccess;
    switch (bits) {
        case 8: hipLaunchKernelGGL(pack_kernel<8>, grid_for(n_bytes), dim3(256), 0, st, codes, packed, n_bytes); break;
        case 4: hipLaunchKernelGGL(pack_kernel<4>, grid_for(n_bytes), dim3(256), 0, st, codes, packed, n_bytes); break;
        case 2: hipLaunchKernelGGL(pack_kernel<2>, grid_for(n_bytes), dim3(256), 0, st, codes, packed, n_bytes); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_unpack(int bits, const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len,
                         hipStream_t st) {
    const int64_t n_bytes = rows * (row_len * bits / 8);
    if (n_bytes == 0) return hipSuccess;
    switch (bits) {
        case 8: hipLaunchKernelGGL(unpack_kernel<8>, grid_for(n_bytes), dim3(256), 0, st, packed, codes, n_bytes); break;
        case 4: hipLaunchKernelGGL(unpack_kernel<4>, grid_for(n_bytes), dim3(256), 0, st, packed, codes, n_bytes); break;
        case 2: hipLaunchKernelGGL(unpack_kernel<2>, grid_for(n_bytes), dim3(256), 0, st, packed, codes, n_bytes); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moedec
