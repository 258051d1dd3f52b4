// Shared pieces of the persistent-workgroup kernels (the split expert
// kernels and the fused layer kernel): workgroup shape, LDS budget, vector
// types, the device-scope store used before a grid exchange, and the host
// helpers that size a launch to the device.
#pragma once

#include "common.h"

namespace moedec {
namespace mfma {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMT = 512;                 // threads of a persistent workgroup
constexpr int kMW = kMT / kWave;         // its waves
constexpr int kNBMax = 5;                // 16-row blocks per gate/up group at most
constexpr int kNBD = 2;                  // 16-row blocks per down workgroup at most
constexpr int kCols = 16;                // MFMA N: tokens per segment at most
constexpr int kMaxActive = MOEDEC_MAX_EXPERTS + 8;
constexpr size_t kLdsMax = 160 * 1024;
constexpr size_t kStatic = 16 * 1024;    // static LDS of these kernels, rounded up

// Largest j in [0, n) with v[j] <= q (v ascending, v[0] <= q).
__device__ __forceinline__ int mw_upper_index(const int* v, int n, int q) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (v[mid] <= q) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// A store that other workgroups of the same launch read after a grid barrier:
// device scope, so it goes through to the device-coherent level at once and
// the barrier needs no cache write-back.
__device__ __forceinline__ void store_device(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------- host side

// Compute units of the current device (cached per device).
inline int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Dynamic LDS a persistent workgroup asks for at least, so that no two of them
// share a compute unit.
constexpr size_t kLdsOnePerCu = 84 * 1024;

template <typename Kern>
hipError_t allow_lds(Kern k, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

}  // namespace mfma
}  // namespace moedec
