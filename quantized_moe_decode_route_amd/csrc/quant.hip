// Row quantiser: fp32 weight rows -> int8 / int4 / int2 codes with one fp32
// scale per row, as codes (one per byte) or already packed.
//
// Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
// the converter dequantises the block-scaled checkpoint and requantises it into
// the engine's container, whose kernels keep one scale per weight row.  The
// pages give no rule; the one used here: s = absmax(row) / qmax (qmax = 127,
// 7, 1), code = rint(w / s) (ties to even) clamped to the field, a zero row
// (or one whose s rounds to zero) gets s = 0 and codes 0, and a row holding a
// NaN or an infinity gets s = NaN and codes 0.  Every step is IEEE fp32 (the
// division correctly rounded), so codes and scales are fully determined.
//
// HBM-bound (4 bytes read per weight, 1 or less written): one, two or four
// waves per row (by row length), float4 loads that cover 1 KB per wave instruction and
// bypass the caches (each byte is read once), the row held in registers
// between the absmax and the quantise pass for rows up to 8192 columns
// (longer rows are read twice), codes from a multiply by 1/s that falls back
// to the division only near a rounding boundary.
#include "common.h"

namespace moedec {

namespace {

constexpr int kQThreads = 256;         // 4 waves per workgroup
constexpr int kQWaves = kQThreads / kWave;
constexpr float kFltMax = 3.402823466e38f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int BITS>
struct QField {
    static constexpr int qmax = (1 << (BITS - 1)) - 1, qmin = -(1 << (BITS - 1));
};

// The four codes of v given the row scale s > 0 and inv = 1/s.  The quotient
// that decides a code is the correctly rounded x / s; x * inv lies within
// 2^-23 |x / s| of the exact quotient (two roundings), so rint of the product
// equals rint of the rounded quotient unless the product sits within that
// distance of a half-way point: only then (or when inv overflows, fast =
// false) is the division done.
template <int BITS>
__device__ __forceinline__ void codes4(const f32x4& v, float s, float inv, bool fast, int* c) {
    float q[4] = {v.x, v.y, v.z, v.w};
    bool exact = !fast;
    if (fast) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float y = q[k] * inv;
            const float r = rintf(y);
            exact = exact || fabsf(fabsf(y - r) - 0.5f) <= fabsf(y) * 0x1p-21f;
            q[k] = r;
        }
    }
    if (exact) {
        q[0] = rintf(v.x / s);
        q[1] = rintf(v.y / s);
        q[2] = rintf(v.z / s);
        q[3] = rintf(v.w / s);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = (int)fminf(fmaxf(q[k], (float)QField<BITS>::qmin), (float)QField<BITS>::qmax);
}

// Stores the codes of float4 j of row r (zero when s is 0 or NaN).  PACK:
// 8/BITS codes per byte, the lowest column in the lowest bits.
template <int BITS, bool PACK>
__device__ __forceinline__ void store4(void* out, int64_t r, int64_t n4, int64_t j, const f32x4& v, float s,
                                       float inv, bool ok, bool fast) {
    int c[4] = {0, 0, 0, 0};
    if (ok) codes4<BITS>(v, s, inv, fast, c);
    if (!PACK || BITS == 8) {
        const uint32_t d = (uint32_t)(c[0] & 0xFF) | (uint32_t)(c[1] & 0xFF) << 8 | (uint32_t)(c[2] & 0xFF) << 16 |
                           (uint32_t)(c[3] & 0xFF) << 24;
        reinterpret_cast<uint32_t*>(out)[r * n4 + j] = d;
    } else if (BITS == 4) {
        const uint32_t d = (uint32_t)(c[0] & 0xF) | (uint32_t)(c[1] & 0xF) << 4 | (uint32_t)(c[2] & 0xF) << 8 |
                           (uint32_t)(c[3] & 0xF) << 12;
        reinterpret_cast<uint16_t*>(out)[r * n4 + j] = (uint16_t)d;
    } else {
        const uint32_t d = (uint32_t)(c[0] & 3) | (uint32_t)(c[1] & 3) << 2 | (uint32_t)(c[2] & 3) << 4 |
                           (uint32_t)(c[3] & 3) << 6;
        reinterpret_cast<uint8_t*>(out)[r * n4 + j] = (uint8_t)d;
    }
}

__device__ __forceinline__ void absmax4(const f32x4& v, float& amax, bool& bad) {
    const float a = fabsf(v.x), b = fabsf(v.y), c = fabsf(v.z), d = fabsf(v.w);
    // a NaN fails every comparison, an infinity fails <= FLT_MAX
    bad = bad || !(a <= kFltMax) || !(b <= kFltMax) || !(c <= kFltMax) || !(d <= kFltMax);
    amax = fmaxf(amax, fmaxf(fmaxf(a, b), fmaxf(c, d)));
}

// Row scale from every lane's partial absmax and non-finite flag, reduced
// over the wave, then over the WPR waves of the row through LDS.  ok = codes
// are to be computed (s finite and nonzero); fast = 1/s is finite.
template <int BITS, int WPR>
__device__ __forceinline__ float row_scale(float amax, bool bad, float& inv, bool& ok, bool& fast) {
    const unsigned m = wave_max_u(__float_as_uint(amax));     // amax >= +0: bit order = value order
    const bool b = __ballot(bad) != 0;
    unsigned mm = m;
    bool any_bad = b;
    if (WPR > 1) {
        __shared__ unsigned wmax[kQWaves];
        __shared__ int wbad[kQWaves];
        const int wave = threadIdx.x / kWave, w0 = wave - wave % WPR;
        if ((threadIdx.x & (kWave - 1)) == 0) {
            wmax[wave] = m;
            wbad[wave] = b;
        }
        __syncthreads();
        mm = wmax[w0];
        any_bad = wbad[w0] != 0;
#pragma unroll
        for (int k = 1; k < WPR; ++k) {
            mm = max(mm, wmax[w0 + k]);
            any_bad = any_bad || wbad[w0 + k] != 0;
        }
    }
    const float s = any_bad ? __uint_as_float(0x7FC00000u) : __uint_as_float(mm) / (float)QField<BITS>::qmax;
    ok = !any_bad && s != 0.f;
    inv = 1.0f / s;
    fast = inv <= kFltMax;
    return s;
}

// WPR waves per row (4 / WPR rows per workgroup), NC float4 per thread held
// in registers: rows of up to 256 * WPR * NC columns.
template <int BITS, bool PACK, int WPR, int NC>
__global__ __launch_bounds__(kQThreads) void quantize_rows_cached(const float* __restrict__ w, void* __restrict__ out,
                                                                   float* __restrict__ scales, int64_t rows,
                                                                   int64_t n4) {
    constexpr int kRowThreads = WPR * kWave;
    const int t = threadIdx.x % kRowThreads;
    const int64_t r = (int64_t)blockIdx.x * (kQWaves / WPR) + threadIdx.x / kRowThreads;
    const bool live = r < rows;                              // the last workgroup's spare waves still reduce
    const f32x4* row = reinterpret_cast<const f32x4*>(w) + (live ? r : rows - 1) * n4;
    f32x4 v[NC];
    float amax = 0.f;
    bool bad = false;
    if (n4 > 0) {
        // every load issued before any is used; a thread past the row's end
        // reloads the last float4 (in bounds) and ignores it
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t j = t + (int64_t)i * kRowThreads;
            v[i] = __builtin_nontemporal_load(row + (j < n4 ? j : n4 - 1));
        }
#pragma unroll
        for (int i = 0; i < NC; ++i)
            if (t + (int64_t)i * kRowThreads < n4) absmax4(v[i], amax, bad);
    }
    float inv;
    bool ok, fast;
    const float s = row_scale<BITS, WPR>(amax, bad, inv, ok, fast);
    if (!live) return;
    if (t == 0) scales[r] = s;                               // NaN, 0 or absmax / qmax
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int64_t j = t + (int64_t)i * kRowThreads;
        if (j < n4) store4<BITS, PACK>(out, r, n4, j, v[i], s, inv, ok, fast);
    }
}

// Rows too long for the registers (one row per workgroup): an absmax pass,
// then a second read.
template <int BITS, bool PACK>
__global__ __launch_bounds__(kQThreads) void quantize_rows_long(const float* __restrict__ w, void* __restrict__ out,
                                                                float* __restrict__ scales, int64_t n4) {
    const int64_t r = blockIdx.x;
    const f32x4* row = reinterpret_cast<const f32x4*>(w) + r * n4;
    float amax = 0.f;
    bool bad = false;
    for (int64_t j = threadIdx.x; j < n4; j += kQThreads) absmax4(row[j], amax, bad);
    float inv;
    bool ok, fast;
    const float s = row_scale<BITS, kQWaves>(amax, bad, inv, ok, fast);
    if (threadIdx.x == 0) scales[r] = s;
    for (int64_t j = threadIdx.x; j < n4; j += kQThreads) store4<BITS, PACK>(out, r, n4, j, row[j], s, inv, ok, fast);
}

template <int BITS, bool PACK, int WPR, int NC>
void launch_cached(const float* w, void* out, float* scales, int64_t rows, int64_t n4, hipStream_t st) {
    constexpr int rpb = kQWaves / WPR;
    hipLaunchKernelGGL((quantize_rows_cached<BITS, PACK, WPR, NC>), dim3((unsigned)((rows + rpb - 1) / rpb)),
                       dim3(kQThreads), 0, st, w, out, scales, rows, n4);
}

// Waves per row: one while a row fits 8 float4 per lane (<= 2048 columns),
// else two or four, so each thread holds 1-8 float4 and the row stays in
// registers up to 8192 columns.
template <int BITS, bool PACK>
hipError_t launch_bits(const float* w, void* out, float* scales, int64_t rows, int64_t row_len, hipStream_t st) {
    const int64_t n4 = row_len / 4;
    if (n4 <= 64) launch_cached<BITS, PACK, 1, 1>(w, out, scales, rows, n4, st);
    else if (n4 <= 128) launch_cached<BITS, PACK, 1, 2>(w, out, scales, rows, n4, st);
    else if (n4 <= 256) launch_cached<BITS, PACK, 1, 4>(w, out, scales, rows, n4, st);
    else if (n4 <= 512) launch_cached<BITS, PACK, 1, 8>(w, out, scales, rows, n4, st);
    else if (n4 <= 768) launch_cached<BITS, PACK, 2, 6>(w, out, scales, rows, n4, st);
    else if (n4 <= 1024) launch_cached<BITS, PACK, 2, 8>(w, out, scales, rows, n4, st);
    else if (n4 <= 1536) launch_cached<BITS, PACK, 4, 6>(w, out, scales, rows, n4, st);
    else if (n4 <= 2048) launch_cached<BITS, PACK, 4, 8>(w, out, scales, rows, n4, st);
    else
        hipLaunchKernelGGL((quantize_rows_long<BITS, PACK>), dim3((unsigned)rows), dim3(kQThreads), 0, st, w, out,
                           scales, n4);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(int bits, bool pack, const float* w, void* out, float* scales, int64_t rows,
                                int64_t row_len, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    switch (bits * 2 + (pack ? 1 : 0)) {
        case 16: return launch_bits<8, false>(w, out, scales, rows, row_len, st);
        case 17: return launch_bits<8, true>(w, out, scales, rows, row_len, st);
        case 8: return launch_bits<4, false>(w, out, scales, rows, row_len, st);
        case 9: return launch_bits<4, true>(w, out, scales, rows, row_len, st);
        case 4: return launch_bits<2, false>(w, out, scales, rows, row_len, st);
        case 5: return launch_bits<2, true>(w, out, scales, rows, row_len, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moedec
