// Integer matrix-core building blocks of the fused layer kernel: codes as
// int8 A operands, activations as an int8 hi/lo pair, dot products on
// v_mfma_i32_16x16x64_i8 in exact 32-bit integer arithmetic.
//
// Codes are dequantised on use (Show HN page "धीमे कंप्यूटर पर GLM 5.2
// चलाना", section "implemented features": int8, packed int4, packed int2 with
// one scale per row).  A b-bit two's-complement field moved to the top of a
// byte IS the signed byte 2^(8-b) * q, so one shift and one AND per 32-bit
// word turn four packed fields into four int8 operands, with no offset to
// correct: every product carries the exact factor 2^(8-b), folded into the
// final power-of-two unscale.  int8 codes are used as loaded.
//
// Activations: each token (column) gets its own power-of-two scale 2^e with
// max|x| * 2^e <= 32512; x * 2^e is rounded to the integer v = 256 * hi + lo
// with hi in [-127, 127] and lo in [-128, 127], and a product is two MFMAs
// (hi and lo) into separate int32 accumulators.  Sums of products of codes and
// hi or lo stay far below 2^31 for rows up to MOEDEC_MAX_DIM long, so the
// whole dot product is exact given v; the only rounding of the matrix
// product is that of x to 16 significant bits relative to its column's
// largest magnitude.
//
// MFMA operands: lane l supplies row l % 16 (A) or column l % 16 (B) and 16
// byte slots for K; the MFMA pairs slot s of lane group l / 16 in A with the
// same slot and group in B, so only the slot <-> column map has to agree
// between codes and staged activations.  A lane's 16-byte load of a code row
// (CW = 128 / b columns) becomes NM = 8 / b operands; operand m, slot s holds
// column col(m, s) of the group.
#pragma once

#include "common.h"

namespace moedec {
namespace imma {

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int BITS>
struct I8Codec;

template <>
struct I8Codec<4> {
    static constexpr int NM = 2, CW = 32, kShift = 4;
    // dword d of the load holds columns 8d .. 8d+7 (nibble n = column 8d + n);
    // operand 0 takes the even nibbles, operand 1 the odd ones
    __device__ static int col(int m, int s) { return 8 * (s >> 2) + 2 * (s & 3) + m; }
    __device__ static void place(int p, int& m, int& s) {
        m = p & 1;
        s = 4 * (p >> 3) + ((p >> 1) & 3);
    }
    __device__ static uint32_t field(uint32_t w, int m) { return (m == 0 ? w << 4 : w) & 0xF0F0F0F0u; }
};

template <>
struct I8Codec<8> {
    static constexpr int NM = 1, CW = 16, kShift = 0;
    __device__ static int col(int, int s) { return s; }
    __device__ static void place(int p, int& m, int& s) {
        m = 0;
        s = p;
    }
    __device__ static uint32_t field(uint32_t w, int) { return w; }
};

template <>
struct I8Codec<2> {
    static constexpr int NM = 4, CW = 64, kShift = 6;
    // dword d holds columns 16d .. 16d+15 (field f at bits 2f); operand m
    // takes fields m, m+4, m+8, m+12, each moved to the top of its byte
    __device__ static int col(int m, int s) { return 16 * (s >> 2) + 4 * (s & 3) + m; }
    __device__ static void place(int p, int& m, int& s) {
        m = p & 3;
        s = 4 * (p >> 4) + ((p >> 2) & 3);
    }
    __device__ static uint32_t field(uint32_t w, int m) { return (w << (6 - 2 * m)) & 0xC0C0C0C0u; }
};

// Operand m of a lane's 16-byte code load.
template <int BITS>
__device__ __forceinline__ i32x4 operand(const uint4& q, int m) {
    using C = I8Codec<BITS>;
    return i32x4{(int)C::field(q.x, m), (int)C::field(q.y, m), (int)C::field(q.z, m), (int)C::field(q.w, m)};
}

__device__ __forceinline__ i32x4 mma(const i32x4& a, const i32x4& b, const i32x4& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// The value of a hi/lo pair of accumulators in fp32 (exact while |hi| < 2^16).
__device__ __forceinline__ float combine(int hi, int lo) { return (float)hi * 256.0f + (float)lo; }

// Largest power-of-two exponent e with m * 2^e <= 32512 (0 for m = 0 or a
// non-finite m, whose column then holds garbage either way).
__device__ __forceinline__ int q16_exponent(float m) {
    if (!(m > 0.f) || !isfinite(m)) return 0;
    int e;
    frexpf(m, &e);                      // m in [2^(e-1), 2^e)
    int k = 15 - e;                     // m * 2^k in [2^14, 2^15)
    if (ldexpf(m, k) > 32512.f) --k;
    return k > 100 ? 100 : k < -100 ? -100 : k;
}

// x * 2^e (already scaled) -> (hi, lo) bytes of its rounded 16-bit value.
__device__ __forceinline__ void split16(float xs, int& hi, int& lo) {
    const float r = fminf(fmaxf(rintf(xs), -32512.f), 32512.f);
    const int v = (int)r;
    hi = (v + 128) >> 8;
    lo = v - (hi << 8);
}

// Bytes (as stored in LDS) of one staged activation row of `cols` columns:
// hi and lo, every 16-byte group of codes padded to whole 4-group chunks.
template <int BITS>
__host__ __device__ constexpr size_t staged_row_bytes_i8(int cols) {
    return (size_t)((cols / (128 / BITS) + 3) / 4) * 4 * (8 / BITS) * 16 * 2;
}

}  // namespace imma
}  // namespace moedec
