// Device helpers and internal launch interfaces of libmoedec (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moedec.h"   // include/ is on the include path

namespace moedec {

constexpr int kWave = 64;

// ----------------------------------------------------------------- reductions

__device__ __forceinline__ float bits_f(int v) { return __int_as_float(v); }
__device__ __forceinline__ int f_bits(float v) { return __float_as_int(v); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    // DPP move with every row and bank enabled; lanes without a source read 0.
    return bits_f(__builtin_amdgcn_update_dpp(0, f_bits(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPR lanes (LPR a power of two <= 64); the sum is
// returned in every lane of the group.  Within a row of 16 lanes the exchange
// uses DPP (quad swaps, half-row mirror, row mirror); beyond it, lane swizzles.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPR >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (LPR >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
    if constexpr (LPR >= 16) v += dpp_f<0x140>(v);  // row_mirror
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Largest value / smallest int over the wave, returned in every lane: DPP
// inside each row of 16 lanes, then the four rows' results read as scalars.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    const int b = f_bits(v);
    const float r0 = bits_f(__builtin_amdgcn_readlane(b, 0)), r1 = bits_f(__builtin_amdgcn_readlane(b, 16));
    const float r2 = bits_f(__builtin_amdgcn_readlane(b, 32)), r3 = bits_f(__builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// Sum over the wave, complete in lane 63 only: DPP sums each row of 16 lanes,
// then row 1 (3) adds lane 15 (47) of the row before it and rows 2 and 3 add
// lane 31 (row broadcasts; rows outside the mask add 0).
__device__ __forceinline__ float wave_sum_last(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    v += bits_f(__builtin_amdgcn_update_dpp(0, f_bits(v), 0x142, 0xA, 0xF, false));   // row_bcast:15
    v += bits_f(__builtin_amdgcn_update_dpp(0, f_bits(v), 0x143, 0xC, 0xF, false));   // row_bcast:31
    return v;
}

// Inclusive prefix sum over the wave's lanes: within each row, the sums of
// the three lanes before (shifted in with zeros), then of the four and the
// eight before; then the row broadcasts carry each row's total onward.
__device__ __forceinline__ int wave_scan_incl(int v) {
    int s = v + dpp_i<0x111>(v) + dpp_i<0x112>(v) + dpp_i<0x113>(v);   // row_shr:1, 2, 3
    s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xF, 0xE, false);    // row_shr:4 into lanes 4-15
    s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xF, 0xC, false);    // row_shr:8 into lanes 8-15
    s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xA, 0xF, false);    // row_bcast:15 into rows 1, 3
    s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xC, 0xF, false);    // row_bcast:31 into rows 2, 3
    return s;
}

__device__ __forceinline__ int wave_min(int v) {
    v = min(v, dpp_i<0xB1>(v));
    v = min(v, dpp_i<0x4E>(v));
    v = min(v, dpp_i<0x141>(v));
    v = min(v, dpp_i<0x140>(v));
    const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return min(min(r0, r1), min(r2, r3));
}

__device__ __forceinline__ unsigned wave_max_u(unsigned v) {
    v = max(v, (unsigned)dpp_i<0xB1>((int)v));
    v = max(v, (unsigned)dpp_i<0x4E>((int)v));
    v = max(v, (unsigned)dpp_i<0x141>((int)v));
    v = max(v, (unsigned)dpp_i<0x140>((int)v));
    const unsigned r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const unsigned r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Same for a group size known only at run time (small shapes; not hot).
__device__ __forceinline__ float group_sum_rt(float v, int lpr) {
    for (int off = 1; off < lpr; off <<= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ------------------------------------------------------------ code decoding
//
// A lane reads 16 bytes of a packed row: 16 * (8/BITS) consecutive columns.
// The decoder turns each 32-bit word into floats without any per-field shift:
//   t = word ^ OFFSET_PATTERN   maps every two's-complement field q to the
//                                unsigned value q + 2^(BITS-1)
//   m_j = t & FIELD_MASK_j      isolates field j of all four bytes in place
//   v_cvt_f32_ubyte{k}(m_j)     = (q + 2^(BITS-1)) * 2^(j*BITS) for byte k
// so a dot product over the word is sum_j 2^(-j*BITS) * sum_k m_jk * x, minus
// 2^(BITS-1) * sum(x), which the callers subtract once per row.

template <int BITS>
struct Codec;

template <>
struct Codec<4> {
    static constexpr int F = 2;                     // fields per byte
    static constexpr uint32_t kFlip = 0x88888888u;
    static constexpr float kOffset = 8.0f;
    __device__ static constexpr uint32_t mask(int j) { return j == 0 ? 0x0F0F0F0Fu : 0xF0F0F0F0u; }
    __device__ static constexpr float scale(int j) { return j == 0 ? 1.0f : 0.0625f; }
};

template <>
struct Codec<8> {
    static constexpr int F = 1;
    static constexpr uint32_t kFlip = 0x80808080u;
    static constexpr float kOffset = 128.0f;
    __device__ static constexpr uint32_t mask(int) { return 0xFFFFFFFFu; }
    __device__ static constexpr float scale(int) { return 1.0f; }
};

template <>
struct Codec<2> {
    static constexpr int F = 4;
    static constexpr uint32_t kFlip = 0xAAAAAAAAu;
    static constexpr float kOffset = 2.0f;
    __device__ static constexpr uint32_t mask(int j) {
        return j == 0 ? 0x03030303u : j == 1 ? 0x0C0C0C0Cu : j == 2 ? 0x30303030u : 0xC0C0C0C0u;
    }
    __device__ static constexpr float scale(int j) {
        return j == 0 ? 1.0f : j == 1 ? 0.25f : j == 2 ? 0.0625f : 0.015625f;
    }
};

// Unsigned byte k of w as a float: one v_cvt_f32_ubyte{k}.  Written as asm
// because the compiler otherwise re-derives each byte with a bit-field extract
// from the unmasked word (two instructions per field instead of one).
template <int K>
__device__ __forceinline__ float ubyte_f(uint32_t w) {
    float r;
    if constexpr (K == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(w));
    else if constexpr (K == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(w));
    else if constexpr (K == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(w));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(w));
    return r;
}

// Decode one 16-byte group into 16*F floats (scaled field values, see above):
// out[(4*d + k) * F + j] belongs to column (4*d + k) * F + j of the group.
template <int BITS>
__device__ __forceinline__ void decode16(const uint4& q, float* out) {
    using C = Codec<BITS>;
    const uint32_t w[4] = {q.x ^ C::kFlip, q.y ^ C::kFlip, q.z ^ C::kFlip, q.w ^ C::kFlip};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int j = 0; j < C::F; ++j) {
            const uint32_t m = w[d] & C::mask(j);
            out[(4 * d + 0) * C::F + j] = ubyte_f<0>(m);
            out[(4 * d + 1) * C::F + j] = ubyte_f<1>(m);
            out[(4 * d + 2) * C::F + j] = ubyte_f<2>(m);
            out[(4 * d + 3) * C::F + j] = ubyte_f<3>(m);
        }
    }
}

// 128-bit global load.
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// ------------------------------------------------------------ launch interfaces

struct ExpertArgs {
    const uint8_t* w_gate;
    const uint8_t* w_up;
    const uint8_t* w_down;
    const float* s_gate;
    const float* s_up;
    const float* s_down;
    const int32_t* n_active;
    const int32_t* expert_id;
    const int32_t* seg;
    const int32_t* assign;
    int T, H, I, top_k, slots, max_active;
};

hipError_t launch_route(const float* x, const float* router_w, const float* bias, int T, int H,
                        int E, int n_group, int topk_group, int top_k, int n_shared, float rsf, float top_p,
                        float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                        hipStream_t stream);

hipError_t launch_gate_up(int bits, const float* x, const ExpertArgs& a, float* h, hipStream_t stream);
hipError_t launch_down_valu(int bits, const float* h, const float* topk_w, const ExpertArgs& a, float* y,
                            hipStream_t stream);

hipError_t launch_down_em(int bits, const float* h, const float* topk_w, const int32_t* topk_idx, const ExpertArgs& a,
                          float* part, float* y, hipStream_t stream);
// launch_down_em with its partial outputs in the library's per-device static
// array (hipErrorInvalidValue when T * slots * H exceeds it)
hipError_t launch_down_em_noalloc(int bits, const float* h, const float* topk_w, const int32_t* topk_idx,
                                  const ExpertArgs& a, float* y, hipStream_t stream);
hipError_t launch_down(int bits, const float* h, const float* topk_w, const ExpertArgs& a, float* y,
                       hipStream_t stream);

// Everything the fused layer launch needs (the worklist fields of `ex` unused).
struct FusedLayerArgs {
    ExpertArgs ex;
    const float* x;
    const float* router_w;
    const float* bias;
    float* scores;
    int32_t* topk_idx;
    float* topk_w;
    int32_t* wl_n_active;
    int32_t* wl_expert_id;
    int32_t* wl_seg;
    int32_t* wl_assign;
    float* h;
    float* y;
    int32_t* workspace;
    int T, E, n_group, topk_group, n_shared;
    float rsf;
    float top_p;               // >= 1: plain top-k
    float* x_out;              // non-null: residual form, x_out = x + y with x normalised inside
    float eps;                 // its RMSNorm epsilon
    int act8;                  // 1: Q8_0-style int8 activations in blocks
};

hipError_t launch_layer_fused(int bits, const FusedLayerArgs& args, hipStream_t stream);   // int8 activations
hipError_t launch_layer_pipe(int bits, const FusedLayerArgs& args, hipStream_t stream);    // 24-bit activations

hipError_t launch_pack(int bits, const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len,
                       hipStream_t stream);
hipError_t launch_unpack(int bits, const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len,
                         hipStream_t stream);

hipError_t launch_residual_rmsnorm(float* x, const float* y, float* xn, int T, int H, float eps,
                                   hipStream_t stream);

}  // namespace moedec
