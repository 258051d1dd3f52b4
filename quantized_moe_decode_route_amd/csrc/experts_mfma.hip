// Expert kernels on the matrix cores: gate/up + SwiGLU, and down + weighted
// combine, over row-scaled int8 / packed int4 / packed int2 codes (the row
// loops, the code -> f16 conversion and the operand layouts are in mfma.h).
//
// The codes of each selected expert are streamed from HBM exactly once per
// token batch (the batch union of the worklist): one persistent 8-wave
// workgroup per compute unit, each owning a contiguous share of the rows.
#include "mfma.h"

namespace moedec {

namespace {

using namespace mfma;

// Gate/up: all tokens staged once when they fit (T <= ns), then this
// workgroup's share of the (segment, row) units.
template <int BITS>
__global__ __launch_bounds__(kMT) void gate_up_mfma_kernel(const float* __restrict__ x, const ExpertArgs a,
                                                           float* __restrict__ h, int ns) {
    constexpr int NCALL = MfmaCodec<BITS>::NCALL;
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ int eid[kMaxActive];
    __shared__ int seg[kMaxActive + 1];
    __shared__ GateUpLds s;
    const int NCH = ((a.H * BITS / 8) / 16 + 3) / 4;
    half8* xhi = reinterpret_cast<half8*>(dyn);
    half8* xlo = xhi + (size_t)NCH * 4 * ns * NCALL;
    float* red = reinterpret_cast<float*>(xlo + (size_t)NCH * 4 * ns * NCALL);
    const bool stage_all = a.T <= ns;
    if (stage_all) stage_tokens<BITS>(x, a.T, a.H, ns, xhi, xlo, s);
    const int n_act = mw_load_worklist(a, eid, seg);
    gate_up_units<BITS>(a, x, h, eid, seg, a.assign, n_act, ns, stage_all, blockIdx.x, gridDim.x, xhi, xlo, red, s);
}

// Down: workgroup b owns output rows [b*rows, (b+1)*rows) for the whole batch.
template <int BITS>
__global__ __launch_bounds__(kMT) void down_mfma_kernel(const float* __restrict__ h,
                                                        const float* __restrict__ topk_w, const ExpertArgs a,
                                                        float* __restrict__ y, int qc, int rows_per_wg) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ int eid[kMaxActive];
    __shared__ int seg[kMaxActive + 1];
    __shared__ float scratch[kMW];
    const int r0 = blockIdx.x * rows_per_wg;
    const int r1 = min(r0 + rows_per_wg, a.H);
    if (r0 >= r1) return;
    const int n_act = mw_load_worklist(a, eid, seg);
    NoGate gate;
    down_rows<BITS>(h, topk_w, a, y, r0, r1, qc, dyn, eid, seg, a.assign, n_act, scratch, gate);
}

// Down, expert-major: this workgroup's share of the (segment, row) units, each
// segment staging only its own assignments' h; partial outputs to part.
template <int BITS>
__global__ __launch_bounds__(kMT) void down_em_kernel(const float* __restrict__ h, const float* __restrict__ topk_w,
                                                      const ExpertArgs a, float* __restrict__ part, int ns) {
    constexpr int NCALL = MfmaCodec<BITS>::NCALL;
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ int eid[kMaxActive];
    __shared__ int seg[kMaxActive + 1];
    __shared__ DownEmLds s;
    const int NCH = ((a.I * BITS / 8) / 16 + 3) / 4;
    half8* hhi = reinterpret_cast<half8*>(dyn);
    half8* hlo = hhi + (size_t)NCH * 4 * ns * NCALL;
    float* red = reinterpret_cast<float*>(hlo + (size_t)NCH * 4 * ns * NCALL);
    const int n_act = mw_load_worklist(a, eid, seg);
    down_em_units<BITS>(a, h, topk_w, part, eid, seg, a.assign, n_act, ns, blockIdx.x, gridDim.x, hhi, hlo, red, s);
}

// y[t][r] = sum over token t's slots, in slot order, of part[t*slots + slot][r]
// (routed slots without an expert -- dropped by top-p -- skipped).
__global__ __launch_bounds__(256) void down_reduce_kernel(const float* __restrict__ part,
                                                          const int32_t* __restrict__ topk_idx, int T, int H, int K,
                                                          int slots, float* __restrict__ y) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)T * H) return;
    const int t = (int)(i / H), r = (int)(i - (long long)t * H);
    float acc = 0.f;
    for (int sl = 0; sl < slots; ++sl)
        if (sl >= K || topk_idx == nullptr || topk_idx[t * K + sl] >= 0) acc += part[((size_t)t * slots + sl) * H + r];
    y[i] = acc;
}

template <int BITS>
hipError_t down_em_bits(const float* h, const float* topk_w, const int32_t* topk_idx, const ExpertArgs& a, float* part,
                        float* y, hipStream_t st) {
    const size_t per_col = down_em_lds_per_col<BITS>(a.I);
    int fit = (int)((kLdsMax - kStatic) / per_col);
    if (fit > kCols) fit = kCols;
    if (fit < 1) return hipErrorInvalidValue;
    const int ns = fit;
    size_t lds = (size_t)ns * per_col;
    if (lds < kLdsOnePerCu) lds = kLdsOnePerCu;
    auto k = down_em_kernel<BITS>;
    hipError_t err = allow_lds(k, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(cu_count()), dim3(kMT), lds, st, h, topk_w, a, part, ns);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const long long n = (long long)a.T * a.H;
    hipLaunchKernelGGL(down_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, topk_idx, a.T,
                       a.H, a.top_k, a.slots, y);
    return hipGetLastError();
}

template <int BITS>
hipError_t gate_up_mfma_bits(const float* x, const ExpertArgs& a, float* h, hipStream_t st) {
    // per staged token: hi + lo B operands and the reduction buffer
    const size_t per_tok = gate_up_lds_per_token<BITS>(a.H);
    int fit = (int)((kLdsMax - kStatic) / per_tok);
    if (fit > kCols) fit = kCols;
    if (fit < 1) return hipErrorInvalidValue;
    const int ns = a.T < fit ? a.T : fit;
    size_t lds = (size_t)ns * per_tok;
    if (lds < kLdsOnePerCu) lds = kLdsOnePerCu;
    auto k = gate_up_mfma_kernel<BITS>;
    hipError_t err = allow_lds(k, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(cu_count()), dim3(kMT), lds, st, x, a, h, ns);
    return hipGetLastError();
}

template <int BITS>
hipError_t down_mfma_bits(const float* h, const float* topk_w, const ExpertArgs& a, float* y, hipStream_t st) {
    const int n_wg = cu_count();
    int rows = (a.H + n_wg - 1) / n_wg;
    if (rows > kNBD * 16) rows = kNBD * 16;          // then more workgroups than CUs
    if (a.T > kCols) return hipErrorInvalidValue;
    const int A = a.T * a.slots;
    const size_t fixed = down_lds_fixed_bytes();
    const size_t per_q = down_lds_bytes_per_assignment<BITS>(a.I);
    int qc = (int)((kLdsMax - kStatic - fixed) / per_q);
    if (qc < 1) return hipErrorInvalidValue;
    if (qc > A) qc = A;
    size_t lds = fixed + (size_t)qc * per_q;
    if (lds < kLdsOnePerCu) lds = kLdsOnePerCu;
    auto k = down_mfma_kernel<BITS>;
    hipError_t err = allow_lds(k, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3((a.H + rows - 1) / rows), dim3(kMT), lds, st, h, topk_w, a, y, qc, rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(int bits, const float* x, const ExpertArgs& a, float* h, hipStream_t st) {
    switch (bits) {
        case 4: return gate_up_mfma_bits<4>(x, a, h, st);
        case 8: return gate_up_mfma_bits<8>(x, a, h, st);
        case 2: return gate_up_mfma_bits<2>(x, a, h, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_down_em(int bits, const float* h, const float* topk_w, const int32_t* topk_idx, const ExpertArgs& a,
                          float* part, float* y, hipStream_t st) {
    switch (bits) {
        case 4: return down_em_bits<4>(h, topk_w, topk_idx, a, part, y, st);
        case 8: return down_em_bits<8>(h, topk_w, topk_idx, a, part, y, st);
        case 2: return down_em_bits<2>(h, topk_w, topk_idx, a, part, y, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_down(int bits, const float* h, const float* topk_w, const ExpertArgs& a, float* y,
                       hipStream_t st) {
    if (a.T > kCols) return launch_down_valu(bits, h, topk_w, a, y, st);
    switch (bits) {
        case 4: return down_mfma_bits<4>(h, topk_w, a, y, st);
        case 8: return down_mfma_bits<8>(h, topk_w, a, y, st);
        case 2: return down_mfma_bits<2>(h, topk_w, a, y, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moedec
