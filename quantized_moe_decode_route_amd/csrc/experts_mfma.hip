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

// Gate/up work units are (segment, row): segment = (active expert j, a chunk
// of up to `ns` of its tokens), enumerated expert-ascending; workgroup b takes
// the b-th equal contiguous share.  With T <= ns all tokens are staged once and
// a segment's columns point at their tokens' slots; otherwise each segment
// stages its own tokens (skipped when they are the ones already staged).
template <int BITS>
__global__ __launch_bounds__(kMT) void gate_up_mfma_kernel(const float* __restrict__ x, const ExpertArgs a,
                                                           float* __restrict__ h, int ns) {
    using M = MfmaCodec<BITS>;
    constexpr int NCALL = M::NCALL;
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ int eid[kMaxActive];
    __shared__ int seg[kMaxActive + 1];
    __shared__ int cpre[kMaxActive + 1];
    __shared__ int tok_s[kCols], asg_s[kCols], col_s[kCols], staged_s[kCols];
    __shared__ float scratch[kMW];
    __shared__ int kexp_s;
    __shared__ float sg_s[kNBMax * 16], su_s[kNBMax * 16];

    const int H = a.H, I = a.I, T = a.T;
    const int NCH = ((H * BITS / 8) / 16 + 3) / 4;
    half8* xhi = reinterpret_cast<half8*>(dyn);
    half8* xlo = xhi + (size_t)NCH * 4 * ns * NCALL;
    float* red = reinterpret_cast<float*>(xlo + (size_t)NCH * 4 * ns * NCALL);
    const bool stage_all = T <= ns;

    if (threadIdx.x < kCols) staged_s[threadIdx.x] = -1;
    if (stage_all) {   // all tokens once: slot = token index
        if (threadIdx.x < kCols) tok_s[threadIdx.x] = threadIdx.x;
        __syncthreads();
        const int k = stage_b<BITS>(x, H, H, tok_s, nullptr, T, ns, xhi, xlo, scratch);
        if (threadIdx.x == 0) kexp_s = k;
    }
    const int n_act = mw_load_worklist(a, eid, seg);
    mw_segment_prefix(seg, n_act, ns, cpre);

    const int n_seg = cpre[n_act];
    const long long n_units = (long long)n_seg * I;
    const long long u0 = n_units * blockIdx.x / gridDim.x;
    const long long u1 = n_units * (blockIdx.x + 1) / gridDim.x;
    if (u0 >= u1) return;

    for (int sidx = (int)(u0 / I); (long long)sidx * I < u1; ++sidx) {
        const int rlo = (int)max(u0 - (long long)sidx * I, 0LL);
        const int rhi = (int)min(u1 - (long long)sidx * I, (long long)I);
        const int j = mw_upper_index(cpre, n_act, sidx);
        const int e = eid[j];
        const int first = seg[j] + (sidx - cpre[j]) * ns;
        const int nc = min(ns, seg[j + 1] - first);
        __syncthreads();   // everyone is done with the previous segment's LDS
        if ((int)threadIdx.x < nc) {
            const int as = a.assign[first + threadIdx.x];
            asg_s[threadIdx.x] = as;
            tok_s[threadIdx.x] = as / a.slots;
            col_s[threadIdx.x] = stage_all ? as / a.slots : (int)threadIdx.x;
        }
        __syncthreads();
        if (!stage_all) {
            bool same = true;
            for (int k = 0; k < nc; ++k) same = same && staged_s[k] == tok_s[k];
            if (!same) {
                const int k = stage_b<BITS>(x, H, H, tok_s, nullptr, nc, ns, xhi, xlo, scratch);
                if (threadIdx.x == 0) kexp_s = k;
                if (threadIdx.x < kCols) staged_s[threadIdx.x] = (int)threadIdx.x < nc ? tok_s[threadIdx.x] : -1;
                __syncthreads();
            }
        }
        gate_up_rows<BITS>(a, h, e, rlo, rhi, nc, col_s, asg_s, xhi, xlo, ns, ldexpf(1.0f, -kexp_s), red, sg_s,
                           su_s);
    }
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
    down_rows<BITS>(h, topk_w, a, y, r0, r1, qc, dyn, eid, seg, a.assign, n_act, scratch);
}

template <int BITS>
hipError_t gate_up_mfma_bits(const float* x, const ExpertArgs& a, float* h, hipStream_t st) {
    // per staged token: hi + lo B operands and the reduction buffer
    const size_t per_tok = staged_row_bytes<BITS>(a.H) + gate_up_red_bytes_per_token<BITS>();
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
