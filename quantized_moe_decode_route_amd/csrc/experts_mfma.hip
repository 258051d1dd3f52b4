// Expert kernels on the matrix cores: gate/up + SwiGLU, and down + weighted
// combine, over row-scaled int8 / packed int4 / packed int2 codes (the row
// loops, the code -> f16 conversion and the operand layouts are in mfma.h;
// the expert-major down's row loop is here).
//
// The codes of each selected expert are streamed from HBM exactly once per
// token batch (the batch union of the worklist): one persistent 8-wave
// workgroup per compute unit, each owning a contiguous share of the rows.
#include <mutex>

#include "mfma.h"

namespace moedec {

namespace {

using namespace mfma;

// ------------------------------------------------- down, expert-major
//
// For larger batches: work units (segment, output row), a segment being an
// expert and up to ns of its assignments; each segment stages only its own
// assignments' h rows times their routing weights (as B columns), so a
// workgroup reads h for the experts it streams, not for the whole batch.
// Every unit writes its assignments' partial outputs part[a][r] =
// s_down[r] * (Qd . h_a w_a)[r]; down_reduce adds them per token in slot
// order afterwards.  No atomics: deterministic.

// Rows [rlo, rhi) of expert e's down matrix for the nc staged columns.
// red: LDS [kMW][NBE][16][ns]; sd_s: LDS [NBE*16].
template <int BITS>
__device__ __forceinline__ void down_em_rows(const ExpertArgs& a, float* __restrict__ part, int e, int rlo, int rhi,
                                             int nc, const int* asg, const half8* hhi, const half8* hlo, int ns,
                                             float unscale, float* red, float* sd_s) {
    using M = MfmaCodec<BITS>;
    constexpr int NCALL = M::NCALL;
    constexpr int kNB = M::NBE;
    static_assert(kNB <= kNBMax, "the row-scale array holds kNBMax blocks");
    const int H = a.H, I = a.I;
    const int row_bytes = I * BITS / 8;
    const int P = row_bytes >> 4;
    const int NCH = (P + 3) / 4;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int ln = lane & 15, lq = lane >> 4;
    const int cw0 = wave * NCH / kMW, cw1 = (wave + 1) * NCH / kMW;
    const int nk = cw1 - cw0;
    const int bslot = ln < nc ? ln : -1;
    const uint8_t* db = a.w_down + (size_t)e * H * row_bytes;

    constexpr int G = kNB * 16;
    // chunk ch of the group starting at row gs
    auto issue_at = [&](int gs, int ch, uint4* dd) {
        const int grp = min(ch * 4 + lq, P - 1);
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            const int r = min(gs + b * 16 + ln, rhi - 1);
            dd[b] = ld16(db + (size_t)r * row_bytes + grp * 16);
        }
    };
    // With an even chunk count per wave the next group's first two chunks go
    // out as soon as this group's buffers are free, ahead of its reduction
    // (the last group re-reads its own first chunks instead).
    const bool ahead = nk > 0 && (nk & 1) == 0;
    uint4 d0[kNB], d1[kNB];
    if (ahead) {
        issue_at(rlo, cw0, d0);
        issue_at(rlo, cw0 + 1, d1);
    }
    for (int g0 = rlo; g0 < rhi; g0 += G) {
        const int gn = min(rhi - g0, G);
        const int nb = (gn + 15) >> 4;
        const int sr = min((int)threadIdx.x, gn - 1);
        const float sdv = a.s_down[(size_t)e * H + g0 + sr];
        floatx4 acc[kNB];
#pragma unroll
        for (int b = 0; b < kNB; ++b) acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
        auto issue = [&](int ch, uint4* dd) { issue_at(g0, ch, dd); };
        auto compute = [&](int ch, const uint4* dd) {
            half8 bh[NCALL], bl[NCALL];
#pragma unroll
            for (int c = 0; c < NCALL; ++c) {
                if (bslot >= 0) {
                    const int src = ((ch * 4 + lq) * ns + bslot) * NCALL + c;
                    bh[c] = hhi[src];
                    bl[c] = hlo[src];
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2) bh[c][e2] = bl[c][e2] = (_Float16)0.f;
                }
            }
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                if (b < nb) {
#pragma unroll
                    for (int c = 0; c < NCALL; ++c) {
                        const half8 ad = a_operand<BITS>(dd[b], c);
                        acc[b] = mfma::mfma(ad, bh[c], acc[b]);
                        acc[b] = mfma::mfma(ad, bl[c], acc[b]);
                    }
                }
            }
        };
        if (ahead) {
            const int gnx = g0 + G < rhi ? g0 + G : g0;
            for (int t = 0; t < nk; t += 2) {          // chunks t, t+1 are in d0, d1
                compute(cw0 + t, d0);
                const bool in0 = t + 2 < nk;
                issue_at(in0 ? g0 : gnx, in0 ? cw0 + t + 2 : cw0, d0);
                compute(cw0 + t + 1, d1);
                issue_at(in0 ? g0 : gnx, in0 ? cw0 + t + 3 : cw0 + 1, d1);
            }
        } else if (nk > 0) {
            issue(cw0, d0);
            for (int t = 0; t < nk; t += 2) {          // two register buffers, alternating
                issue(cw0 + min(t + 1, nk - 1), d1);
                compute(cw0 + t, d0);
                issue(cw0 + min(t + 2, nk - 1), d0);
                if (t + 1 < nk) compute(cw0 + t + 1, d1);
            }
        }
        if ((int)threadIdx.x < gn) sd_s[threadIdx.x] = sdv;
        if (ln < nc) {
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                if (b < nb) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) red[((wave * kNB + b) * 16 + 4 * lq + i) * ns + ln] = acc[b][i];
                }
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < gn * nc; idx += kMT) {
            const int r = idx / nc, n = idx - r * nc;
            const int b = r >> 4, rr = r & 15;
            float v = 0.f;
            for (int w = 0; w < kMW; ++w) v += red[((w * kNB + b) * 16 + rr) * ns + n];
            part[(size_t)asg[n] * H + g0 + r] = v * unscale * sd_s[r];
        }
        __syncthreads();
    }
}

struct DownEmLds {
    int cpre[kMaxActive + 1];
    int asg[kCols];
    float mul[kCols];
    float scratch[kMW];
    float sd[kNBMax * 16];
    int kexp;
};

// This workgroup's share `part` of `nparts` of the (segment, row) units.
template <int BITS>
__device__ __forceinline__ void down_em_units(const ExpertArgs& a, const float* __restrict__ h,
                                              const float* __restrict__ topk_w, float* __restrict__ part_out,
                                              const int* eid, const int* seg, const int* assign, int n_exp, int ns,
                                              int part, int nparts, half8* hhi, half8* hlo, float* red,
                                              DownEmLds& s) {
    const int H = a.H, I = a.I;
    mw_segment_prefix(seg, n_exp, ns, s.cpre);
    const int n_seg = s.cpre[n_exp];
    const long long n_units = (long long)n_seg * H;
    const long long u0 = n_units * part / nparts;
    const long long u1 = n_units * (part + 1) / nparts;
    if (u0 >= u1) return;                        // uniform over the workgroup
    for (int sidx = (int)(u0 / H); (long long)sidx * H < u1; ++sidx) {
        const int rlo = (int)max(u0 - (long long)sidx * H, 0LL);
        const int rhi = (int)min(u1 - (long long)sidx * H, (long long)H);
        const int j = mw_upper_index(s.cpre, n_exp, sidx);
        const int first = seg[j] + (sidx - s.cpre[j]) * ns;
        const int nc = min(ns, seg[j + 1] - first);
        __syncthreads();   // everyone is done with the previous segment's LDS
        if ((int)threadIdx.x < nc) {
            const int as = assign[first + threadIdx.x];
            const int t = as / a.slots, sl = as - t * a.slots;
            s.asg[threadIdx.x] = as;
            s.mul[threadIdx.x] = sl < a.top_k ? topk_w[t * a.top_k + sl] : 1.0f;
        }
        __syncthreads();
        const int k = stage_b<BITS>(h, I, I, s.asg, s.mul, nc, ns, hhi, hlo, s.scratch);
        if (threadIdx.x == 0) s.kexp = k;
        __syncthreads();
        down_em_rows<BITS>(a, part_out, eid[j], rlo, rhi, nc, s.asg, hhi, hlo, ns, ldexpf(1.0f, -s.kexp), red, s.sd);
    }
}

// LDS per staged assignment of down_em_units: hi + lo B operands and the reduction.
template <int BITS>
__host__ __device__ constexpr size_t down_em_lds_per_col(int I) {
    return staged_row_bytes<BITS>(I) + (size_t)kMW * MfmaCodec<BITS>::NBE * 16 * sizeof(float);
}

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
    for (int s0 = 0; s0 < slots; s0 += 8) {
        // the loads of 8 slots at once (valid rows and indices), then the sum in slot order
        float v[8];
        int id[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int sl = min(s0 + k, slots - 1);
            v[k] = part[((size_t)t * slots + sl) * H + r];
            id[k] = topk_idx != nullptr && sl < K ? topk_idx[t * K + sl] : 0;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (s0 + k < slots && id[k] >= 0) acc += v[k];
    }
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

// ------------------------------------------------ the no-allocation down call
//
// The expert-major down call with its partial outputs in a file-scope device
// array instead of a caller buffer, for callers that cannot allocate.  Each
// GPU holds its own copy of the array until the process ends; the host finds
// its address once per device with hipGetSymbolAddress (the array's name in
// host code is not a device address).  Every call on a GPU reuses that GPU's
// array, so calls that overlap on one GPU race; every row a call reads back
// was written earlier in the same call, so nothing needs clearing.
static __device__ __align__(256) float scratch[MOEDEC_NOALLOC_PART_FLOATS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_part(float** out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<float*>(g_scratch_ptr[dev]);
    return hipSuccess;
}

hipError_t launch_down_em_noalloc(int bits, const float* h, const float* topk_w, const int32_t* topk_idx,
                                  const ExpertArgs& a, float* y, hipStream_t st) {
    if ((long long)a.T * a.slots * a.H > MOEDEC_NOALLOC_PART_FLOATS) return hipErrorInvalidValue;
    float* part = nullptr;
    const hipError_t err = noalloc_part(&part);
    if (err != hipSuccess) return err;
    return launch_down_em(bits, h, topk_w, topk_idx, a, part, y, st);
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
