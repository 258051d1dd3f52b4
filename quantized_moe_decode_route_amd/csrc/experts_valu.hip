// Down projection + weighted combine on the vector ALUs, over row-scaled int8
// / packed int4 / packed int2 codes (dequantised on use), for the batches the
// matrix-core down kernels (experts_mfma.hip) do not take: more than 16
// tokens.  Gate/up always runs on the matrix cores.
//
// The kernel is persistent: one workgroup of 8 waves per compute unit, each
// owning a contiguous block of output rows for the whole batch, so every
// selected expert's packed rows are streamed exactly once per token batch
// (the batch union of the worklist).  Rows are split into 16-byte groups and
// the lanes of a lane group take consecutive groups, so one wave-wide load
// covers a contiguous 1 KB.  Each wave keeps W such loads in flight in a
// register ring while it decodes earlier ones.  The worklist is copied to LDS
// first so no weight load waits behind a global lookup.  The activations (h)
// are staged in LDS in a group-transposed layout [row][column-in-group][group],
// so the lanes of a wave read consecutive LDS words (no bank conflicts).
#include "common.h"

namespace moedec {

constexpr int kPThreads = 512;
constexpr int kPWaves = kPThreads / kWave;
constexpr int kMaxActive = MOEDEC_MAX_EXPERTS + 8;

// Copy n_active, expert_id[] and seg[] of the worklist to LDS (whole workgroup).
__device__ __forceinline__ int load_worklist(const ExpertArgs& a, int* eid, int* seg) {
    __shared__ int n_s;
    if (threadIdx.x == 0) n_s = *a.n_active;
    __syncthreads();
    const int n = n_s;
    for (int j = threadIdx.x; j <= n; j += blockDim.x) {
        if (j < n) eid[j] = a.expert_id[j];
        seg[j] = a.seg[j];
    }
    __syncthreads();
    return n;
}

// Largest j in [0, n) with v[j] <= q (v ascending, v[0] <= q).
__device__ __forceinline__ int upper_index(const int* v, int n, int q) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (v[mid] <= q) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ------------------------------------------------------------ down + combine
//
// Each workgroup owns a contiguous block of output rows for the whole batch.
// It walks the worklist (experts ascending) in chunks of up to `qc`
// assignments, stages those assignments' h (pre-multiplied by their routing
// weight) in LDS, and adds every expert's contribution to its rows in a fixed
// order, so the sum needs no atomics and is deterministic.  DEFER (one
// token): lanes accumulate over all experts of a row before one reduction;
// otherwise each (row, assignment) partial is reduced and added to the row's
// per-token accumulator in LDS by the row's owning lane.

template <int BITS, bool DEFER, int LPR, int W>
__global__ __launch_bounds__(kPThreads) void down_kernel(const float* __restrict__ h,
                                                         const float* __restrict__ topk_w, const ExpertArgs a,
                                                         float* __restrict__ y, int lpr_rt, int qc, int rows_per_wg) {
    using C = Codec<BITS>;
    constexpr int F = C::F;
    constexpr int CW = 16 * F;
    extern __shared__ float lds[];
    __shared__ int eid[kMaxActive];
    __shared__ int seg[kMaxActive + 1];

    const int H = a.H, I = a.I, T = a.T, K = a.top_k, slots = a.slots;
    const int row_bytes = I * BITS / 8;
    const int P = row_bytes >> 4;
    const int lpr = LPR > 0 ? LPR : lpr_rt;
    const int spl = P / lpr;
    const int gpw = kWave / lpr;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int grp = lane / lpr, li = lane - grp * lpr;
    const int r0 = blockIdx.x * rows_per_wg;
    const int r1 = min(r0 + rows_per_wg, H);
    if (r0 >= r1) return;
    const int nrows = r1 - r0;
    const int rows_per_iter = kPWaves * gpw;
    const int n_iter = (nrows + rows_per_iter - 1) / rows_per_iter;

    float* hs = lds;                          // [qc][CW][P]
    float* hsum = hs + (size_t)qc * CW * P;   // [qc][P]
    float* yacc = hsum + (size_t)qc * P;      // [rows_per_wg][T]
    int* qtok = reinterpret_cast<int*>(yacc + (size_t)rows_per_wg * T);  // [qc]

    for (int i = threadIdx.x; i < rows_per_wg * T; i += kPThreads) yacc[i] = 0.f;
    const int n_act = load_worklist(a, eid, seg);
    const int A = seg[n_act];
    const uint8_t* wd_base = a.w_down + (size_t)r0 * row_bytes;

    for (int q0 = 0; q0 < A; q0 += qc) {
        const int q1 = min(A, q0 + qc);
        const int nq = q1 - q0;
        const int j_first = upper_index(seg, n_act, q0);
        const int j_last = upper_index(seg, n_act, q1 - 1);
        const int ipr = (j_last - j_first + 1) * spl;          // items per row iteration
        const int n_items = n_iter * ipr;

        auto row_of = [&](int it) { return it * rows_per_iter + wave * gpw + grp; };   // relative to r0
        uint4 buf[W];
        float bsd[W];
        auto issue = [&](int i, int w) {
            const int it = i / ipr, rem = i - it * ipr;
            const int jq = rem / spl, s = rem - jq * spl;
            const int rl = min(row_of(it), nrows - 1);
            const int ex = eid[j_first + jq];
            buf[w] = ld16(wd_base + ((size_t)ex * H + rl) * row_bytes + (li + s * lpr) * 16);
            bsd[w] = a.s_down[(size_t)ex * H + r0 + rl];
        };
        // weights first: these loads fly while h is staged
#pragma unroll
        for (int w = 0; w < W; ++w)
            if (w < n_items) issue(w, w);

        __syncthreads();   // previous chunk's readers are done with hs
        for (int ql = threadIdx.x; ql < nq; ql += kPThreads) qtok[ql] = a.assign[q0 + ql] / slots;
        for (int idx = threadIdx.x; idx < nq * P; idx += kPThreads) {
            const int ql = idx / P, p = idx - ql * P;
            const int as = a.assign[q0 + ql];
            const int t = as / slots, slot = as - t * slots;
            const float wq = slot < K ? topk_w[t * K + slot] : 1.0f;
            const float4* s4 = reinterpret_cast<const float4*>(h + (size_t)as * I + p * CW);
            float sum = 0.f;
#pragma unroll
            for (int c4 = 0; c4 < CW / 4; ++c4) {
                const float4 v = s4[c4];
                const float v0 = wq * v.x, v1 = wq * v.y, v2 = wq * v.z, v3 = wq * v.w;
                hs[(ql * CW + 4 * c4 + 0) * P + p] = v0;
                hs[(ql * CW + 4 * c4 + 1) * P + p] = v1;
                hs[(ql * CW + 4 * c4 + 2) * P + p] = v2;
                hs[(ql * CW + 4 * c4 + 3) * P + p] = v3;
                sum += (v0 + v1) + (v2 + v3);
            }
            hsum[ql * P + p] = sum;
        }
        __syncthreads();

        float acc = 0.f;
        for (int base = 0; base < n_items; base += W) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const int i = base + w;
                if (i >= n_items) break;
                const uint4 cq = buf[w];
                const float sd = bsd[w];
                if (i + W < n_items) issue(i + W, w);
                const int it = i / ipr, rem = i - it * ipr;
                const int jq = rem / spl, s = rem - jq * spl;
                const int jj = j_first + jq;
                const int rl = row_of(it);
                const int p = li + s * lpr;
                const int qa = max(seg[jj], q0) - q0, qb = min(seg[jj + 1], q1) - q0;
                for (int ql = qa; ql < qb; ++ql) {
                    float pr[F];
#pragma unroll
                    for (int f = 0; f < F; ++f) pr[f] = 0.f;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        float hv[4 * F];
#pragma unroll
                        for (int m = 0; m < 4 * F; ++m) hv[m] = hs[(ql * CW + 4 * d * F + m) * P + p];
                        const uint32_t wdw = (d == 0 ? cq.x : d == 1 ? cq.y : d == 2 ? cq.z : cq.w) ^ C::kFlip;
#pragma unroll
                        for (int f = 0; f < F; ++f) {
                            const uint32_t m = wdw & C::mask(f);
                            pr[f] = fmaf(ubyte_f<0>(m), hv[0 * F + f], pr[f]);
                            pr[f] = fmaf(ubyte_f<1>(m), hv[1 * F + f], pr[f]);
                            pr[f] = fmaf(ubyte_f<2>(m), hv[2 * F + f], pr[f]);
                            pr[f] = fmaf(ubyte_f<3>(m), hv[3 * F + f], pr[f]);
                        }
                    }
                    float v = -C::kOffset * hsum[ql * P + p];
#pragma unroll
                    for (int f = 0; f < F; ++f) v += C::scale(f) * pr[f];
                    if constexpr (DEFER) {
                        acc = fmaf(sd, v, acc);
                    } else {
                        if constexpr (LPR > 0) v = group_sum<LPR>(v);
                        else v = group_sum_rt(v, lpr);
                        if (li == 0 && rl < nrows) yacc[rl * T + qtok[ql]] += sd * v;
                    }
                }
                if constexpr (DEFER) {
                    if (rem == ipr - 1) {
                        float v = acc;
                        acc = 0.f;
                        if constexpr (LPR > 0) v = group_sum<LPR>(v);
                        else v = group_sum_rt(v, lpr);
                        if (li == 0 && rl < nrows) yacc[rl * T] += v;
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nrows * T; i += kPThreads) {
        const int t = i / nrows, rl = i - t * nrows;
        y[(size_t)t * H + r0 + rl] = yacc[rl * T + t];
    }
}

// --------------------------------------------------------------------- launch

namespace {

constexpr int kDnW = 8;   // down items in flight per wave
constexpr size_t kLdsMax = 160 * 1024;
// Static LDS of the persistent kernels (worklist copies) plus headroom.
constexpr size_t kStaticLds = 16 * 1024;
// Dynamic LDS a persistent workgroup asks for at least, so that no two of
// them share a compute unit.
constexpr size_t kLdsOnePerCu = 84 * 1024;

// Lanes sharing one row: the largest power of two dividing the row's group
// count, at most a wave; each lane then takes P / lanes groups.
int lanes_per_row(int P) {
    const int pow2 = P & (-P);
    return pow2 >= kWave ? kWave : pow2;
}

// Compute units of the current device (queried once per device).
int cu_count() {
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

template <typename Kern>
hipError_t allow_lds(Kern k, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int BITS>
hipError_t down_bits(const float* h, const float* topk_w, const ExpertArgs& a, float* y, hipStream_t st) {
    constexpr int CW = 16 * Codec<BITS>::F;
    const int P = (a.I * BITS / 8) / 16;
    const int lpr = lanes_per_row(P);
    const int n_wg = cu_count();
    const int rows = (a.H + n_wg - 1) / n_wg;
    const int A = a.T * a.slots;
    const size_t fixed = (size_t)rows * a.T * sizeof(float);
    const size_t per_q = (size_t)(CW * P + P) * sizeof(float) + sizeof(int);
    int qc = (int)((kLdsMax - kStaticLds - fixed) / per_q);
    if (qc < 1) return hipErrorInvalidValue;
    if (qc > A) qc = A;
    size_t lds = fixed + (size_t)qc * per_q;
    if (lds < kLdsOnePerCu) lds = kLdsOnePerCu;
    const dim3 grid((a.H + rows - 1) / rows);
    const bool defer = a.T == 1;
#define MOEDEC_DOWN(DEF, L)                                                                     \
    do {                                                                                        \
        auto k = down_kernel<BITS, DEF, L, kDnW>;                                                 \
        hipError_t err = allow_lds(k, lds);                                                     \
        if (err != hipSuccess) return err;                                                      \
        hipLaunchKernelGGL(k, grid, dim3(kPThreads), lds, st, h, topk_w, a, y, lpr, qc, rows); \
    } while (0)
    if (lpr == kWave) {
        if (defer) MOEDEC_DOWN(true, kWave);
        else MOEDEC_DOWN(false, kWave);
    } else {
        if (defer) MOEDEC_DOWN(true, 0);
        else MOEDEC_DOWN(false, 0);
    }
#undef MOEDEC_DOWN
    return hipGetLastError();
}

}  // namespace

hipError_t launch_down_valu(int bits, const float* h, const float* topk_w, const ExpertArgs& a, float* y,
                            hipStream_t st) {
    switch (bits) {
        case 4: return down_bits<4>(h, topk_w, a, y, st);
        case 8: return down_bits<8>(h, topk_w, a, y, st);
        case 2: return down_bits<2>(h, topk_w, a, y, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moedec
