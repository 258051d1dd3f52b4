// Expert kernels: gate/up + SwiGLU, and down + weighted combine, over
// row-scaled int8 / packed int4 / packed int2 codes (dequantised on use).
//
// Both kernels stream every selected expert's packed rows exactly once per
// token batch (the batch union of the worklist) with 16-byte coalesced loads:
// a row is split into 16-byte groups and the lanes of a lane group take
// consecutive groups, so one wave-wide load covers a contiguous 1 KB.
// Activations (x for gate/up, h for down) are staged in LDS in a
// group-transposed layout [token][column-in-group][group], so the lanes of a
// wave read consecutive LDS words (no bank conflicts).
#include "common.h"

namespace moedec {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// ------------------------------------------------------------------ gate / up
//
// Grid: (row blocks of `rows_per_wg` rows, max_active); block y = active expert
// j (blocks beyond n_active exit).  A workgroup walks the expert's tokens in
// chunks of up to NTMAX, stages their activations, and computes RR gate rows
// and RR up rows per lane group per step.  h[a][r] = silu(g) * v.

template <int BITS, int NC, int RR, int LPR, int W>
__device__ __forceinline__ void gate_up_rows(const ExpertArgs& a, float* __restrict__ h, const float* xs,
                                             const float* xsum, const int* asg, int e, int row0,
                                             int row_end, int lpr) {
    using C = Codec<BITS>;
    constexpr int F = C::F;
    constexpr int CW = 16 * F;
    const int H = a.H, I = a.I;
    const int row_bytes = H * BITS / 8;
    const int P = row_bytes >> 4;
    const int spl = P / lpr;
    const int gpw = kWave / lpr;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int grp = lane / lpr, li = lane - grp * lpr;
    const int rows_per_iter = kWaves * gpw * RR;
    const int n_iter = (row_end - row0 + rows_per_iter - 1) / rows_per_iter;
    const int n_items = n_iter * spl;
    const uint8_t* gb = a.w_gate + (size_t)e * I * row_bytes;
    const uint8_t* ub = a.w_up + (size_t)e * I * row_bytes;
    const float* sg = a.s_gate + (size_t)e * I;
    const float* su = a.s_up + (size_t)e * I;

    // this lane's share of 2^(BITS-1) * sum(x) over its groups
    float xoff[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        float v = 0.f;
        for (int s = 0; s < spl; ++s) v += xsum[k * P + li + s * lpr];
        xoff[k] = C::kOffset * v;
    }

    auto row_of = [&](int it, int rr) {
        return row0 + it * rows_per_iter + (wave * gpw + grp) * RR + rr;
    };
    uint4 bg[W][RR], bu[W][RR];
    auto issue = [&](int i, uint4* dg, uint4* du) {
        const int it = i / spl, s = i - it * spl;
        const int p = li + s * lpr;
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            const int r = min(row_of(it, rr), I - 1);
            dg[rr] = ld16(gb + (size_t)r * row_bytes + p * 16);
            du[rr] = ld16(ub + (size_t)r * row_bytes + p * 16);
        }
    };
#pragma unroll
    for (int w = 0; w < W; ++w)
        if (w < n_items) issue(w, bg[w], bu[w]);

    float ag[RR][NC][F], au[RR][NC][F];
#pragma unroll
    for (int rr = 0; rr < RR; ++rr)
#pragma unroll
        for (int k = 0; k < NC; ++k)
#pragma unroll
            for (int f = 0; f < F; ++f) ag[rr][k][f] = au[rr][k][f] = 0.f;

    for (int base = 0; base < n_items; base += W) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int i = base + w;
            if (i >= n_items) break;
            uint4 cg[RR], cu[RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) { cg[rr] = bg[w][rr]; cu[rr] = bu[w][rr]; }
            if (i + W < n_items) issue(i + W, bg[w], bu[w]);
            const int it = i / spl, s = i - it * spl;
            const int p = li + s * lpr;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float xv[NC][4 * F];
#pragma unroll
                for (int k = 0; k < NC; ++k)
#pragma unroll
                    for (int m = 0; m < 4 * F; ++m) xv[k][m] = xs[(k * CW + 4 * d * F + m) * P + p];
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    const uint32_t wgd = (d == 0 ? cg[rr].x : d == 1 ? cg[rr].y : d == 2 ? cg[rr].z : cg[rr].w) ^ C::kFlip;
                    const uint32_t wud = (d == 0 ? cu[rr].x : d == 1 ? cu[rr].y : d == 2 ? cu[rr].z : cu[rr].w) ^ C::kFlip;
#pragma unroll
                    for (int f = 0; f < F; ++f) {
                        const uint32_t mg = wgd & C::mask(f), mu = wud & C::mask(f);
                        const float g0 = ubyte_f<0>(mg), g1 = ubyte_f<1>(mg), g2 = ubyte_f<2>(mg), g3 = ubyte_f<3>(mg);
                        const float u0 = ubyte_f<0>(mu), u1 = ubyte_f<1>(mu), u2 = ubyte_f<2>(mu), u3 = ubyte_f<3>(mu);
#pragma unroll
                        for (int k = 0; k < NC; ++k) {
                            ag[rr][k][f] = fmaf(g0, xv[k][0 * F + f], ag[rr][k][f]);
                            ag[rr][k][f] = fmaf(g1, xv[k][1 * F + f], ag[rr][k][f]);
                            ag[rr][k][f] = fmaf(g2, xv[k][2 * F + f], ag[rr][k][f]);
                            ag[rr][k][f] = fmaf(g3, xv[k][3 * F + f], ag[rr][k][f]);
                            au[rr][k][f] = fmaf(u0, xv[k][0 * F + f], au[rr][k][f]);
                            au[rr][k][f] = fmaf(u1, xv[k][1 * F + f], au[rr][k][f]);
                            au[rr][k][f] = fmaf(u2, xv[k][2 * F + f], au[rr][k][f]);
                            au[rr][k][f] = fmaf(u3, xv[k][3 * F + f], au[rr][k][f]);
                        }
                    }
                }
            }
            if (s == spl - 1) {
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    const int r = row_of(it, rr);
#pragma unroll
                    for (int k = 0; k < NC; ++k) {
                        float g = -xoff[k], v = -xoff[k];
#pragma unroll
                        for (int f = 0; f < F; ++f) {
                            g += C::scale(f) * ag[rr][k][f];
                            v += C::scale(f) * au[rr][k][f];
                            ag[rr][k][f] = au[rr][k][f] = 0.f;
                        }
                        if constexpr (LPR > 0) {
                            g = group_sum<LPR>(g);
                            v = group_sum<LPR>(v);
                        } else {
                            g = group_sum_rt(g, lpr);
                            v = group_sum_rt(v, lpr);
                        }
                        if (li == 0 && r < row_end) {
                            g *= sg[r];
                            v *= su[r];
                            h[(size_t)asg[k] * I + r] = g / (1.0f + __expf(-g)) * v;
                        }
                    }
                }
            }
        }
    }
}

template <int BITS, int NTMAX, int RR, int LPR, int W>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(const float* __restrict__ x, const ExpertArgs a,
                                                           float* __restrict__ h, int rows_per_wg, int lpr_rt) {
    using C = Codec<BITS>;
    constexpr int CW = 16 * C::F;
    extern __shared__ float lds[];
    __shared__ int asg_s[NTMAX];
    __shared__ int tok_s[NTMAX];

    const int j = blockIdx.y;
    if (j >= *a.n_active) return;
    const int e = a.expert_id[j];
    const int s0 = a.seg[j];
    const int n = a.seg[j + 1] - s0;
    const int H = a.H;
    const int P = (H * BITS / 8) >> 4;
    const int lpr = LPR > 0 ? LPR : lpr_rt;
    const int row0 = blockIdx.x * rows_per_wg;
    const int row_end = min(row0 + rows_per_wg, a.I);
    float* xs = lds;                      // [NTMAX][CW][P]
    float* xsum = lds + NTMAX * CW * P;   // [NTMAX][P]

    for (int c0 = 0; c0 < n; c0 += NTMAX) {
        const int nc = min(NTMAX, n - c0);
        __syncthreads();
        if (threadIdx.x < NTMAX) {
            const int as = (int)threadIdx.x < nc ? a.assign[s0 + c0 + threadIdx.x] : 0;
            asg_s[threadIdx.x] = as;
            tok_s[threadIdx.x] = as / a.slots;
        }
        __syncthreads();
        for (int k = 0; k < nc; ++k) {
            const float* src = x + (size_t)tok_s[k] * H;
            for (int p = threadIdx.x; p < P; p += kThreads) {
                const float4* s4 = reinterpret_cast<const float4*>(src + p * CW);
                float sum = 0.f;
#pragma unroll
                for (int c4 = 0; c4 < CW / 4; ++c4) {
                    const float4 v = s4[c4];
                    xs[(k * CW + 4 * c4 + 0) * P + p] = v.x;
                    xs[(k * CW + 4 * c4 + 1) * P + p] = v.y;
                    xs[(k * CW + 4 * c4 + 2) * P + p] = v.z;
                    xs[(k * CW + 4 * c4 + 3) * P + p] = v.w;
                    sum += (v.x + v.y) + (v.z + v.w);
                }
                xsum[k * P + p] = sum;
            }
        }
        __syncthreads();
        if constexpr (NTMAX >= 2) {
            if (nc == 2) {
                gate_up_rows<BITS, 2, RR, LPR, W>(a, h, xs, xsum, asg_s, e, row0, row_end, lpr);
                continue;
            }
        }
        gate_up_rows<BITS, 1, RR, LPR, W>(a, h, xs, xsum, asg_s, e, row0, row_end, lpr);
    }
}

// ------------------------------------------------------------ down + combine
//
// Grid: row blocks of `rows_per_wg` output rows.  A workgroup owns its rows for
// the whole batch: it walks the worklist (experts ascending) in chunks of up
// to `qc` assignments, stages those assignments' h (pre-multiplied by their
// routing weight) in LDS, and accumulates every expert's contribution to its
// rows in a fixed order, so the sum needs no atomics and is deterministic.
// DEFER (one token): lanes accumulate over all experts before one reduction
// per row; otherwise each (row, assignment) partial is reduced and added to
// the row's per-token accumulator in LDS by its owning lane.

template <int BITS, bool DEFER, int RR, int LPR, int W>
__global__ __launch_bounds__(kThreads) void down_kernel(const float* __restrict__ h,
                                                        const float* __restrict__ topk_w, const ExpertArgs a,
                                                        float* __restrict__ y, int rows_per_wg, int lpr_rt,
                                                        int qc) {
    using C = Codec<BITS>;
    constexpr int F = C::F;
    constexpr int CW = 16 * F;
    extern __shared__ float lds[];
    const int H = a.H, I = a.I, T = a.T, K = a.top_k, slots = a.slots;
    const int row_bytes = I * BITS / 8;
    const int P = row_bytes >> 4;
    const int lpr = LPR > 0 ? LPR : lpr_rt;
    const int spl = P / lpr;
    const int gpw = kWave / lpr;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int grp = lane / lpr, li = lane - grp * lpr;
    const int row0 = blockIdx.x * rows_per_wg;
    const int row_end = min(row0 + rows_per_wg, H);
    const int nrows = row_end - row0;
    const int rows_per_iter = kWaves * gpw * RR;
    const int n_iter = (nrows + rows_per_iter - 1) / rows_per_iter;
    const int n_act = *a.n_active;
    const int A = a.seg[n_act];

    float* hs = lds;                          // [qc][CW][P]
    float* hsum = hs + (size_t)qc * CW * P;   // [qc][P]
    float* yacc = hsum + (size_t)qc * P;      // [rows_per_wg][T]
    int* qtok = reinterpret_cast<int*>(yacc + (size_t)rows_per_wg * T);  // [qc]
    int* qexp = qtok + qc;                    // [qc]

    for (int i = threadIdx.x; i < rows_per_wg * T; i += kThreads) yacc[i] = 0.f;

    for (int q0 = 0; q0 < A; q0 += qc) {
        const int q1 = min(A, q0 + qc);
        const int nq = q1 - q0;
        __syncthreads();
        for (int ql = threadIdx.x; ql < nq; ql += kThreads) {
            const int q = q0 + ql;
            int lo = 0, hi = n_act - 1;           // expert j with seg[j] <= q < seg[j+1]
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (a.seg[mid] <= q) lo = mid; else hi = mid - 1;
            }
            qexp[ql] = lo;
            qtok[ql] = a.assign[q] / slots;
        }
        for (int idx = threadIdx.x; idx < nq * P; idx += kThreads) {
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
        const int j_first = qexp[0], j_last = qexp[nq - 1];
        const int n_items = (j_last - j_first + 1) * spl;

        for (int it = 0; it < n_iter; ++it) {
            const int rbase = row0 + it * rows_per_iter + (wave * gpw + grp) * RR;
            uint4 buf[W][RR];
            auto issue = [&](int i, uint4* dst) {
                const int jj = j_first + i / spl, s = i % spl;
                const int ex = a.expert_id[jj];
                const int p = li + s * lpr;
                const uint8_t* base = a.w_down + (size_t)ex * H * row_bytes + p * 16;
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    const int r = min(rbase + rr, H - 1);
                    dst[rr] = ld16(base + (size_t)r * row_bytes);
                }
            };
#pragma unroll
            for (int w = 0; w < W; ++w)
                if (w < n_items) issue(w, buf[w]);
            float acc[RR];
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) acc[rr] = 0.f;

            for (int base = 0; base < n_items; base += W) {
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const int i = base + w;
                    if (i >= n_items) break;
                    uint4 cq[RR];
#pragma unroll
                    for (int rr = 0; rr < RR; ++rr) cq[rr] = buf[w][rr];
                    if (i + W < n_items) issue(i + W, buf[w]);
                    const int jj = j_first + i / spl, s = i % spl;
                    const int ex = a.expert_id[jj];
                    const int p = li + s * lpr;
                    const int qa = max(a.seg[jj], q0) - q0, qb = min(a.seg[jj + 1], q1) - q0;
                    float sd[RR];
#pragma unroll
                    for (int rr = 0; rr < RR; ++rr) sd[rr] = a.s_down[(size_t)ex * H + min(rbase + rr, H - 1)];
                    for (int ql = qa; ql < qb; ++ql) {
                        float pr[RR][F];
#pragma unroll
                        for (int rr = 0; rr < RR; ++rr)
#pragma unroll
                            for (int f = 0; f < F; ++f) pr[rr][f] = 0.f;
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            float hv[4 * F];
#pragma unroll
                            for (int m = 0; m < 4 * F; ++m) hv[m] = hs[(ql * CW + 4 * d * F + m) * P + p];
#pragma unroll
                            for (int rr = 0; rr < RR; ++rr) {
                                const uint32_t wd = (d == 0 ? cq[rr].x : d == 1 ? cq[rr].y : d == 2 ? cq[rr].z : cq[rr].w) ^ C::kFlip;
#pragma unroll
                                for (int f = 0; f < F; ++f) {
                                    const uint32_t m = wd & C::mask(f);
                                    pr[rr][f] = fmaf(ubyte_f<0>(m), hv[0 * F + f], pr[rr][f]);
                                    pr[rr][f] = fmaf(ubyte_f<1>(m), hv[1 * F + f], pr[rr][f]);
                                    pr[rr][f] = fmaf(ubyte_f<2>(m), hv[2 * F + f], pr[rr][f]);
                                    pr[rr][f] = fmaf(ubyte_f<3>(m), hv[3 * F + f], pr[rr][f]);
                                }
                            }
                        }
                        const float hoff = C::kOffset * hsum[ql * P + p];
#pragma unroll
                        for (int rr = 0; rr < RR; ++rr) {
                            float v = -hoff;
#pragma unroll
                            for (int f = 0; f < F; ++f) v += C::scale(f) * pr[rr][f];
                            if constexpr (DEFER) {
                                acc[rr] += sd[rr] * v;
                            } else {
                                if constexpr (LPR > 0) v = group_sum<LPR>(v);
                                else v = group_sum_rt(v, lpr);
                                const int r = rbase + rr;
                                if (li == 0 && r < row_end) yacc[(r - row0) * T + qtok[ql]] += sd[rr] * v;
                            }
                        }
                    }
                }
            }
            if constexpr (DEFER) {
#pragma unroll
                for (int rr = 0; rr < RR; ++rr) {
                    float v = acc[rr];
                    if constexpr (LPR > 0) v = group_sum<LPR>(v);
                    else v = group_sum_rt(v, lpr);
                    const int r = rbase + rr;
                    if (li == 0 && r < row_end) yacc[(r - row0) * T] += v;
                }
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nrows * T; i += kThreads) {
        const int t = i / nrows, rl = i - t * nrows;
        y[(size_t)t * H + row0 + rl] = yacc[rl * T + t];
    }
}

// --------------------------------------------------------------------- launch

namespace {

constexpr int kRR = 2;
constexpr int kW = 2;
constexpr int kGuRowsPerWg = 32;
constexpr int kDownRowsPerWg = 16;
constexpr size_t kDownLdsBudget = 80 * 1024;

// Lanes sharing one row: the largest power of two dividing the row's group
// count, at most a wave; each lane then takes P / lanes groups.
int lanes_per_row(int P) {
    const int pow2 = P & (-P);
    return pow2 >= kWave ? kWave : pow2;
}

template <typename Kern>
hipError_t allow_lds(Kern k, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int BITS, int NTMAX>
hipError_t gate_up_bits(const float* x, const ExpertArgs& a, float* h, hipStream_t st) {
    constexpr int CW = 16 * Codec<BITS>::F;
    const int P = (a.H * BITS / 8) / 16;
    const int lpr = lanes_per_row(P);
    const int gpw = kWave / lpr;
    // rows per workgroup: a multiple of the rows covered per iteration
    const int per_iter = kWaves * gpw * kRR;
    const int rows = ((kGuRowsPerWg + per_iter - 1) / per_iter) * per_iter;
    const dim3 grid((a.I + rows - 1) / rows, a.max_active);
    const size_t lds = (size_t)NTMAX * (CW * P + P) * sizeof(float);
    if (lpr == kWave) {
        auto k = gate_up_kernel<BITS, NTMAX, kRR, kWave, kW>;
        hipError_t err = allow_lds(k, lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(k, grid, dim3(kThreads), lds, st, x, a, h, rows, lpr);
    } else {
        auto k = gate_up_kernel<BITS, NTMAX, kRR, 0, kW>;
        hipError_t err = allow_lds(k, lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(k, grid, dim3(kThreads), lds, st, x, a, h, rows, lpr);
    }
    return hipGetLastError();
}

template <int BITS>
hipError_t down_bits(const float* h, const float* topk_w, const ExpertArgs& a, float* y, hipStream_t st) {
    constexpr int CW = 16 * Codec<BITS>::F;
    const int P = (a.I * BITS / 8) / 16;
    const int lpr = lanes_per_row(P);
    const int gpw = kWave / lpr;
    const int per_iter = kWaves * gpw * kRR;
    const int rows = ((kDownRowsPerWg + per_iter - 1) / per_iter) * per_iter;
    const int A = a.T * a.slots;
    const size_t fixed = (size_t)rows * a.T * sizeof(float);
    const size_t per_q = (size_t)(CW * P + P) * sizeof(float) + 2 * sizeof(int);
    int qc = (int)((kDownLdsBudget - fixed) / per_q);
    if (qc < 1) qc = 1;
    if (qc > A) qc = A;
    const size_t lds = fixed + (size_t)qc * per_q;
    const dim3 grid((a.H + rows - 1) / rows);
    const bool defer = a.T == 1;
#define MOEDEC_LAUNCH_DOWN(DEF, L)                                                              \
    do {                                                                                         \
        auto k = down_kernel<BITS, DEF, kRR, L, 4>;                                              \
        hipError_t err = allow_lds(k, lds);                                                      \
        if (err != hipSuccess) return err;                                                       \
        hipLaunchKernelGGL(k, grid, dim3(kThreads), lds, st, h, topk_w, a, y, rows, lpr, qc);   \
    } while (0)
    if (lpr == kWave) {
        if (defer) MOEDEC_LAUNCH_DOWN(true, kWave);
        else MOEDEC_LAUNCH_DOWN(false, kWave);
    } else {
        if (defer) MOEDEC_LAUNCH_DOWN(true, 0);
        else MOEDEC_LAUNCH_DOWN(false, 0);
    }
#undef MOEDEC_LAUNCH_DOWN
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(int bits, const float* x, const ExpertArgs& a, float* h, hipStream_t st) {
    const bool one = a.T == 1;
    switch (bits) {
        case 4: return one ? gate_up_bits<4, 1>(x, a, h, st) : gate_up_bits<4, 2>(x, a, h, st);
        case 8: return one ? gate_up_bits<8, 1>(x, a, h, st) : gate_up_bits<8, 2>(x, a, h, st);
        case 2: return one ? gate_up_bits<2, 1>(x, a, h, st) : gate_up_bits<2, 2>(x, a, h, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_down(int bits, const float* h, const float* topk_w, const ExpertArgs& a, float* y,
                       hipStream_t st) {
    switch (bits) {
        case 4: return down_bits<4>(h, topk_w, a, y, st);
        case 8: return down_bits<8>(h, topk_w, a, y, st);
        case 2: return down_bits<2>(h, topk_w, a, y, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moedec
