// Routing device code shared by the route_select kernel and the fused layer
// kernel: group-limited top-k from sigmoid scores and the batch union.
//
// Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
// DeepSeek-V3-style sigmoid router (noaux_tc correction, routed_scaling_factor,
// shared expert) and batch-union MoE.  Readings: a group's score is the sum of
// its two largest corrected scores c = s + bias; c selects groups and experts,
// the unbiased s weighs them; ties go to the lower index; weights are
// (s_k / sum over the chosen s in slot order) * routed_scaling_factor.
#pragma once

#include "common.h"

namespace moedec {

// LDS of route_select_block for batches of up to TM tokens and EM routed
// experts (top_k <= 32, n_group <= 64, n_shared <= 8).
template <int TM, int EM>
struct RouteLdsT {
    int sel[TM * 32];                      // chosen experts [T][K], slot order
    float selw[TM * 32];                   // their weights
    float c[EM];                           // one token's corrected scores
    float s[EM];                           //   and sigmoid scores
    int cand[EM];                          //   candidates: at kept group rank * min(per, K) + rank in group,
    float cand_c[EM];                      //   with their corrected and sigmoid scores
    float cand_s[EM];
    float gs[64];                          //   group scores
    int gslot[64];                         //   rank of a kept group among the groups, else -1
    float ws[32];                          //   chosen experts' sigmoid scores, slot order
    int key[TM * 40];                      // assignment sort keys, then "new expert starts here"
    int sexp[TM * 40];                     // expert of each sorted position
    int eid[EM + 8];                       // worklist: unique experts ascending
    int seg[EM + 9];                       //           offsets into assign
    int assign[TM * 40];                   //           assignments by expert
    int n_active;
};
using RouteLds = RouteLdsT<MOEDEC_MAX_TOKENS, MOEDEC_MAX_EXPERTS>;

// (v, i) beats (u, j) if v > u, or v == u and i < j: a strict total order.
__device__ __forceinline__ bool beats(float v, int i, float u, int j) { return v > u || (v == u && i < j); }

// Route T tokens whose sigmoid scores are in global memory (s[t][e]) and build
// the batch union, all in LDS `r`; the whole workgroup calls this (any
// multiple of 64 threads) and every
// selection is a rank count, so no step waits on a serial chain of rounds:
//   1. thread per expert: c = s + bias into LDS;
//   2. thread per group: score = largest + second largest c of the group;
//   3. thread per group: rank among the group scores; kept if rank < topk_group;
//   4. thread per expert of a kept group: rank within its group; only the
//      group's top min(per, top_k) can be among the token's top_k, so they are
//      the candidates, placed without atomics at (group rank, rank in group);
//   5. thread per candidate: rank among all candidates = its slot if < top_k;
//   6. thread per slot: weight = s / (sum of the chosen s in slot order) * rsf.
// The worklist is then a rank sort of the assignments by (expert, assignment).
// A NaN corrected score or group score ranks below every number (as -inf,
// ties by index), so the ranks are always permutations and every slot gets a
// valid expert whatever the inputs hold.
template <int TM, int EM>
__device__ void route_select_block(const float* scores, const float* __restrict__ bias, int T, int E,
                                   int n_group, int topk_group, int top_k, int n_shared, float rsf,
                                   RouteLdsT<TM, EM>& r) {
    const int nthr = blockDim.x;
    const int per = E / n_group;
    const int kg = per < top_k ? per : top_k;        // candidates per kept group
    const int n_cand = topk_group * kg;
    for (int t = 0; t < T; ++t) {
        const float* st = scores + (size_t)t * E;
        for (int e = threadIdx.x; e < E; e += nthr) {
            const float sv = st[e];
            const float cv = sv + bias[e];
            r.s[e] = sv;
            r.c[e] = cv == cv ? cv : -INFINITY;
        }
        __syncthreads();
        for (int g = threadIdx.x; g < n_group; g += nthr) {
            float m1 = -INFINITY, m2 = -INFINITY;
            const float* cg = r.c + g * per;
#pragma unroll 8
            for (int k = 0; k < per; ++k) {          // branch-free, so the reads issue back to back
                const float v = cg[k];
                m2 = fmaxf(m2, fminf(m1, v));
                m1 = fmaxf(m1, v);
            }
            const float gsum = m1 + m2;                 // NaN only from +inf + -inf
            r.gs[g] = gsum == gsum ? gsum : -INFINITY;
        }
        __syncthreads();
        for (int g = threadIdx.x; g < n_group; g += nthr) {
            const float v = r.gs[g];
            int rank = 0;
#pragma unroll 8
            for (int h = 0; h < n_group; ++h) rank += beats(r.gs[h], h, v, g);
            r.gslot[g] = rank < topk_group ? rank : -1;   // kept groups get distinct slots
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += nthr) {
            const int g = e / per;
            const int gsl = r.gslot[g];
            if (gsl >= 0) {
                const float v = r.c[e];
                const float* cg = r.c + g * per;
                int rank = 0;
#pragma unroll 8
                for (int k = 0; k < per; ++k) rank += beats(cg[k], g * per + k, v, e);
                if (rank < kg) {
                    r.cand[gsl * kg + rank] = e;
                    r.cand_c[gsl * kg + rank] = v;
                    r.cand_s[gsl * kg + rank] = r.s[e];
                }
            }
        }
        __syncthreads();
        for (int q = threadIdx.x; q < n_cand; q += nthr) {
            const int e = r.cand[q];
            const float v = r.cand_c[q];
            int rank = 0;
#pragma unroll 8
            for (int p = 0; p < n_cand; ++p) rank += beats(r.cand_c[p], r.cand[p], v, e);
            if (rank < top_k) {
                r.sel[t * top_k + rank] = e;
                r.ws[rank] = r.cand_s[q];
            }
        }
        __syncthreads();
        if ((int)threadIdx.x < top_k) {
            float total = 0.f;
            for (int k = 0; k < top_k; ++k) total += r.ws[k];   // slot order
            r.selw[t * top_k + threadIdx.x] = (r.ws[threadIdx.x] / total) * rsf;
        }
        __syncthreads();
    }
    __syncthreads();

    // batch union: rank sort of the assignments by (expert, assignment index)
    const int slots = top_k + n_shared;
    const int A = T * slots;
    for (int a = threadIdx.x; a < A; a += blockDim.x) {
        const int t = a / slots, s = a - t * slots;
        const int e = s < top_k ? r.sel[t * top_k + s] : E + (s - top_k);
        r.key[a] = (e << 16) | a;
    }
    __syncthreads();
    for (int a = threadIdx.x; a < A; a += blockDim.x) {
        const int k = r.key[a];
        int rank = 0;
#pragma unroll 8
        for (int b = 0; b < A; ++b) rank += r.key[b] < k;
        r.assign[rank] = a;
        r.sexp[rank] = k >> 16;
    }
    __syncthreads();
    int* first = r.key;                  // the keys are no longer needed
    for (int p = threadIdx.x; p < A; p += blockDim.x)
        first[p] = (p == 0 || r.sexp[p - 1] != r.sexp[p]) ? 1 : 0;
    __syncthreads();
    for (int p = threadIdx.x; p < A; p += blockDim.x) {
        if (first[p]) {
            int sidx = 0;
#pragma unroll 8
            for (int q = 0; q < p; ++q) sidx += first[q];
            r.eid[sidx] = r.sexp[p];
            r.seg[sidx] = p;
        }
    }
    if (threadIdx.x == 0) {
        int n = 0;
#pragma unroll 8
        for (int p = 0; p < A; ++p) n += first[p];
        r.n_active = n;
        r.seg[n] = A;
    }
    __syncthreads();
}

}  // namespace moedec
