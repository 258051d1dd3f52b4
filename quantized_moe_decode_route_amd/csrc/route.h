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

#include <climits>

#include "common.h"

namespace moedec {

// LDS of route_select_block for batches of up to TM tokens, EM routed experts
// and NW waves (top_k <= 32, n_group <= 64, n_shared <= 8).
template <int TM, int EM, int NW>
struct RouteLdsT {
    int sel[TM * 32];                      // chosen experts [T][K], slot order
    float selw[TM * 32];                   // their weights
    float c[NW][EM];                       // each wave's token: corrected scores
    float gs[NW][64];                      //   and group scores
    int key[TM * 40];                      // assignment sort keys, then "new expert starts here"
    int sexp[TM * 40];                     // expert of each sorted position
    int eid[EM + 8];                       // worklist: unique experts ascending
    int seg[EM + 9];                       //           offsets into assign
    int assign[TM * 40];                   //           assignments by expert
    int n_active;
    int n_assign;                          // assignments (dropped top-p slots have none)
};

// n / d for 0 <= n < 4096 and 1 <= d <= 64 from one float product: (n + 1/2) / d
// lies at least 1/128 from an integer, and the product's rounding moves it by
// under 2^-11 (checked for every such n and d).
__device__ __forceinline__ int small_quot(int n, float inv_d) { return (int)(((float)n + 0.5f) * inv_d); }

// (v, i) beats (u, j) if v > u, or v == u and i < j: a strict total order.
__device__ __forceinline__ bool beats(float v, int i, float u, int j) { return v > u || (v == u && i < j); }

// Orders one wave's LDS writes before its later LDS reads (LDS serves a wave
// in issue order; this keeps the compiler from reordering across it).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One token's group-limited top-k (wave-wide operations only; the whole wave
// calls this).  NVT experts per lane, contiguous: lane l holds experts
// l*NVT .. l*NVT + NVT - 1, so the lowest lane holding the round's largest
// key also holds the lowest expert index among those with that key.
template <int NVT, int TM, int EM, int NW, bool kCoherentScores, bool kTopP>
__device__ __forceinline__ void route_one_token(const float* scores, const float* __restrict__ bias, int t, int E,
                                                int n_group, int topk_group, int top_k, float rsf, float top_p,
                                                RouteLdsT<TM, EM, NW>& r) {
    static_assert(NVT <= 32, "the candidate mask is 32 bits");
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int per = E / n_group;
    float* cw = r.c[wave];
    float cl[NVT], sl[NVT], bl[NVT];
#pragma unroll
    for (int j = 0; j < NVT; ++j) {                    // every load first (clamped index), then use
        const int e = min(lane * NVT + j, E - 1);
        if constexpr (kCoherentScores)
            sl[j] = __int_as_float(__hip_atomic_load(reinterpret_cast<const int*>(scores + (size_t)t * E + e),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        else
            sl[j] = scores[(size_t)t * E + e];
        bl[j] = bias[e];
    }
    unsigned live = 0;                                 // bit j: expert lane * NVT + j exists
#pragma unroll
    for (int j = 0; j < NVT; ++j) {
        const float v = sl[j] + bl[j];
        cl[j] = v == v ? v : -INFINITY;
        if (lane * NVT + j < E) live |= 1u << j;
    }
    // Group scores.  When a group fills whole lanes (per = lpg * NVT, lpg a
    // power of two <= 16), each lane's top two are merged over its group's
    // lanes by DPP (xor 1, xor 2, half-row mirror, row mirror) and the ranks
    // come from lane reads; otherwise lane g < n_group scans group g in LDS.
    const int lpg = per / NVT;
    const bool lane_groups = per % NVT == 0 && lpg <= 16 && (lpg & (lpg - 1)) == 0;
    unsigned long long kept = 0;                       // bit g: group g kept (LDS form)
    bool kept_mine = false;                            // this lane's group kept (lane form)
    if (lane_groups) {
        float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            const float v = ((live >> j) & 1u) ? cl[j] : -INFINITY;
            m2 = fmaxf(m2, fminf(m1, v));
            m1 = fmaxf(m1, v);
        }
        auto merge = [&](float b1, float b2) {
            const float n2 = fmaxf(fminf(m1, b1), fmaxf(m2, b2));
            m1 = fmaxf(m1, b1);
            m2 = n2;
        };
        if (lpg >= 2) merge(dpp_f<0xB1>(m1), dpp_f<0xB1>(m2));
        if (lpg >= 4) merge(dpp_f<0x4E>(m1), dpp_f<0x4E>(m2));
        if (lpg >= 8) merge(dpp_f<0x141>(m1), dpp_f<0x141>(m2));
        if (lpg >= 16) merge(dpp_f<0x140>(m1), dpp_f<0x140>(m2));
        const float gsum = m1 + m2;                     // NaN only from +inf + -inf
        const float gsv = gsum == gsum ? gsum : -INFINITY;
        const int g = lane / lpg;
        int grank = 0;
        for (int h = 0; h < n_group; ++h)
            grank += beats(bits_f(__builtin_amdgcn_readlane(f_bits(gsv), h * lpg)), h, gsv, g);
        kept_mine = g < n_group && grank < topk_group;
    } else {
#pragma unroll
        for (int j = 0; j < NVT; ++j)
            if ((live >> j) & 1u) cw[lane * NVT + j] = cl[j];
        wave_lds_sync();
        float gsv = -INFINITY;
        if (lane < n_group) {
            float m1 = -INFINITY, m2 = -INFINITY;
            const float* cg = cw + lane * per;
#pragma unroll 8
            for (int k = 0; k < per; ++k) {            // branch-free, so the reads issue back to back
                const float v = cg[k];
                m2 = fmaxf(m2, fminf(m1, v));
                m1 = fmaxf(m1, v);
            }
            const float gsum = m1 + m2;                 // NaN only from +inf + -inf
            gsv = gsum == gsum ? gsum : -INFINITY;
            r.gs[wave][lane] = gsv;
        }
        wave_lds_sync();
        int grank = 0;
        if (lane < n_group) {
#pragma unroll 8
            for (int h = 0; h < n_group; ++h) grank += beats(r.gs[wave][h], h, gsv, lane);
        }
        kept = __ballot(lane < n_group && grank < topk_group);
    }
    // Candidates as order-preserving 32-bit keys of c (+0 for -0, so equal
    // values tie and go by index); 0 (below -inf's key) marks an expert
    // that is not, or no longer, a candidate.
    const float inv_per = 1.0f / (float)per;
    unsigned key[NVT];
#pragma unroll
    for (int j = 0; j < NVT; ++j) {
        const int e = lane * NVT + j;
        int g = (int)((float)e * inv_per);              // e / per, then corrected
        g += (g + 1) * per <= e;
        g -= g * per > e;
        const unsigned u = __float_as_uint(cl[j] + 0.0f);
        const unsigned ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        const bool in_kept = lane_groups ? kept_mine : (bool)((kept >> min(g, 63)) & 1ull);
        key[j] = (((live >> j) & 1u) && in_kept) ? ord : 0u;
    }
    // round k: each lane's best (largest key, lowest j on ties), the wave's
    // largest key, then the lowest lane holding it (= the lowest expert index)
    float total = 0.f, my_s = 0.f;
    int my_e = 0;
    if constexpr (NVT == 4) {
        // the lane's four candidates sorted once by (key descending, j
        // ascending); a round takes every lane's head and the owner's list
        // moves up by one
        unsigned k0 = key[0], k1 = key[1], k2 = key[2], k3 = key[3];
        int j0 = 0, j1 = 1, j2 = 2, j3 = 3;
        float s0 = sl[0], s1 = sl[1], s2 = sl[2], s3 = sl[3];
        auto order = [](unsigned& ka, int& ja, float& sa, unsigned& kb, int& jb, float& sb) {
            const bool sw = kb > ka || (kb == ka && jb < ja);
            const unsigned kt = ka;
            const int jt = ja;
            const float st = sa;
            ka = sw ? kb : ka;
            ja = sw ? jb : ja;
            sa = sw ? sb : sa;
            kb = sw ? kt : kb;
            jb = sw ? jt : jb;
            sb = sw ? st : sb;
        };
        order(k0, j0, s0, k1, j1, s1);
        order(k2, j2, s2, k3, j3, s3);
        order(k0, j0, s0, k2, j2, s2);
        order(k1, j1, s1, k3, j3, s3);
        order(k1, j1, s1, k2, j2, s2);
        for (int k = 0; k < top_k; ++k) {
            const unsigned m = wave_max_u(k0);
            const int owner = (int)__builtin_ctzll(__ballot(k0 == m));    // top_k <= candidates: m > 0
            const int win = owner * NVT + __builtin_amdgcn_readlane(j0, owner);
            const float sw = bits_f(__builtin_amdgcn_readlane(f_bits(s0), owner));
            if (lane == owner) {
                k0 = k1;
                j0 = j1;
                s0 = s1;
                k1 = k2;
                j1 = j2;
                s1 = s2;
                k2 = k3;
                j2 = j3;
                s2 = s3;
                k3 = 0u;
            }
            if (lane == 0) r.sel[t * top_k + k] = win;
            if (lane == k) {
                my_s = sw;
                my_e = win;
            }
            total += sw;                               // slot order
        }
    } else {
        for (int k = 0; k < top_k; ++k) {
            unsigned bk = key[NVT - 1];
            int bj = NVT - 1;
            float bs = sl[NVT - 1];
#pragma unroll
            for (int j = NVT - 2; j >= 0; --j) {
                const bool better = key[j] >= bk;
                bk = better ? key[j] : bk;
                bj = better ? j : bj;
                bs = better ? sl[j] : bs;
            }
            const unsigned m = wave_max_u(bk);
            const int owner = (int)__builtin_ctzll(__ballot(bk == m));    // top_k <= candidates: m > 0
            const int win = owner * NVT + __builtin_amdgcn_readlane(bj, owner);
            const float sw = bits_f(__builtin_amdgcn_readlane(f_bits(bs), owner));
            const bool mine = lane == owner;
#pragma unroll
            for (int j = 0; j < NVT; ++j) key[j] = (mine && j == bj) ? 0u : key[j];
            if (lane == 0) r.sel[t * top_k + k] = win;
            if (lane == k) {
                my_s = sw;
                my_e = win;
            }
            total += sw;                               // slot order
        }
    }
    if (!kTopP || !(top_p < 1.f)) {
        if (lane < top_k) r.selw[t * top_k + lane] = (my_s / total) * rsf;
        return;
    }
    // adaptive top-p: rank of slot `lane` by (s descending, NaN last, index)
    const unsigned us = __float_as_uint(my_s + 0.0f);
    const unsigned ks = my_s == my_s ? ((us & 0x80000000u) ? ~us : (us | 0x80000000u)) : 0u;
    int wr = 0;
    for (int j = 0; j < top_k; ++j) {
        const unsigned kj = __builtin_amdgcn_readlane(ks, j);
        const int ej = __builtin_amdgcn_readlane(my_e, j);
        wr += (kj > ks) || (kj == ks && ej < my_e);
    }
    const float thr = top_p * total;
    float cum = 0.f;
    int m = top_k;
    for (int i = 0; i < top_k; ++i) {                  // the ranks are a permutation of 0 .. top_k-1
        const int ln = (int)__builtin_ctzll(__ballot(lane < top_k && wr == i));
        cum += bits_f(__builtin_amdgcn_readlane(f_bits(my_s), ln));
        if (cum >= thr) {
            m = i + 1;
            break;
        }
    }
    const bool keep = lane < top_k && wr < m;
    const unsigned long long kb = __ballot(keep);
    float kept_total = 0.f;
    for (int j = 0; j < top_k; ++j)                    // slot order
        if ((kb >> j) & 1ull) kept_total += bits_f(__builtin_amdgcn_readlane(f_bits(my_s), j));
    // rewrite the token's slots (LDS writes of one wave land in order)
    const int ns = __popcll(kb & ((1ull << lane) - 1ull));
    if (keep) {
        r.sel[t * top_k + ns] = my_e;
        r.selw[t * top_k + ns] = (my_s / kept_total) * rsf;
    }
    if (lane >= m && lane < top_k) {
        r.sel[t * top_k + lane] = -1;
        r.selw[t * top_k + lane] = 0.f;
    }
}

// The batch union of the selections in r.sel (every token's top_k slots):
// a rank sort of the assignments by (expert, assignment index) into the
// worklist in LDS.  The whole workgroup calls this (with A <= 64 one wave
// does the work: wave 0, or the last wave with kLastWaves).
template <int TM, int EM, int NW, bool kTopP = false, bool kLastWaves = false>
__device__ __forceinline__ void route_union_block(int T, int E, int top_k, int n_shared, RouteLdsT<TM, EM, NW>& r) {
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    const int wave = kLastWaves ? nwaves - 1 - (int)(threadIdx.x / kWave) : (int)(threadIdx.x / kWave);
    const int slots = top_k + n_shared;
    const int A = T * slots;
    if (A <= kWave) {                  // one wave, no workgroup barriers
        if (wave == 0) {                // (the last wave with kLastWaves)
            int k = INT_MAX;                   // a dropped slot keeps INT_MAX: sorted last, not written
            if (lane < A) {
                const int tt = lane / slots, s = lane - tt * slots;
                const int e = s < top_k ? r.sel[tt * top_k + s] : E + (s - top_k);
                k = e >= 0 ? (e << 16) | lane : INT_MAX;
                r.key[lane] = k;
            }
            wave_lds_sync();
            int rank = 0;
            for (int b = 0; b < A; ++b) rank += r.key[b] < k;
            const bool valid = lane < A && (!kTopP || k != INT_MAX);
            const int Av = kTopP ? __popcll(__ballot(valid)) : A;
            if (valid) {
                r.assign[rank] = lane;
                r.sexp[rank] = k >> 16;
            }
            wave_lds_sync();
            const int ex = lane < Av ? r.sexp[lane] : -1;
            const bool first = lane < Av && (lane == 0 || r.sexp[max(lane - 1, 0)] != ex);
            const unsigned long long fm = __ballot(first);
            const int sidx = __popcll(fm & ((1ull << lane) - 1ull));
            if (first) {
                r.eid[sidx] = ex;
                r.seg[sidx] = lane;
            }
            if (lane == 0) {
                const int n = __popcll(fm);
                r.n_active = n;
                r.n_assign = Av;
                r.seg[n] = Av;
            }
        }
        __syncthreads();
        return;
    }
    for (int a = threadIdx.x; a < A; a += blockDim.x) {
        const int t = a / slots, s = a - t * slots;
        const int e = s < top_k ? r.sel[t * top_k + s] : E + (s - top_k);
        r.key[a] = (!kTopP || e >= 0) ? (e << 16) | a : INT_MAX;   // dropped top-p slot: sorted last, not written
    }
    __syncthreads();
    for (int a = threadIdx.x; a < A; a += blockDim.x) {
        const int k = r.key[a];
        if (kTopP && k == INT_MAX) continue;
        int rank = 0;
#pragma unroll 8
        for (int b = 0; b < A; ++b) rank += r.key[b] < k;
        r.assign[rank] = a;
        r.sexp[rank] = k >> 16;
    }
    if (threadIdx.x == 0) {
        int n = A;
        if (kTopP)
            for (int a = 0; a < A; ++a) n -= r.key[a] == INT_MAX;
        r.n_assign = n;
    }
    __syncthreads();
    const int Av = r.n_assign;
    int* first = r.key;                  // the keys are no longer needed
    for (int p = threadIdx.x; p < Av; p += blockDim.x)
        first[p] = (p == 0 || r.sexp[p - 1] != r.sexp[p]) ? 1 : 0;
    __syncthreads();
    for (int p = threadIdx.x; p < Av; p += blockDim.x) {
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
        for (int p = 0; p < Av; ++p) n += first[p];
        r.n_active = n;
        r.seg[n] = Av;
    }
    __syncthreads();
}

// The same batch union by a counting sort, for up to 64 tokens; the whole
// workgroup calls this.  Bin b (routed expert b, or shared expert b - E)
// gets the bit mask of the tokens that chose it; the bins' sizes and their
// prefix sums give the segments, and assignment a of token t lands at its
// bin's offset plus the number of earlier tokens in the bin.  Within a bin
// that is the order of the assignment index, since a token picks each expert
// at most once, so the result equals the rank sort's.
template <int TM, int EM, int NW, bool kTopP = false>
__device__ __forceinline__ void route_union_counting(int T, int E, int top_k, int n_shared,
                                                     RouteLdsT<TM, EM, NW>& r) {
    static_assert(TM <= 64, "token masks are 64 bits");
    static_assert(sizeof(r.key) >= (EM + 8) * sizeof(unsigned long long), "bin masks alias the sort keys");
    static_assert(sizeof(r.sexp) >= (EM + 8) * sizeof(int), "bin offsets alias the sorted experts");
    static_assert(sizeof(r.gs) >= 2 * NW * sizeof(int), "wave totals alias the group scores");
    unsigned long long* m = reinterpret_cast<unsigned long long*>(r.key);
    int* base = r.sexp;
    int* wtot = reinterpret_cast<int*>(&r.gs[0][0]);   // [0, nw): sizes, [nw, 2 nw): non-empty bins
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int nw = nt / kWave;
    const int nb = E + n_shared, slots = top_k + n_shared;
    const unsigned long long all = T >= 64 ? ~0ull : (1ull << T) - 1ull;
    for (int b = tid; b < nb; b += nt) m[b] = b < E ? 0ull : all;   // every token takes each shared expert
    __syncthreads();
    const float inv_k = 1.0f / (float)top_k, inv_slots = 1.0f / (float)slots;
    for (int i = tid; i < T * top_k; i += nt) {
        const int e = r.sel[i];
        if (!kTopP || e >= 0) atomicOr(m + e, 1ull << small_quot(i, inv_k));
    }
    __syncthreads();
    // thread i owns bins i*pb .. i*pb+pb-1: their sizes, then block prefix sums
    const int pb = (nb + nt - 1) / nt, b0 = tid * pb;
    int cnt = 0, act = 0;
    for (int j = 0; j < pb; ++j) {
        const int b = b0 + j;
        if (b < nb) {
            const int c = __popcll(m[b]);
            cnt += c;
            act += c != 0;
        }
    }
    int ic = wave_scan_incl(cnt), ia = wave_scan_incl(act);   // inclusive scans within the wave
    if (lane == kWave - 1) {
        wtot[wave] = ic;
        wtot[nw + wave] = ia;
    }
    __syncthreads();
    for (int w = 0; w < wave; ++w) {
        ic += wtot[w];
        ia += wtot[nw + w];
    }
    int pos = ic - cnt, k = ia - act;
    for (int j = 0; j < pb; ++j) {
        const int b = b0 + j;
        if (b < nb) {
            const int c = __popcll(m[b]);
            base[b] = pos;
            if (c != 0) {
                r.eid[k] = b;
                r.seg[k] = pos;
                ++k;
            }
            pos += c;
        }
    }
    if (tid == nt - 1) {                             // its inclusive sums are the totals
        r.n_active = ia;
        r.n_assign = ic;
        r.seg[ia] = ic;
    }
    __syncthreads();
    for (int a = tid; a < T * slots; a += nt) {
        const int t = small_quot(a, inv_slots), s = a - t * slots;
        const int e = s < top_k ? r.sel[t * top_k + s] : E + (s - top_k);
        if (!kTopP || e >= 0) r.assign[base[e] + __popcll(m[e] & ((1ull << t) - 1ull))] = a;
    }
    __syncthreads();
}

// Route T tokens whose sigmoid scores are in global memory (s[t][e]) and build
// the batch union, all in LDS `r`; the whole workgroup (NW waves) calls this.
// Each wave routes its own tokens with wave-wide operations only (no
// workgroup barrier per token):
//   1. lane l holds experts l*NV .. l*NV+NV-1: s, and c = s + bias (also to
//      LDS); NV is 4 when E <= 256, else EM / 64;
//   2. lane g < n_group: group score = largest + second largest c of group g;
//   3. lane g: rank among the group scores; kept if rank < topk_group;
//   4. top_k rounds of a wave arg-max over the kept groups' experts, by
//      (c descending, index ascending), on order-preserving integer keys of
//      c -- branch-free selects, DPP and lane reads, no LDS round trips;
//      round k's winner is slot k, and the total of the chosen s is summed
//      in slot order as the rounds go;
//   5. lane k < top_k: weight k = s_k / total * rsf.
// With top_p < 1 (adaptive expert top-p; Show HN page, run options), step 5
// becomes: rank the slots by s (descending, NaN last, ties to the lower
// index), add s in that order until the sum reaches top_p * total, keep that
// prefix (at least one slot), move the kept slots to the front in their slot
// order, weight them s_k / (their slot-order sum) * rsf, and mark the rest
// index -1, weight 0 -- such slots get no assignment.
// The worklist is then a rank sort of the assignments by (expert, assignment)
// (one wave when they fit its lanes, else the whole workgroup).
// A NaN corrected score or group score ranks below every number (as -inf,
// ties by index), so every slot gets a distinct valid expert whatever the
// inputs hold.
// kCoherentScores: read the scores with device-coherent loads (scores that
// other workgroups of the same launch have just written), else plain loads.
// kTopP: compile the top-p step in (top_p is read only then; without it the
// selection is plain top-k and the code stays as small as before).
// kLastWaves: token t is routed by wave NW-1-(t % NW) and a one-wave union
// runs on wave NW-1, so the first waves issue no loads here (their own
// loads, already in flight, are not waited for).
template <int TM, int EM, int NW, bool kCoherentScores = false, bool kTopP = false, bool kLastWaves = false>
__device__ __forceinline__ void route_select_block(const float* scores, const float* __restrict__ bias, int T,
                                                   int E, int n_group, int topk_group, int top_k, int n_shared,
                                                   float rsf, float top_p, RouteLdsT<TM, EM, NW>& r) {
    constexpr int NV = EM / kWave;                    // experts per lane at most
    constexpr int NV4 = NV < 4 ? NV : 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    const int wave = kLastWaves ? nwaves - 1 - (int)(threadIdx.x / kWave) : (int)(threadIdx.x / kWave);
    for (int t = wave; t < T; t += nwaves) {
        if (NV == NV4 || E <= NV4 * kWave)
            route_one_token<NV4, TM, EM, NW, kCoherentScores, kTopP>(scores, bias, t, E, n_group, topk_group, top_k,
                                                                    rsf, top_p, r);
        else
            route_one_token<NV, TM, EM, NW, kCoherentScores, kTopP>(scores, bias, t, E, n_group, topk_group, top_k,
                                                                   rsf, top_p, r);
    }
    __syncthreads();
    route_union_block<TM, EM, NW, kTopP, kLastWaves>(T, E, top_k, n_shared, r);
}

}  // namespace moedec
