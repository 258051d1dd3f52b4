// Router: sigmoid scores, noaux_tc-corrected group-limited top-k, weights, and
// the batch union (worklist) of the selected experts.
//
// Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
// DeepSeek-V3-style sigmoid router with noaux_tc correction,
// routed_scaling_factor and a shared expert; batch-union MoE.  The
// group-score rule (top-2 sum), the use of the corrected score for selection
// only and the tie-breaking (lower index) are this library's reading.
//
// Kernel 1 (router_gemv): one workgroup per expert row; every thread issues all
// of its 16-byte loads of the row before using them, then the row is dotted
// with each token and s = sigmoid(W_r[e] . x_t) is written.
// Kernel 2 (route_select): one workgroup; each wave routes one token at a time
// with the token's scores in registers (a lane holds a contiguous run of
// experts): group top-2 sums by a lane butterfly, topk_group rounds of a wave
// arg-max over groups, top_k rounds over the kept experts, weights from the
// winners' scores passed by lane shuffles; then the workgroup builds the
// expert-ascending worklist with a counting sort.
#include "common.h"

namespace moedec {

namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvMaxF4 = MOEDEC_MAX_DIM / 4 / kGemvThreads;   // float4 per thread
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxEPL = MOEDEC_MAX_EXPERTS / kWave;              // experts per lane

__global__ __launch_bounds__(kGemvThreads) void router_gemv_kernel(const float* __restrict__ x,
                                                                   const float* __restrict__ W, int T, int H,
                                                                   int E, float* __restrict__ scores) {
    __shared__ float red[MOEDEC_MAX_TOKENS][kGemvThreads / kWave];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const float4* w4 = reinterpret_cast<const float4*>(W + (size_t)e * H);
    const int n4 = H >> 2;
    float4 wr[kGemvMaxF4];
#pragma unroll
    for (int k = 0; k < kGemvMaxF4; ++k) {
        const int i = threadIdx.x + k * kGemvThreads;
        wr[k] = i < n4 ? w4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int t = 0; t < T; ++t) {
        const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)t * H);
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < kGemvMaxF4; ++k) {
            const int i = threadIdx.x + k * kGemvThreads;
            if (i < n4) {
                const float4 v = x4[i];
                acc += (wr[k].x * v.x + wr[k].y * v.y) + (wr[k].z * v.z + wr[k].w * v.w);
            }
        }
        acc = group_sum<kWave>(acc);
        if (lane == 0) red[t][wave] = acc;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < T; t += kGemvThreads) {
        const float z = (red[t][0] + red[t][1]) + (red[t][2] + red[t][3]);
        scores[(size_t)t * E + e] = 1.0f / (1.0f + expf(-z));
    }
}

// (v, i) beats (u, j) if v > u, or v == u and i < j.
__device__ __forceinline__ bool beats(float v, int i, float u, int j) { return v > u || (v == u && i < j); }

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float u = __shfl_xor(v, off, kWave);
        const int j = __shfl_xor(i, off, kWave);
        if (beats(u, j, v, i)) { v = u; i = j; }
    }
}

// Merge the top-2 pair (b1 >= b2) into (m1 >= m2).
__device__ __forceinline__ void top2_merge(float& m1, float& m2, float b1, float b2) {
    const float lo = fminf(m1, b1);
    m1 = fmaxf(m1, b1);
    m2 = fmaxf(lo, fmaxf(m2, b2));
}

// Exclusive scan of `v` over the workgroup; returns the prefix, writes the total.
__device__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += u;
    }
    if (lane == kWave - 1) wave_tot[wave] = inc;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < kSelWaves; ++w) {
        if (w < wave) before += wave_tot[w];
        total += wave_tot[w];
    }
    __syncthreads();
    return before + inc - v;
}

__global__ __launch_bounds__(kSelThreads) void route_select_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int T, int E, int n_group, int topk_group,
    int top_k, int n_shared, float rsf, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ wl_n_active, int32_t* __restrict__ wl_expert_id, int32_t* __restrict__ wl_seg,
    int32_t* __restrict__ wl_assign) {
    __shared__ float cs[kSelWaves][MOEDEC_MAX_EXPERTS];
    __shared__ int sel[MOEDEC_MAX_TOKENS * 32];
    __shared__ int cnt[MOEDEC_MAX_EXPERTS + 8];
    __shared__ int ea[MOEDEC_MAX_TOKENS * 40];
    __shared__ int start[MOEDEC_MAX_EXPERTS + 8];
    __shared__ int wave_tot[kSelWaves];

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int per = E / n_group;
    const int epl = (E + kWave - 1) / kWave;
    const int lpg = per / epl;            // lanes per group on the butterfly path
    const bool butterfly = (per % epl == 0) && ((lpg & (lpg - 1)) == 0) && lpg <= kWave;
    const int e0 = lane * epl;            // this lane's experts: e0 .. e0 + epl - 1

    for (int t = wave; t < T; t += kSelWaves) {
        const float* st = scores + (size_t)t * E;
        float sv[kMaxEPL], cv[kMaxEPL];
#pragma unroll
        for (int i = 0; i < kMaxEPL; ++i) {
            const int e = e0 + i;
            const bool ok = i < epl && e < E;
            sv[i] = ok ? st[e] : 0.f;
            cv[i] = ok ? sv[i] + bias[e] : -INFINITY;
        }
        // group score: largest plus second largest corrected score of the group
        float gs = -INFINITY;
        int gid = 0x7fffffff;
        if (butterfly) {
            float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
            for (int i = 0; i < kMaxEPL; ++i) top2_merge(m1, m2, cv[i], -INFINITY);
            for (int off = 1; off < lpg; off <<= 1) {
                const float b1 = __shfl_xor(m1, off, kWave), b2 = __shfl_xor(m2, off, kWave);
                top2_merge(m1, m2, b1, b2);
            }
            if (e0 < E && (lane % lpg) == 0) {
                gs = m1 + m2;
                gid = e0 / per;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kMaxEPL; ++i)
                if (i < epl && e0 + i < E) cs[wave][e0 + i] = cv[i];
            __threadfence_block();
            if (lane < n_group) {
                float m1 = -INFINITY, m2 = -INFINITY;
                for (int k = 0; k < per; ++k) top2_merge(m1, m2, cs[wave][lane * per + k], -INFINITY);
                gs = m1 + m2;
                gid = lane;
            }
        }
        // keep topk_group groups (ties: lower group)
        uint64_t kept = 0;
        for (int r = 0; r < topk_group; ++r) {
            float v = gs;
            int g = gid;
            wave_argmax(v, g);
            kept |= 1ull << g;
            if (gid == g) gs = -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < kMaxEPL; ++i) {
            const int e = e0 + i;
            if (i < epl && e < E && !((kept >> (e / per)) & 1ull)) cv[i] = -INFINITY;
        }
        // top_k rounds of an arg-max over (c, -index); weights from unbiased scores
        int mine = 0;
        float mine_s = 0.f, total = 0.f;
        for (int k = 0; k < top_k; ++k) {
            float v = -INFINITY;
            int ie = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < kMaxEPL; ++i)
                if (i < epl && beats(cv[i], e0 + i, v, ie)) { v = cv[i]; ie = e0 + i; }
            wave_argmax(v, ie);
            const int owner = ie / epl, slot = ie - owner * epl;
            float s_here = 0.f;
#pragma unroll
            for (int i = 0; i < kMaxEPL; ++i)
                if (i == slot) s_here = sv[i];
            const float s_win = __shfl(s_here, owner, kWave);
            if (lane == owner) {
#pragma unroll
                for (int i = 0; i < kMaxEPL; ++i)
                    if (i == slot) cv[i] = -INFINITY;
            }
            total += s_win;                      // slot order
            if (lane == k) { mine = ie; mine_s = s_win; }
        }
        if (lane < top_k) {
            topk_idx[t * top_k + lane] = mine;
            topk_w[t * top_k + lane] = (mine_s / total) * rsf;
            sel[t * top_k + lane] = mine;
        }
    }
    if (wl_n_active == nullptr) return;
    __syncthreads();

    // batch union: counting sort of the assignments by expert
    const int slots = top_k + n_shared;
    const int A = T * slots;
    const int NE = E + n_shared;
    for (int i = threadIdx.x; i < NE; i += kSelThreads) cnt[i] = 0;
    for (int a = threadIdx.x; a < A; a += kSelThreads) {
        const int t = a / slots, s = a - t * slots;
        ea[a] = s < top_k ? sel[t * top_k + s] : E + (s - top_k);
    }
    __syncthreads();
    for (int a = threadIdx.x; a < A; a += kSelThreads) atomicAdd(&cnt[ea[a]], 1);
    __syncthreads();
    // per-thread contiguous run of experts, then a workgroup scan
    const int chunk = (NE + kSelThreads - 1) / kSelThreads;
    const int x0 = threadIdx.x * chunk;
    int my_cnt = 0, my_act = 0;
    for (int e = x0; e < min(NE, x0 + chunk); ++e) {
        my_cnt += cnt[e];
        my_act += cnt[e] > 0;
    }
    int tot_cnt, tot_act;
    int cnt_before = block_exclusive_scan(my_cnt, wave_tot, tot_cnt);
    int act_before = block_exclusive_scan(my_act, wave_tot, tot_act);
    for (int e = x0; e < min(NE, x0 + chunk); ++e) {
        start[e] = cnt_before;
        if (cnt[e] > 0) {
            wl_expert_id[act_before] = e;
            wl_seg[act_before] = cnt_before;
            ++act_before;
        }
        cnt_before += cnt[e];
    }
    if (threadIdx.x == 0) {
        *wl_n_active = tot_act;
        wl_seg[tot_act] = tot_cnt;
    }
    __syncthreads();
    for (int a = threadIdx.x; a < A; a += kSelThreads) {
        const int e = ea[a];
        int r = 0;
        for (int b = 0; b < a; ++b) r += ea[b] == e;
        wl_assign[start[e] + r] = a;
    }
}

}  // namespace

hipError_t launch_route(const float* x, const float* router_w, const float* bias, int T, int H, int E,
                        int n_group, int topk_group, int top_k, int n_shared, float rsf, float* scores,
                        int32_t* topk_idx, float* topk_w, const moedec_worklist* wl, hipStream_t st) {
    hipLaunchKernelGGL(router_gemv_kernel, dim3(E), dim3(kGemvThreads), 0, st, x, router_w, T, H, E, scores);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_select_kernel, dim3(1), dim3(kSelThreads), 0, st, scores, bias, T, E, n_group,
                       topk_group, top_k, n_shared, rsf, topk_idx, topk_w, wl ? wl->n_active : nullptr,
                       wl ? wl->expert_id : nullptr, wl ? wl->seg : nullptr, wl ? wl->assign : nullptr);
    return hipGetLastError();
}

}  // namespace moedec
