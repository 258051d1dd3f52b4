// Router: sigmoid scores, noaux_tc-corrected group-limited top-k, weights, and
// the batch union (worklist) of the selected experts.
//
// Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
// DeepSeek-V3-style sigmoid router with noaux_tc correction,
// routed_scaling_factor and a shared expert; batch-union MoE.  The
// group-score rule (top-2 sum), the use of the corrected score for selection
// only and the tie-breaking (lower index) are this library's reading.
//
// Kernel 1 (router_gemv): an 8-wave workgroup per tile of EB expert rows and
// TB tokens, so each workgroup reads EB + TB rows of H floats (a one-row
// workgroup would read the row and every token's x); s = sigmoid(W_r[e] . x_t).
// A split over the hidden dimension would read every row once, but needs
// scratch space the call does not have.
// Kernel 2 (route_tokens): one one-wave workgroup per token routes it with
// wave-wide arg-max rounds (route_one_token, see route.h); the last
// workgroup to finish builds the expert-ascending worklist by a counting sort
// in LDS (route_union_counting).
#include "route.h"

namespace moedec {

namespace {

constexpr int kGemvThreads = 512;
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr int kGemvMaxSweeps = MOEDEC_MAX_DIM / 4 / kGemvThreads;   // float4 columns per thread at most

// Block b -> (expert tile, token tile).  The token tiles of one expert tile
// get blocks with the same b % 8: blocks are dealt round-robin to the eight
// XCDs, so they share an L2 and the tile's rows come from HBM once.
// Per sweep s every thread loads column 512*s + tid (a float4) of its EB
// rows and TB tokens, the next sweep's loads going out before this sweep is
// dotted; columns past the row's end are clamped for the load and their
// products masked to zero.  Each wave's partial sums go to LDS and one
// thread per (expert, token) adds the 8 waves' sums in wave order.
template <int EB, int TB, int NS>
__global__ __launch_bounds__(kGemvThreads) void router_gemv_kernel(const float* __restrict__ x,
                                                                   const float* __restrict__ W, int T, int H,
                                                                   int E, float* __restrict__ scores,
                                                                   int32_t* __restrict__ arrivals) {
    if (arrivals != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *arrivals = 0;   // route_tokens counts here
    const int nEt = (E + EB - 1) / EB, nTt = (T + TB - 1) / TB;
    const int q = blockIdx.x >> 3;
    const int tt = q % nTt, et = (q / nTt) * 8 + (blockIdx.x & 7);
    if (et >= nEt) return;                               // the grid's last row of eight may be short
    const int e0 = et * EB, t0 = tt * TB;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int n4 = H >> 2;
    const float4* rows[EB + TB];
#pragma unroll
    for (int i = 0; i < EB; ++i) rows[i] = reinterpret_cast<const float4*>(W + (size_t)min(e0 + i, E - 1) * H);
#pragma unroll
    for (int j = 0; j < TB; ++j) rows[EB + j] = reinterpret_cast<const float4*>(x + (size_t)min(t0 + j, T - 1) * H);
    float4 buf[2][EB + TB];
    auto load = [&](float4 (&r)[EB + TB], int s) {
        const int c = min(tid + s * kGemvThreads, n4 - 1);
#pragma unroll
        for (int i = 0; i < EB + TB; ++i) r[i] = rows[i][c];
    };
    float acc[EB][TB];
#pragma unroll
    for (int i = 0; i < EB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = 0.f;
    load(buf[0], 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s + 1 < NS) load(buf[(s + 1) & 1], s + 1);
        const unsigned keep = tid + s * kGemvThreads < n4 ? ~0u : 0u;
        const float4* r = buf[s & 1];
#pragma unroll
        for (int i = 0; i < EB; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const float4 w = r[i], v = r[EB + j];
                const float d = (w.x * v.x + w.y * v.y) + (w.z * v.z + w.w * v.w);
                acc[i][j] += __uint_as_float(__float_as_uint(d) & keep);
            }
    }
    __shared__ float red[EB * TB][kGemvWaves];
#pragma unroll
    for (int i = 0; i < EB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = wave_sum_last(acc[i][j]);
    if (lane == kWave - 1) {
#pragma unroll
        for (int i = 0; i < EB; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) red[i * TB + j][wave] = acc[i][j];
    }
    __syncthreads();
    if (tid < EB * TB) {
        const int i = tid / TB, j = tid - (tid / TB) * TB;
        if (e0 + i < E && t0 + j < T) {
            float z = 0.f;
#pragma unroll
            for (int w = 0; w < kGemvWaves; ++w) z += red[tid][w];
            scores[(size_t)(t0 + j) * E + e0 + i] = 1.0f / (1.0f + expf(-z));
        }
    }
}

template <int EB, int TB, int MaxNS = kGemvMaxSweeps>
hipError_t launch_gemv(const float* x, const float* W, int T, int H, int E, float* scores, int32_t* arrivals,
                       hipStream_t st) {
    const int sweeps = (H / 4 + kGemvThreads - 1) / kGemvThreads;
    const int nEt = (E + EB - 1) / EB, nTt = (T + TB - 1) / TB;
    const dim3 grid(((nEt + 7) / 8) * 8 * nTt);
    auto k = router_gemv_kernel<EB, TB, MaxNS>;
    if (sweeps <= 1) k = router_gemv_kernel<EB, TB, 1>;
    else if (sweeps <= 2) k = router_gemv_kernel<EB, TB, 2>;
    else if (sweeps <= 3) k = router_gemv_kernel<EB, TB, 3>;
    else if (sweeps <= 4) k = router_gemv_kernel<EB, TB, 4>;
    hipLaunchKernelGGL(k, grid, dim3(kGemvThreads), 0, st, x, W, T, H, E, scores, arrivals);
    return hipGetLastError();
}

// One one-wave workgroup per token (tokens on separate SIMDs: one wave's
// routing is a chain of dependent wave-wide steps, and waves sharing a SIMD
// would take turns).  Each writes its slots with device-scope stores, counts
// itself on the worklist's n_active word (zeroed by router_gemv), and the
// last to arrive reads every token's slots back and builds the worklist.
template <bool kTopP, int NV, int EMT>
__global__ __launch_bounds__(kWave) void route_tokens_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int T, int E, int n_group, int topk_group,
    int top_k, int n_shared, float rsf, float top_p, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ wl_n_active, int32_t* __restrict__ wl_expert_id, int32_t* __restrict__ wl_seg,
    int32_t* __restrict__ wl_assign) {
    static_assert(NV * kWave == EMT, "lane l holds experts l*NV .. l*NV+NV-1");
    __shared__ RouteLdsT<MOEDEC_MAX_TOKENS, EMT, 1> r;
    const int t = blockIdx.x, lane = threadIdx.x;
    route_one_token<NV, MOEDEC_MAX_TOKENS, EMT, 1, false, kTopP>(scores, bias, t, E, n_group, topk_group, top_k, rsf,
                                                                top_p, r);
    wave_lds_sync();
    if (lane < top_k) {                // device-scope stores: the last workgroup reads them back
        __hip_atomic_store(topk_idx + t * top_k + lane, r.sel[t * top_k + lane], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        topk_w[t * top_k + lane] = r.selw[t * top_k + lane];
    }
    if (wl_n_active == nullptr) return;
    __builtin_amdgcn_s_waitcnt(0);     // this wave's slot stores have completed: arrive
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(wl_n_active, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, kWave);
    if (old != T - 1) return;
    // the last to arrive: every token's slots (device-scope loads), then the union
    for (int i = lane; i < T * top_k; i += kWave)
        r.sel[i] = __hip_atomic_load(topk_idx + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wave_lds_sync();
    route_union_counting<MOEDEC_MAX_TOKENS, EMT, 1, kTopP>(T, E, top_k, n_shared, r);
    const int n = min(r.n_active, E + n_shared);      // (bounds for the writes below)
    const int A = min(r.n_assign, T * (top_k + n_shared));   // = seg[n]
    for (int j = lane; j <= n; j += kWave) {
        if (j < n) wl_expert_id[j] = r.eid[j];
        wl_seg[j] = r.seg[j];
    }
    for (int a = lane; a < A; a += kWave) wl_assign[a] = r.assign[a];
    if (lane == 0) *wl_n_active = n;
}

}  // namespace

hipError_t launch_route(const float* x, const float* router_w, const float* bias, int T, int H, int E,
                        int n_group, int topk_group, int top_k, int n_shared, float rsf, float top_p,
                        float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                        hipStream_t st) {
    // tiles: about 256 workgroups for E = 256 at every T, at most 8 rows each
    int32_t* arrivals = wl ? wl->n_active : nullptr;
    hipError_t err;
    if (T == 1) err = launch_gemv<1, 1>(x, router_w, T, H, E, scores, arrivals, st);
    else if (T == 2) err = launch_gemv<1, 2>(x, router_w, T, H, E, scores, arrivals, st);
    else if (T <= 4) err = launch_gemv<1, 4>(x, router_w, T, H, E, scores, arrivals, st);
    else if (T <= 8) err = launch_gemv<2, 4>(x, router_w, T, H, E, scores, arrivals, st);
    else if (H <= 4 * 4 * kGemvThreads) err = launch_gemv<4, 4, 4>(x, router_w, T, H, E, scores, arrivals, st);
    else err = launch_gemv<2, 4>(x, router_w, T, H, E, scores, arrivals, st);      // (4, 4) would spill at 8 sweeps
    if (err != hipSuccess) return err;
    // E <= 256: 4 experts per lane; more: 16
    const bool topp = top_p < 1.f, wide = E > 4 * kWave;
    auto k = topp ? route_tokens_kernel<true, 4, 4 * kWave> : route_tokens_kernel<false, 4, 4 * kWave>;
    if (wide)
        k = topp ? route_tokens_kernel<true, 16, MOEDEC_MAX_EXPERTS> : route_tokens_kernel<false, 16, MOEDEC_MAX_EXPERTS>;
    hipLaunchKernelGGL(k, dim3(T), dim3(kWave), 0, st, scores, bias, T, E, n_group, topk_group, top_k, n_shared, rsf,
                       top_p, topk_idx, topk_w, arrivals, wl ? wl->expert_id : nullptr, wl ? wl->seg : nullptr,
                       wl ? wl->assign : nullptr);
    return hipGetLastError();
}

}  // namespace moedec
