// The whole routed-MoE decode step of one layer in one launch: router scores,
// group-limited top-k and batch union, gate/up + SwiGLU of every unique
// expert, down + weighted combine.
//
// Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented
// features": sigmoid router with noaux_tc correction, routed_scaling_factor
// and a shared expert; row-scaled int8 / int4 / int2 experts dequantised on
// use; batch-union MoE (each unique expert of the batch read once).
//
// A decode step moves ~170 MB of codes (GLM-5.2 shape, one token) in a few
// tens of microseconds, so separate kernels pay their launch gaps, start-up
// (worklist loads, activation staging) and drain tails several times over.
// Here one persistent workgroup per compute unit runs four phases, with two
// grid-wide barriers:
//   1. (needs no routing) router rows e = b, b + nwg, ...: s = sigmoid(W_r x);
//      stage x as MFMA B operands in LDS; gate/up of the shared experts, whose
//      tokens are known up front, over this workgroup's share of their rows;
//   -- barrier: every score is written --
//   2. every workgroup routes the batch itself from the scores (route.h), so
//      the worklist needs no second exchange; workgroup 0 also writes the
//      routing and worklist outputs;
//   3. gate/up of the routed experts over this workgroup's share of rows;
//   -- barrier: every h row is written; each workgroup arrives, issues its
//      first down-weight loads, and only then waits --
//   4. down + combine for this workgroup's output rows over every expert.
//
// The barrier is a counter and a generation number in a caller-owned
// workspace (device memory, zeroed once before first use): a workgroup reads
// the generation, adds one to the counter; the last to arrive resets the
// counter and advances the generation; the rest wait for the generation to
// change.  The counter returns to zero by the end of every launch, so the
// workspace needs no clearing between launches.  All workgroups must be
// resident at once: the grid is one workgroup per compute unit and each asks
// for more than half of a compute unit's LDS.  The wait is bounded: after the
// spin limit the workgroup sets the workspace's error word and goes on, so a
// launch that cannot be co-resident (the GPU shared with other work) ends
// with garbage outputs and a raised flag instead of hanging.
#include "mfma.h"
#include "route.h"

namespace moedec {

namespace {

using namespace mfma;

constexpr int kFusedExperts = 512;                      // routed experts at most
using FusedRoute = RouteLdsT<kCols, kFusedExperts>;
constexpr int kRowF4 = MOEDEC_MAX_DIM / 4 / kMT;        // float4 of a router row per thread
constexpr int kSpinDefault = 1 << 21;                   // ~1 us per round: a couple of seconds

// workspace words
constexpr int kWsCount = 0, kWsGen = 1, kWsError = 2, kWsSpin = 3;

struct FusedArgs {
    ExpertArgs a;                  // experts; its worklist pointers are unused
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
    int32_t* ws;
    int E, n_group, topk_group, n_shared;
    float rsf;
    int ns;                        // tokens staged at once for gate/up
    int qc;                        // assignments staged at once for down
    int down_rows;                 // output rows of one down pass of a workgroup
};

// Split-phase grid barrier (see the file comment).  arrive(): every wave makes
// its global writes visible device-wide, then one thread arrives.  wait():
// that thread waits for the last arrival, with acquire ordering, then the
// workgroup resynchronises; the acquire (by the one thread) invalidates the
// compute unit's caches that the whole workgroup reads through.
struct GridGate {
    int32_t* ws;
    int spin_max;
    int* gen_s;                    // LDS: the generation read before arriving

    __device__ void arrive() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (threadIdx.x == 0) {
            const int g0 = __hip_atomic_load(ws + kWsGen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *gen_s = g0;
            const int old = __hip_atomic_fetch_add(ws + kWsCount, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            if (old == (int)gridDim.x - 1) {
                __hip_atomic_store(ws + kWsCount, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_add(ws + kWsGen, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    __device__ void wait() {
        if (threadIdx.x == 0) {
            const int g0 = *gen_s;
            int n = 0;
            while (__hip_atomic_load(ws + kWsGen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == g0) {
                if (++n >= spin_max) {
                    __hip_atomic_store(ws + kWsError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
    }
};

// Router rows e = part, part + nparts, ... for all T tokens: every thread holds
// its float4s of the row, dots them with each token, the wave sums by DPP and
// the 8 waves' sums are added in wave order.
__device__ void router_rows(const FusedArgs& f, int part, int nparts, float (*red)[kMW]) {
    const int H = f.a.H, T = f.a.T, E = f.E;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n4 = H >> 2;
    for (int e = part; e < E; e += nparts) {
        const float4* w4 = reinterpret_cast<const float4*>(f.router_w + (size_t)e * H);
        float4 wr[kRowF4];
#pragma unroll
        for (int k = 0; k < kRowF4; ++k) {
            const int i = threadIdx.x + k * kMT;
            wr[k] = i < n4 ? w4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int t = 0; t < T; ++t) {
            const float4* x4 = reinterpret_cast<const float4*>(f.x + (size_t)t * H);
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < kRowF4; ++k) {
                const int i = threadIdx.x + k * kMT;
                if (i < n4) {
                    const float4 v = x4[i];
                    acc = fmaf(wr[k].x, v.x, acc);
                    acc = fmaf(wr[k].y, v.y, acc);
                    acc = fmaf(wr[k].z, v.z, acc);
                    acc = fmaf(wr[k].w, v.w, acc);
                }
            }
            acc = group_sum<kWave>(acc);
            if (lane == 0) red[t][wave] = acc;
        }
        __syncthreads();
        if ((int)threadIdx.x < T) {
            float z = 0.f;
            for (int w = 0; w < kMW; ++w) z += red[threadIdx.x][w];
            f.scores[(size_t)threadIdx.x * E + e] = 1.0f / (1.0f + expf(-z));
        }
        __syncthreads();
    }
}

template <int BITS>
__global__ __launch_bounds__(kMT) void layer_fused_kernel(const FusedArgs f) {
    constexpr int NCALL = MfmaCodec<BITS>::NCALL;
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ FusedRoute r;
    __shared__ GateUpLds s;
    __shared__ float gemv_red[kCols][kMW];
    __shared__ int sh_eid[8], sh_seg[9], sh_assign[8 * kCols];
    __shared__ int gen_s;

    const ExpertArgs& a = f.a;
    const int T = a.T, H = a.H, K = a.top_k, S = f.n_shared, E = f.E;
    const int NCH = ((H * BITS / 8) / 16 + 3) / 4;
    half8* xhi = reinterpret_cast<half8*>(dyn);
    half8* xlo = xhi + (size_t)NCH * 4 * f.ns * NCALL;
    float* red = reinterpret_cast<float*>(xlo + (size_t)NCH * 4 * f.ns * NCALL);
    const bool stage_all = T <= f.ns;
    const int spin = f.ws[kWsSpin] > 0 ? f.ws[kWsSpin] : kSpinDefault;
    GridGate gate{f.ws, spin, &gen_s};

    // ---- phase 1: router rows, staging, shared experts' gate/up
    router_rows(f, blockIdx.x, gridDim.x, gemv_red);
    if (stage_all) stage_tokens<BITS>(f.x, T, H, f.ns, xhi, xlo, s);
    for (int i = threadIdx.x; i < S * T; i += kMT) {   // the shared experts' worklist: every token
        const int j = i / T, t = i - j * T;
        sh_assign[i] = t * a.slots + K + j;
    }
    if ((int)threadIdx.x <= S) {
        if ((int)threadIdx.x < S) sh_eid[threadIdx.x] = E + threadIdx.x;
        sh_seg[threadIdx.x] = threadIdx.x * T;
    }
    __syncthreads();
    gate_up_units<BITS>(a, f.x, f.h, sh_eid, sh_seg, sh_assign, S, f.ns, stage_all, blockIdx.x, gridDim.x, xhi,
                        xlo, red, s);

    // ---- barrier 1, phase 2: routing (every workgroup, identically)
    gate.arrive();
    gate.wait();
    route_select_block<kCols, kFusedExperts>(f.scores, f.bias, T, E, f.n_group, f.topk_group, K, S, f.rsf, r);
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < T * K; i += kMT) {
            f.topk_idx[i] = r.sel[i];
            f.topk_w[i] = r.selw[i];
        }
        const int n = r.n_active;
        if (threadIdx.x == 0) *f.wl_n_active = n;
        for (int j = threadIdx.x; j <= n; j += kMT) {
            if (j < n) f.wl_expert_id[j] = r.eid[j];
            f.wl_seg[j] = r.seg[j];
        }
        for (int i = threadIdx.x; i < T * a.slots; i += kMT) f.wl_assign[i] = r.assign[i];
    }

    // ---- phase 3: routed experts' gate/up (the shared ones are the last S worklist entries)
    gate_up_units<BITS>(a, f.x, f.h, r.eid, r.seg, r.assign, r.n_active - S, f.ns, stage_all, blockIdx.x,
                        gridDim.x, xhi, xlo, red, s);

    // ---- barrier 2 (inside the first down pass), phase 4: down + combine
    struct Once {
        GridGate& g;
        bool done;
        __device__ void arrive() {
            if (!done) g.arrive();
        }
        __device__ void wait() {
            if (!done) g.wait();
            done = true;
        }
    } once{gate, false};
    for (int r0 = blockIdx.x * f.down_rows; r0 < H; r0 += gridDim.x * f.down_rows) {
        const int r1 = min(r0 + f.down_rows, H);
        down_rows<BITS>(f.h, r.selw, a, f.y, r0, r1, f.qc, dyn, r.eid, r.seg, r.assign, r.n_active, s.scratch,
                        once);
    }
    if (!once.done) {          // no rows here: still arrive, so the others can go on
        once.arrive();
        once.wait();
    }
}

struct FusedPlan {
    int ns, qc, rows;
    size_t lds;
};

template <int BITS>
hipError_t fused_plan(const FusedArgs& f, int nwg, FusedPlan& p) {
    static size_t static_lds = 0;        // the kernel's static LDS, read once
    auto k = layer_fused_kernel<BITS>;
    if (static_lds == 0) {
        hipFuncAttributes attr;
        hipError_t err = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(k));
        if (err != hipSuccess) return err;
        static_lds = (attr.sharedSizeBytes + 1023) & ~(size_t)1023;
    }
    if (static_lds + kLdsOnePerCu > kLdsMax) return hipErrorInvalidValue;
    const size_t avail = kLdsMax - static_lds;
    const size_t per_tok = gate_up_lds_per_token<BITS>(f.a.H);
    int fit = (int)(avail / per_tok);
    if (fit > kCols) fit = kCols;
    if (fit < 1) return hipErrorInvalidValue;
    p.ns = f.a.T < fit ? f.a.T : fit;
    const size_t fixed = down_lds_fixed_bytes();
    const size_t per_q = down_lds_bytes_per_assignment<BITS>(f.a.I);
    if (avail < fixed + per_q) return hipErrorInvalidValue;
    const int A = f.a.T * f.a.slots;
    p.qc = (int)((avail - fixed) / per_q);
    if (p.qc > A) p.qc = A;
    int rows = (f.a.H + nwg - 1) / nwg;
    if (rows < 16) rows = 16;
    if (rows > kNBD * 16) rows = kNBD * 16;
    p.rows = rows;
    size_t lds = (size_t)p.ns * per_tok;
    const size_t lds_down = fixed + (size_t)p.qc * per_q;
    if (lds < lds_down) lds = lds_down;
    if (lds < kLdsOnePerCu) lds = kLdsOnePerCu;
    p.lds = lds;
    return hipSuccess;
}

template <int BITS>
hipError_t layer_fused_bits(FusedArgs f, hipStream_t st) {
    const int nwg = cu_count();
    FusedPlan p;
    hipError_t err = fused_plan<BITS>(f, nwg, p);
    if (err != hipSuccess) return err;
    f.ns = p.ns;
    f.qc = p.qc;
    f.down_rows = p.rows;
    auto k = layer_fused_kernel<BITS>;
    err = allow_lds(k, p.lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(nwg), dim3(kMT), p.lds, st, f);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layer_fused(int bits, const FusedLayerArgs& l, hipStream_t st) {
    if (l.T > kCols || l.E > kFusedExperts) return hipErrorInvalidValue;
    FusedArgs f{};
    f.a = l.ex;
    f.x = l.x;
    f.router_w = l.router_w;
    f.bias = l.bias;
    f.scores = l.scores;
    f.topk_idx = l.topk_idx;
    f.topk_w = l.topk_w;
    f.wl_n_active = l.wl_n_active;
    f.wl_expert_id = l.wl_expert_id;
    f.wl_seg = l.wl_seg;
    f.wl_assign = l.wl_assign;
    f.h = l.h;
    f.y = l.y;
    f.ws = l.workspace;
    f.E = l.E;
    f.n_group = l.n_group;
    f.topk_group = l.topk_group;
    f.n_shared = l.n_shared;
    f.rsf = l.rsf;
    switch (bits) {
        case 4: return layer_fused_bits<4>(f, st);
        case 8: return layer_fused_bits<8>(f, st);
        case 2: return layer_fused_bits<2>(f, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moedec
