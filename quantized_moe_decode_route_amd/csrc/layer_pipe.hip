// The whole routed-MoE decode step of one layer in one launch, as one
// continuous weight stream per workgroup with the experts pipelined: router
// scores, group-limited top-k and batch union, then for every unique expert
// its gate/up + SwiGLU rows and its down + weighted-combine rows.
//
// Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented
// features": sigmoid router with noaux_tc correction, routed_scaling_factor
// and a shared expert; row-scaled int8 / int4 / int2 experts dequantised on
// use; batch-union MoE (each unique expert of the batch read once).
//
// Why pipelined.  An expert's down projection needs every row of its h,
// which many workgroups produce, so it waits for a grid-wide exchange; a
// layout that exchanges all experts' h at once leaves HBM idle for the whole
// exchange.  Here every workgroup takes an equal share of EVERY expert (a
// tile of 8 gate/up row pairs, and a fixed block of down output rows) and
// the experts are streamed one after another (slot 0.. the shared experts
// first, they need no routing, then the routed ones).  When the staged-h
// buffers in LDS hold every expert of the batch, the order is all GU(j),
// then all DN(j): each expert's h is exchanged and staged while the later
// experts' gate/up rows stream.  Otherwise DN(j) follows GU(j + L), L = 10:
//     GU(0) .. GU(9) GU(10) DN(0) GU(11) DN(1) ... GU(n-1) DN(n-11) DN(n-10) .. DN(n-1)
// so a staged buffer is freed while later experts still stream, and each
// expert's h has the time of L gate/up units to be exchanged and staged.
//
// Waves of a workgroup (one workgroup per compute unit, 8 waves by default):
//   streaming (0-5): a ring of kRing items per wave in flight, int8
//        matrix-core products of the items; gate/up tiles leave exact int32
//        partial sums in LDS, down items accumulate the layer output in
//        registers.  Each wave's items are listed in LDS once per launch, so
//        the stream does no schedule arithmetic;
//   finalizer (6): per expert, the gate/up partial sums of all streaming
//        waves -> h = silu(g) * u for the workgroup's 8 pairs, stored with
//        device-scope stores; once every expert is finalized it stages the
//        experts the stager has not claimed yet;
//   stager (7): per expert, loads every workgroup's h once it is there and
//        stages it (times the routing weight) as matrix-core operands in LDS;
//        the next row's loads are in flight while a row is staged.
// Streaming waves synchronise with the control waves through LDS counters
// only, so their loads in flight are never waited for.
//
// Activations are exact integers under one power-of-two scale per column
// (token, or staged assignment): x * 2^e is rounded to a 24-bit integer and
// split into three signed bytes hi, mid, lo (x * 2^e = 65536 hi + 256 mid +
// lo).  The three bytes of a token sit in three different B columns of the
// 16x16x64 int8 MFMA, so one MFMA per code operand yields all three partial
// dot products at once (for up to five tokens); they are exact in int32 and
// combined in fp32 at the end.  The only rounding of the products is that of
// x (and of the staged h * weight) to 24 bits relative to its column's
// largest magnitude.
//
// Exchanges.  The scores are exchanged once per launch through arrival
// counters in the caller's workspace that only ever grow (each launch adds
// one per workgroup; a launch finds its index from the count).  Each
// expert's h is exchanged through the h output itself: before its scores
// arrival every workgroup writes a sentinel NaN over its share of h, so once
// the scores exchange has passed, an h value read is either the sentinel or
// this launch's value, and the stager re-reads a row until no sentinel is
// left (a NaN result is stored as the canonical NaN, never the sentinel).
// Under a saturated weight stream every memory round trip is long, and this
// costs one store and one read per exchange where an arrival count costs a
// store, its acknowledgement, an arrival and a counter poll.  Every wait is
// bounded: past the spin limit the waiter raises the workspace's error word
// and goes on, so a launch that cannot be co-resident ends with a raised flag
// instead of hanging.
#include "imma.h"
#include "persist.h"
#include "route.h"

namespace moedec {

namespace {

using namespace mfma;
using namespace imma;

#ifndef MOEDEC_PIPE_RING
#define MOEDEC_PIPE_RING 4
#endif
#ifndef MOEDEC_PIPE_WAVES
#define MOEDEC_PIPE_WAVES 8
#endif
constexpr int kPW = MOEDEC_PIPE_WAVES;                  // waves of a workgroup (one per compute unit)
constexpr int kPT = kPW * kWave;                        // its threads
#ifndef MOEDEC_PIPE_STAGERS
#define MOEDEC_PIPE_STAGERS 1
#endif
constexpr int kNStg = MOEDEC_PIPE_STAGERS;              // stager waves (slots claimed in order, see staging)
constexpr int kSW = kPW - 1 - kNStg;                    // streaming waves
constexpr int kFin = kSW, kStg = kSW + 1;               // control waves: the finalizer, the stagers
constexpr int kRing = MOEDEC_PIPE_RING;                 // items in flight per streaming wave
constexpr int kLag = 10;                                // DN(j) follows GU(j + kLag) when not every slot fits a buffer
constexpr int kNHBMax = 16;                             // staged-h buffers at most (2 where LDS is short)
constexpr int kNPB = 3;                                 // gate/up partial-sum buffers
constexpr int kPieces = 3;                              // bytes of a 24-bit activation
constexpr int kPipeExperts = 512;                       // routed experts at most
using PipeRoute = RouteLdsT<kCols, kPipeExperts, kPW>;
constexpr int kRowF4 = (MOEDEC_MAX_DIM / 4 + kPT - 1) / kPT;   // float4 of a router row per thread
constexpr int kStageX4 = 4;                             // float4 of x a thread holds at once
constexpr int kStageH4 = 8;                             // float4 of an h row the stager's lanes hold at once
constexpr int kSpinDefault = 1 << 21;                   // ~1 us per poll: a couple of seconds
constexpr int kLdsSpin = 1 << 24;
constexpr int kBufWord3 = 0x00020000;                   // raw buffer resource: 32-bit data format
constexpr int kCoherent = 16;                           // buffer load cache policy: device-coherent (sc1)
constexpr float kV24 = 8323072.0f;                      // largest |x * 2^e| (hi stays within +-127)

// Workspace words of this kernel (disjoint from the other fused kernel's).
constexpr int kGates = 8, kGateStride = 32;             // counters per gate, words between counters (128 B)
constexpr int kSetWords = kGates * kGateStride;
constexpr int kWsBase = 1024;                           // the scores exchange's counters
constexpr uint32_t kSentinel = 0x7FBADA55u;             // h not yet written (a NaN no arithmetic here yields)
static_assert(kWsBase + kSetWords <= MOEDEC_FUSED_WORKSPACE_INTS, "workspace layout");
static_assert(MOEDEC_FUSED_WS_SPIN < kWsBase, "workspace layout");

struct PipeArgs {
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
    float* x_out;                  // residual form: x_out = x + y (x is then the un-normalised stream)
    int32_t* ws;
    int E, n_group, topk_group, n_shared;
    float rsf, top_p, eps;
    int nc;                        // B columns per pass (3T for one pass, else 16)
    int ntile_max;                 // gate/up tiles of one expert a workgroup takes at most
    int off_hb, off_part, off_pers, off_route;   // dynamic LDS layout (bytes); x operands at 0
    int off_gsc, off_dsc;          // row-scale tables: [slot][tile][16] gate/up, [slot][32] down
    int off_items, max_items;      // the streaming waves' item lists: [kSW][max_items] uint2
    int off_rows, max_rows;        // the staging row list: [max_rows] uint2, then [max_active + 1] slot offsets
    int nhb;                       // staged-h buffers (2 .. kNHBMax)
};

// LDS words shared by the waves of a workgroup.
struct PipeSync {
    int gu_cnt[kNPB];              // partial-sum tiles written to each buffer (cumulative)
    int gu_free[kNPB];             // 1 + the last gate/up unit finalized from each buffer
    int hb_ready[kNHBMax];         // 1 + the down unit staged in each buffer
    int hb_done[kNHBMax];          // streaming waves done with each buffer (cumulative)
    int fin_cum[kNPB];             // finalizer: partial-sum tiles expected from each buffer so far
    int fin_done;                  // 1 + the last slot whose h this workgroup's finalizer has stored
    int next_slot;                 // staging: the next slot to claim (stagers, then the finalizer too)
    int rows_listed;               // staging: 1 once the row list and slot offsets are in LDS
    float xu[kCols];               // 2^-(e_t + shift): undoes token t's exponent and the code factor
    float xinv[kCols];             // residual form: 1 / rms of token t
    unsigned cmax[kCols];          // largest |x| of token t (bits)
    float dsl[kNHBMax][kCols];     // per staged buffer: token t's unscale times its piece, 0 = not routed
    float gemv_red[kCols][kPW];
    float gemv_ssq[kCols][kPW];
    int n_slots;                   // experts of the batch (shared first)
    int n_assign;
};

// Phase timestamps of every workgroup (-DMOEDEC_PIPE_TRACE builds only, for
// tuning; the product build compiles the marks away): slot k of workgroup b
// holds the realtime counter (100 MHz) when lane 0 of the marking wave passed
// mark k.
[[maybe_unused]] constexpr int kTraceSlots = 96;
#ifdef MOEDEC_PIPE_TRACE
__device__ unsigned long long g_pipe_trace[4096 * kTraceSlots];
#define PIPE_MARK(tr, k)                                                                   \
    do {                                                                                   \
        if ((k) < kTraceSlots && (threadIdx.x & (kWave - 1)) == 0) (tr)[k] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define PIPE_MARK(tr, k) \
    do {                 \
    } while (0)
#endif

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
// The wave index, as a wave-uniform (scalar) value: everything the schedule
// derives from it then stays in scalar registers and its branches are scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

__device__ __forceinline__ void raise_error(int32_t* ws) {
    __hip_atomic_store(ws + MOEDEC_FUSED_WS_ERROR, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (one wave) until an LDS counter reaches v; bounded by `cap` polls
// (read once per launch: a global load here would wait for the wave's loads
// in flight).
__device__ __forceinline__ void lds_wait_ge(const int* p, int v, int32_t* ws, int cap) {
    int n = 0;
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < v) {
        if (++n > cap) {
            raise_error(ws);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Publish this wave's earlier LDS writes, then add to (or set) an LDS counter.
__device__ __forceinline__ void lds_signal_add(int* p, int v) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane_id() == 0) __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_signal_set(int* p, int v) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane_id() == 0) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The scores exchange's arrival counters (see the file comment; gate 0 is
// the only gate).  Workgroup b counts on counter b % kGates.
struct Gates {
    int32_t* ws;
    int spin_max;
    unsigned long long launch;

    __device__ __forceinline__ static int members(int i) { return ((int)gridDim.x - i + kGates - 1) / kGates; }
    __device__ __forceinline__ unsigned long long* counter(int gate, int i) const {
        return reinterpret_cast<unsigned long long*>(ws + kWsBase + gate * kSetWords + i * kGateStride);
    }
    __device__ __forceinline__ void init() {
        const int own = blockIdx.x % kGates;
        const unsigned long long found =
            __hip_atomic_load(counter(0, own), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        launch = found / (unsigned long long)members(own);
    }
    // one lane of the calling wave adds v to this workgroup's counter of `gate`
    __device__ __forceinline__ void add(int gate, unsigned long long v) const {
        if (lane_id() == 0)
            __hip_atomic_fetch_add(counter(gate, blockIdx.x % kGates), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the calling wave polls until every counter of `gate` holds at least
    // per_member arrivals per member workgroup; four polls are kept in flight
    // (each step checks the oldest and issues the next), so completion is
    // seen a fraction of a round trip after it happens
    __device__ __forceinline__ void wait(int gate, unsigned long long per_member) const {
        const int lane = lane_id();
        const int i = lane < kGates ? lane : kGates - 1;
        const unsigned long long target = per_member * (unsigned long long)members(i);
        unsigned long long* cp = counter(gate, i);
        auto poll = [&]() { return __hip_atomic_load(cp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        unsigned long long p0 = poll(), p1, p2, p3;
        __builtin_amdgcn_s_sleep(1);
        p1 = poll();
        __builtin_amdgcn_s_sleep(1);
        p2 = poll();
        __builtin_amdgcn_s_sleep(1);
        p3 = poll();
        int n = 0;
        while (true) {
            if (__ballot(p0 < target) == 0) break;
            if (++n >= spin_max) {
                raise_error(ws);
                break;
            }
            p0 = p1;
            p1 = p2;
            p2 = p3;
            __builtin_amdgcn_s_sleep(1);
            p3 = poll();
        }
    }
};

// Largest power-of-two exponent e with m * 2^e <= kV24 (0 for m = 0 or a
// non-finite m, whose column then holds garbage either way).
__device__ __forceinline__ int q24_exponent(float m) {
    if (!(m > 0.f) || !isfinite(m)) return 0;
    int e;
    frexpf(m, &e);                      // m in [2^(e-1), 2^e)
    int k = 23 - e;                     // m * 2^k in [2^22, 2^23)
    if (ldexpf(m, k) > kV24) --k;
    return k > 100 ? 100 : k < -100 ? -100 : k;
}

// The three signed bytes of x * 2^e (already scaled) rounded to 24 bits, as
// bytes 0 (lo), 1 (mid) and 2 (hi) of the result: with every digit biased by
// 128, v + 0x808080 has the base-256 digits lo+128, mid+128, hi+128, and a
// biased digit d is the signed byte d - 128 = d ^ 0x80.
__device__ __forceinline__ uint32_t bytes24(float xs) {
    const float r = fminf(fmaxf(rintf(xs), -kV24), kV24);
    return ((uint32_t)((int)r + 0x808080)) ^ 0x808080u;
}
// byte q of a and byte q of b as the two bytes of a 16-bit value
__device__ __forceinline__ uint32_t pack_q2(uint32_t a, uint32_t b, int q) {
    return ((a >> (8 * q)) & 0xFFu) | (((b >> (8 * q)) & 0xFFu) << 8);
}

// B operand layout of one staged operand set (x, or one expert's h): for
// K-chunk c, pass p, lane group lq, code operand m and column n, 16 byte
// slots at byte ((((c * NP + p) * 4 + lq) * NM + m) * nc + n) * 16.  Column
// 3t + q (pass (3t+q) / 16) holds byte q of token t.  Slot s of operand m of
// lane group lq stands for the code column I8Codec::col(m, s) of the group.
template <int BITS, int NP>
__device__ __forceinline__ size_t b_unit(int c, int pass, int lq, int m, int n, int nc) {
    return ((((size_t)c * NP + pass) * 4 + lq) * I8Codec<BITS>::NM + m) * nc + n;
}

// Scatter 4 consecutive columns col0.. (col0 % 4 == 0) of token t, already
// scaled by 2^e, into the B layout.
template <int BITS, int NP>
__device__ __forceinline__ void scatter24(float4 v, int col0, int t, int nc, uint8_t* B) {
    using C = I8Codec<BITS>;
    const uint32_t bx = bytes24(v.x), by = bytes24(v.y), bz = bytes24(v.z), bw = bytes24(v.w);
    const int g = col0 / C::CW, p0 = col0 - g * C::CW;
    const int c = g >> 2, lq = g & 3;
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {                  // piece q (hi, mid, lo) = byte 2 - q
        const int col = kPieces * t + q, bq = 2 - q;
        const int pass = NP > 1 ? col >> 4 : 0, n = NP > 1 ? col & 15 : col;
        uint8_t* u0 = B + b_unit<BITS, NP>(c, pass, lq, 0, n, nc) * 16;
        const size_t mstep = (size_t)nc * 16;
        if constexpr (BITS == 4) {
            // columns p0, p0+2 -> operand 0 slots s0, s0+1; p0+1, p0+3 -> operand 1
            const int s0 = 4 * (p0 >> 3) + ((p0 >> 1) & 3);
            *reinterpret_cast<uint16_t*>(u0 + s0) = (uint16_t)pack_q2(bx, bz, bq);
            *reinterpret_cast<uint16_t*>(u0 + mstep + s0) = (uint16_t)pack_q2(by, bw, bq);
        } else if constexpr (BITS == 8) {
            *reinterpret_cast<uint32_t*>(u0 + p0) = pack_q2(bx, by, bq) | pack_q2(bz, bw, bq) << 16;
        } else {
            // columns p0 .. p0+3 -> operands 0..3, one slot
            const int s0 = 4 * (p0 >> 4) + ((p0 >> 2) & 3);
            u0[s0] = (uint8_t)(bx >> (8 * bq));
            u0[mstep + s0] = (uint8_t)(by >> (8 * bq));
            u0[2 * mstep + s0] = (uint8_t)(bz >> (8 * bq));
            u0[3 * mstep + s0] = (uint8_t)(bw >> (8 * bq));
        }
    }
}

// Int4 codes: 16 consecutive columns col0.. (col0 % 16 == 0) of token t, as
// four raw fp32 float4 (each value times ws), into the B layout.  Of a group's
// 32 columns, operand 0 takes the even ones and operand 1 the odd ones, in
// slot order, so 16 columns fill 8 consecutive bytes of each operand (one
// 8-byte write per operand and piece).
template <int NP>
__device__ __forceinline__ void scatter24_quad4(const u32x4* v, float ws, int col0, int t, int nc, uint8_t* B) {
    uint32_t bt[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bt[4 * i + 0] = bytes24(__uint_as_float(v[i].x) * ws);
        bt[4 * i + 1] = bytes24(__uint_as_float(v[i].y) * ws);
        bt[4 * i + 2] = bytes24(__uint_as_float(v[i].z) * ws);
        bt[4 * i + 3] = bytes24(__uint_as_float(v[i].w) * ws);
    }
    const int g = col0 >> 5, s0 = (col0 & 31) >> 1;     // slots s0 .. s0 + 7 of both operands
    const int c = g >> 2, lq = g & 3;
    const size_t mstep = (size_t)nc * 16;
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {                  // piece q (hi, mid, lo) = byte 2 - q
        const int col = kPieces * t + q, sh = 8 * (2 - q);
        const int pass = NP > 1 ? col >> 4 : 0, n = NP > 1 ? col & 15 : col;
        uint8_t* u0 = B + b_unit<4, NP>(c, pass, lq, 0, n, nc) * 16 + s0;
        uint32_t e[4], o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            e[h] = (bt[4 * h] >> sh & 0xFFu) | (bt[4 * h + 2] >> sh & 0xFFu) << 8;
            o[h] = (bt[4 * h + 1] >> sh & 0xFFu) | (bt[4 * h + 3] >> sh & 0xFFu) << 8;
        }
        *reinterpret_cast<uint2*>(u0) = make_uint2(e[0] | e[1] << 16, e[2] | e[3] << 16);
        *reinterpret_cast<uint2*>(u0 + mstep) = make_uint2(o[0] | o[1] << 16, o[2] | o[3] << 16);
    }
}

// Zero the B units of the groups past a row's end ([P, 4 * NCH)) in every
// column of every pass (n_sets copies of set_bytes each, from B).
template <int BITS, int NP>
__device__ __forceinline__ void zero_pad(int P, int NCH, int nc, uint8_t* B, int n_sets, size_t set_bytes, int t0,
                                         int tstep) {
    constexpr int NM = I8Codec<BITS>::NM;
    const int ng = NCH * 4 - P;
    const int per_set = ng * NP * NM * nc;
    for (int u = t0; u < per_set * n_sets; u += tstep) {
        const int set = u / per_set;
        int r = u - set * per_set;
        const int n = r % nc;
        r /= nc;
        const int m = r % NM;
        r /= NM;
        const int pass = r % NP;
        const int g = P + r / NP;
        *reinterpret_cast<uint4*>(B + set * set_bytes + b_unit<BITS, NP>(g >> 2, pass, g & 3, m, n, nc) * 16) =
            make_uint4(0u, 0u, 0u, 0u);
    }
}

// Router rows e = part, part + nparts, ... for all T tokens (as the other
// fused kernel): every thread holds its float4s of the row, dots them with
// each token, the wave sums by DPP and the waves' sums are added in wave
// order.  kResid: every workgroup also computes the tokens' 1 / rms, with the
// same reduction order in every workgroup.
__device__ __forceinline__ float ssq4(const float4& v, float ss) {
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    return fmaf(v.w, v.w, ss);
}

template <bool kResid>
__device__ __forceinline__ void router_rows(const PipeArgs& f, PipeSync& sy) {
    const int H = f.a.H, T = f.a.T, E = f.E;
    const int lane = lane_id(), wave = wave_id();
    const int n4 = H >> 2;
    bool first = true;
    for (int e = blockIdx.x; e < E; e += gridDim.x) {
        const float4* w4 = reinterpret_cast<const float4*>(f.router_w + (size_t)e * H);
        float4 wr[kRowF4];
#pragma unroll
        for (int k = 0; k < kRowF4; ++k) {
            const int i = threadIdx.x + k * kPT;
            wr[k] = i < n4 ? w4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int t = 0; t < T; ++t) {
            const float4* x4 = reinterpret_cast<const float4*>(f.x + (size_t)t * H);
            float acc = 0.f, ss = 0.f;
#pragma unroll
            for (int k = 0; k < kRowF4; ++k) {
                const int i = threadIdx.x + k * kPT;
                if (i < n4) {
                    const float4 v = x4[i];
                    acc = fmaf(wr[k].x, v.x, acc);
                    acc = fmaf(wr[k].y, v.y, acc);
                    acc = fmaf(wr[k].z, v.z, acc);
                    acc = fmaf(wr[k].w, v.w, acc);
                    if (kResid) ss = ssq4(v, ss);
                }
            }
            acc = group_sum<kWave>(acc);
            if (lane == 0) sy.gemv_red[t][wave] = acc;
            if (kResid && first) {
                ss = group_sum<kWave>(ss);
                if (lane == 0) sy.gemv_ssq[t][wave] = ss;
            }
        }
        __syncthreads();
        if ((int)threadIdx.x < T) {
            float z = 0.f;
            for (int w = 0; w < kPW; ++w) z += sy.gemv_red[threadIdx.x][w];
            if (kResid) {
                if (first) {
                    float q = 0.f;
                    for (int w = 0; w < kPW; ++w) q += sy.gemv_ssq[threadIdx.x][w];
                    sy.xinv[threadIdx.x] = 1.0f / sqrtf(q / (float)H + f.eps);
                }
                z *= sy.xinv[threadIdx.x];              // W . (x / rms) = (W . x) / rms
            }
            store_device(f.scores + (size_t)threadIdx.x * E + e, 1.0f / (1.0f + expf(-z)));
        }
        __syncthreads();
        first = false;
    }
    if (kResid && first) {                              // no router row here: the norms alone
        for (int t = 0; t < T; ++t) {
            const float4* x4 = reinterpret_cast<const float4*>(f.x + (size_t)t * H);
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < kRowF4; ++k) {
                const int i = threadIdx.x + k * kPT;
                if (i < n4) ss = ssq4(x4[i], ss);
            }
            ss = group_sum<kWave>(ss);
            if (lane == 0) sy.gemv_ssq[t][wave] = ss;
        }
        __syncthreads();
        if ((int)threadIdx.x < T) {
            float q = 0.f;
            for (int w = 0; w < kPW; ++w) q += sy.gemv_ssq[threadIdx.x][w];
            sy.xinv[threadIdx.x] = 1.0f / sqrtf(q / (float)H + f.eps);
        }
        __syncthreads();
    }
}

// Stage the T token rows of x as 24-bit B operands (whole workgroup).  Token
// t's exponent comes from its largest |x| (times 1 / rms in the residual
// form); xu[t] = 2^-(e_t + kShift).  x is read once when it fits the
// registers, else twice (a max pass and a convert pass).
template <int BITS, int NP, bool kResid>
__device__ __forceinline__ void stage_x(const PipeArgs& f, PipeSync& sy, uint8_t* XB) {
    using C = I8Codec<BITS>;
    const int H = f.a.H, T = f.a.T, nc = f.nc;
    const int H4 = H >> 2, total4 = T * H4;
    const float4* x4 = reinterpret_cast<const float4*>(f.x);
    const bool single = total4 <= kStageX4 * kPT;
    float4 v[kStageX4];
    for (int b0 = 0; b0 < total4; b0 += kStageX4 * kPT) {
#pragma unroll
        for (int u = 0; u < kStageX4; ++u) v[u] = x4[min(b0 + (int)threadIdx.x + u * kPT, total4 - 1)];
#pragma unroll
        for (int u = 0; u < kStageX4; ++u) {
            const int i4 = b0 + (int)threadIdx.x + u * kPT;
            if (i4 < total4) {
                const float m = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
                __hip_atomic_fetch_max(&sy.cmax[i4 / H4], __float_as_uint(m), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < T) {
        float m = __uint_as_float(sy.cmax[threadIdx.x]);
        if (kResid) m *= sy.xinv[threadIdx.x];          // rounding is monotonic: max |x / rms| = max |x| / rms
        const int e = q24_exponent(m);
        sy.cmax[threadIdx.x] = (unsigned)e;             // the exponent from here on
        sy.xu[threadIdx.x] = ldexpf(1.0f, -e - C::kShift);
    }
    __syncthreads();
    for (int b0 = 0; b0 < total4; b0 += kStageX4 * kPT) {
        if (!single) {
#pragma unroll
            for (int u = 0; u < kStageX4; ++u) v[u] = x4[min(b0 + (int)threadIdx.x + u * kPT, total4 - 1)];
        }
#pragma unroll
        for (int u = 0; u < kStageX4; ++u) {
            const int i4 = b0 + (int)threadIdx.x + u * kPT;
            if (i4 < total4) {
                const int t = i4 / H4;
                float sc = ldexpf(1.0f, (int)sy.cmax[t]);
                if (kResid) sc *= sy.xinv[t];
                const float4 vv = make_float4(v[u].x * sc, v[u].y * sc, v[u].z * sc, v[u].w * sc);
                scatter24<BITS, NP>(vv, (i4 - t * H4) * 4, t, nc, XB);
            }
        }
    }
    const int P = H / C::CW;
    zero_pad<BITS, NP>(P, (P + 3) / 4, nc, XB, 1, 0, threadIdx.x, kPT);
}

// ------------------------------------------------------------- the schedule
//
// Units: GU(j) and DN(j) for slots j < n, in the order of the file comment.
// A streaming wave's items of GU(j): the workgroup's tiles of slot j (tile i
// = pairs 8i .. 8i+7: gate rows 0-7 and up rows 8-15 of a 16-row MFMA tile),
// and of each tile the K-chunks c with (c + rot_j) % kSW == wave.  Its items
// of DN(j): the K-chunks of the workgroup's <= 32 down rows, the same way.

struct Geo {
    int n;                         // slots
    int lag;                       // DN(j) follows GU(j + lag)
    int NT;                        // gate/up tiles per expert (I / 8)
    int NCHg, NCHd;                // K-chunks of a gate/up row and of a down row
    int rd;                        // down rows of this workgroup
    int nwg, b;
    int nwg_mask, nwg_log;         // nwg - 1 and log2(nwg) when nwg is a power of two, else -1
};

__device__ __forceinline__ void unit_of(int u, int n, int lag, int& kind, int& j) {
    if (n <= lag) {
        kind = u < n ? 0 : 1;
        j = u < n ? u : u - n;
        return;
    }
    if (u < lag) {
        kind = 0;
        j = u;
    } else if (u < lag + 2 * (n - lag)) {
        const int k = u - lag;
        kind = k & 1;
        j = kind == 0 ? lag + (k >> 1) : (k >> 1);
    } else {
        kind = 1;
        j = n - lag + (u - lag - 2 * (n - lag));
    }
}

// Tiles of slot j that workgroup b takes: i = i0, i0 + nwg, ... < NT.
__device__ __forceinline__ int tiles_of(const Geo& g, int j, int& i0) {
    if (g.nwg_mask >= 0) {                              // (the usual case: 256 compute units)
        i0 = (g.b - j * g.NT) & g.nwg_mask;
        return i0 < g.NT ? ((g.NT - 1 - i0) >> g.nwg_log) + 1 : 0;
    }
    const int base = (j * g.NT) % g.nwg;                // j * NT < 2^31 (slots <= 520, NT <= 2048)
    i0 = (g.b - base + g.nwg) % g.nwg;
    return i0 < g.NT ? (g.NT - 1 - i0) / g.nwg + 1 : 0;
}

// K-chunks of wave w: the contiguous range (w + rot) % kSW of kSW balanced
// ranges, c = c0 .. c0 + count - 1.  (Contiguous ranges keep the waves of a
// workgroup spread over the whole row at any moment; with every workgroup in
// step on the same expert, interleaved chunks would crowd a narrow window of
// every row and so a few HBM channels.)
__device__ __forceinline__ int chunks_of(int NCH, int rot, int w, int& c0) {
    const int r = (w + rot) % kSW;
    c0 = r * NCH / kSW;
    return (r + 1) * NCH / kSW - c0;
}

// the rotation of the ranges for slot j (spreads uneven ranges over the waves)
__device__ __forceinline__ int rot_of(int j) { return j % kSW; }

// Every item issues exactly two 16-byte loads per lane, so the wait before
// each use is a static count: a gate/up item covers two consecutive K-chunks
// of the wave's range (the second a repeat of the first, computed as zero,
// past the range's end), a down item one K-chunk of both row tiles.  A unit
// where a wave has no item still takes one position of its stream (a padding
// item: valid loads, no compute).
//
// A streaming wave's items are listed in LDS once per launch, so the stream
// itself does no schedule arithmetic: per item one word of flags and one row
// index,
//   word 0: j | kind << 10 | pad << 11 | last << 12 | two << 13 | c << 14 | tile << 22
//   word 1: gate/up: eid * I + 8 * i (the tile's first pair); down: eid * H + dr0
// (j < 1024 slots, c < 256 chunks, tile < 1024; last = the wave's last item of
// the tile (gate/up) or unit (down); two = the item's second chunk is in range).
constexpr uint32_t kItemPad = 1u << 11, kItemLast = 1u << 12, kItemTwo = 1u << 13;
__device__ __forceinline__ int item_j(uint32_t d) { return d & 1023; }
__device__ __forceinline__ int item_kind(uint32_t d) { return (d >> 10) & 1; }
__device__ __forceinline__ int item_c(uint32_t d) { return (d >> 14) & 255; }
__device__ __forceinline__ int item_tile(uint32_t d) { return d >> 22; }

// Items of wave w per workgroup at most (the host sizes the lists with it).
__host__ __device__ __forceinline__ int max_items_of(int n_max, int ntile_max, int NCHg, int NCHd) {
    const int per_g = ntile_max * (((NCHg + kSW - 1) / kSW + 1) / 2);
    const int per_d = (NCHd + kSW - 1) / kSW;
    return n_max * ((per_g > 1 ? per_g : 1) + (per_d > 1 ? per_d : 1));
}

// Lists wave w's items of units [0, nu) in L (the lanes take one unit each,
// a prefix sum over the lanes places them); returns the item count.
template <typename EidOf>
__device__ __forceinline__ int build_items(const Geo& g, int w, int nu, uint2* L, EidOf eid_of, int I, int H,
                                           int dr0) {
    const int lane = threadIdx.x & (kWave - 1);
    int base = 0;
    for (int u0 = 0; u0 < nu; u0 += kWave) {
        const int u = u0 + lane;
        int kind = 0, j = 0, c0 = 0, cnt = 0, i0 = 0, ntile = 0, nit = 0, n_items = 0;
        if (u < nu) {
            unit_of(u, g.n, g.lag, kind, j);
            if (kind == 0) {
                ntile = tiles_of(g, j, i0);
                cnt = chunks_of(g.NCHg, rot_of(j), w, c0);
                nit = ntile > 0 ? (cnt + 1) >> 1 : 0;
            } else {
                ntile = 1;
                cnt = chunks_of(g.NCHd, rot_of(j), w, c0);
                nit = g.rd > 0 ? cnt : 0;
            }
            n_items = nit > 0 ? ntile * nit : 1;
        }
        const int incl = wave_scan_incl(n_items);        // inclusive prefix sum over the lanes (DPP)
        if (u < nu) {
            int k = base + incl - n_items;
            const uint32_t jk = (uint32_t)j | (uint32_t)kind << 10;
            const uint32_t eid = (uint32_t)eid_of(j);
            if (nit == 0) {
                L[k] = make_uint2(jk | kItemPad, kind == 0 ? eid * I : eid * H + dr0);
            } else {
                for (int tile = 0; tile < ntile; ++tile) {
                    const uint32_t row = kind == 0 ? eid * I + 8 * (i0 + tile * g.nwg) : eid * H + dr0;
                    for (int ci = 0; ci < nit; ++ci) {
                        const int c = c0 + (kind == 0 ? 2 * ci : ci);
                        const uint32_t fl = (ci == nit - 1 ? kItemLast : 0u) |
                                            (kind == 0 && c + 1 < c0 + cnt ? kItemTwo : 0u);
                        L[k++] = make_uint2(jk | fl | (uint32_t)c << 14 | (uint32_t)tile << 22, row);
                    }
                }
            }
        }
        base += __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave));
    }
    return base;
}

// Worklist index of slot j (the shared experts sort last in the worklist,
// but take the first slots of the schedule).
__device__ __forceinline__ int wl_index(int j, int S, int n_act) { return j < S ? n_act - S + j : j - S; }

// ---------------------------------------------------------------- the kernel

template <int BITS, int NP, bool kTopP, bool kResid>
__global__ __launch_bounds__(kPT) void layer_pipe_kernel(const PipeArgs f) {
    using C = I8Codec<BITS>;
    constexpr int NM = C::NM;
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ PipeSync sy;
#ifdef MOEDEC_PIPE_TRACE
    __shared__ unsigned long long tr[kTraceSlots];
    if (threadIdx.x < kTraceSlots) tr[threadIdx.x] = 0ull;
#endif

    const ExpertArgs& a = f.a;
    const int T = a.T, H = a.H, I = a.I, K = a.top_k, S = f.n_shared, E = f.E, slots = a.slots;
    const int lane = lane_id(), wave = wave_id();
    const int ln = lane & 15, lq = lane >> 4;
    const int nc = f.nc;
    const int nhb = f.nhb;
    const int rbg = H * BITS / 8, Pg = rbg >> 4, NCHg = (Pg + 3) >> 2;
    const int rbd = I * BITS / 8, Pd = rbd >> 4, NCHd = (Pd + 3) >> 2;
    const int nwg = gridDim.x, b = blockIdx.x;
    const int dr0 = b * H / nwg, rd = (b + 1) * H / nwg - dr0;   // b * H < 2^31
    const size_t xb_chunk = (size_t)NP * 4 * NM * nc * 16;
    const size_t hb_bytes = (size_t)NCHd * xb_chunk;   // one staged expert's h

    uint8_t* XB = dyn;
    uint8_t* HB = dyn + f.off_hb;
    int* PART = reinterpret_cast<int*>(dyn + f.off_part);   // [kNPB][ntile_max][kSW][NP][16][nc]
    PipeRoute& route = *reinterpret_cast<PipeRoute*>(dyn + f.off_route);   // overlaps HB/PART until routed
    int* p_sel = reinterpret_cast<int*>(dyn + f.off_pers);                 // [T*K]
    float* p_selw = reinterpret_cast<float*>(p_sel + T * K);               // [T*K]
    int* p_eid = reinterpret_cast<int*>(p_selw + T * K);                   // [max_active]
    int* p_seg = p_eid + a.max_active;                                     // [max_active + 1]
    int* p_asn = p_seg + a.max_active + 1;                                 // [T*slots]
    float* GSC = reinterpret_cast<float*>(dyn + f.off_gsc);                // [max_active][ntile_max][16]
    float* DSC = reinterpret_cast<float*>(dyn + f.off_dsc);                // [max_active][32]

    if (threadIdx.x < kCols) sy.cmax[threadIdx.x] = 0u;
    if (threadIdx.x < kNPB) {
        sy.gu_cnt[threadIdx.x] = 0;
        sy.gu_free[threadIdx.x] = 0;
        sy.fin_cum[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) {
        sy.fin_done = 0;
        sy.next_slot = 0;
        sy.rows_listed = 0;
    }
    if (threadIdx.x < kNHBMax) {
        sy.hb_ready[threadIdx.x] = 0;
        sy.hb_done[threadIdx.x] = 0;
    }
    const int spin_cap = f.ws[MOEDEC_FUSED_WS_SPIN];
    Gates gates{f.ws, spin_cap > 0 ? spin_cap : kSpinDefault, 0ull};
    const int lds_cap = spin_cap > 0 ? 16 * spin_cap : kLdsSpin;
    gates.init();
    if (wave == 0) PIPE_MARK(tr, 0);

    // ---- phase 1: router rows, the scores exchange's arrival, x staged
    router_rows<kResid>(f, sy);
    {   // this workgroup's share of h: the sentinel, settled together with the scores
        const int nh = T * slots * I;
        const int h0 = (int)((long long)nh * b / nwg), h1 = (int)((long long)nh * (b + 1) / nwg);
        for (int i = h0 + (int)threadIdx.x; i < h1; i += kPT)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(f.h) + i, kSentinel, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);                      // this wave's score and sentinel stores have completed
    __syncthreads();
    if (wave == kPW - 1) gates.add(0, 1ull);
    if (wave == 0) PIPE_MARK(tr, 1);
    stage_x<BITS, NP, kResid>(f, sy, XB);
    __syncthreads();
    if (wave == 0) PIPE_MARK(tr, 2);

    Geo g;
    g.n = S;                       // before routing only the shared slots are known
    g.lag = kLag;
    g.NT = I / 8;
    g.NCHg = NCHg;
    g.NCHd = NCHd;
    g.rd = rd;
    g.nwg = nwg;
    g.nwg_mask = (nwg & (nwg - 1)) == 0 ? nwg - 1 : -1;
    g.nwg_log = g.nwg_mask >= 0 ? __builtin_ctz(nwg) : -1;
    g.b = b;

    // streaming waves: this lane's part of an item
    const int tcol = ln;                                 // B column read by this lane
    auto eid_of = [&](int j) { return j < S ? E + j : p_eid[j - S]; };
    // this lane's part of an item's two loads (a padding item's row and chunk are valid too)
    const uint8_t* gu_lane = (ln < 8 ? a.w_gate : a.w_up) + (size_t)(ln & 7) * rbg;
    const size_t dn_lane0 = (size_t)min(ln, max(rd - 1, 0)) * rbd;
    const size_t dn_lane1 = (size_t)min(16 + ln, max(rd - 1, 0)) * rbd;
    auto issue = [&](uint32_t d, uint32_t row, uint4* dst) {
        const int c = item_c(d);
        if (item_kind(d) == 0) {
            const uint8_t* p = gu_lane + (size_t)row * rbg;
            const int c1 = (d & kItemTwo) ? c + 1 : c;
            dst[0] = ld16(p + min(c * 4 + lq, Pg - 1) * 16);
            dst[1] = ld16(p + min(c1 * 4 + lq, Pg - 1) * 16);
        } else {
            const uint8_t* p = a.w_down + (size_t)row * rbd + min(c * 4 + lq, Pd - 1) * 16;
            dst[0] = ld16(p + dn_lane0);
            dst[1] = ld16(p + dn_lane1);
        }
    };
    uint2* items = reinterpret_cast<uint2*>(dyn + f.off_items) + (size_t)(wave < kSW ? wave : 0) * f.max_items;

    // ---- streaming waves that route no token fill their ring with the
    // shared experts' first gate/up items before routing
    const bool streaming = wave < kSW;
    const int n_route_waves = T < kPW ? T : kPW;
    const bool routes = wave >= kPW - n_route_waves;
    uint4 ring[kRing][2];
    if (streaming && !routes && S > 0) {                 // unit 0 = GU(shared slot 0) whatever the routing
        const int n0 = build_items(g, wave, 1, items, eid_of, I, H, dr0);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");   // the lanes' list writes
        if (!(items[0].x & kItemPad)) {
#pragma unroll
            for (int w = 0; w < kRing; ++w)
                if (w < n0) issue(items[w].x, items[w].y, ring[w]);
        }
    }

    // ---- phase 2: routing (the last waves route, the union on the last wave)
    if (routes) gates.wait(0, gates.launch + 1ull);
    if (!kTopP && T == 1) {
        // One token under top-k: its K experts are distinct, so the batch
        // union is them in ascending order, one assignment each (slot k is
        // assignment k), then the shared experts; the routing wave writes it
        // straight to the arrays the launch reads.
        if (wave == kPW - 1) {
            constexpr int NV = kPipeExperts / kWave, NV4 = NV < 4 ? NV : 4;
            if (NV == NV4 || E <= NV4 * kWave)
                route_one_token<NV4, kCols, kPipeExperts, kPW, true, false>(f.scores, f.bias, 0, E, f.n_group,
                                                                        f.topk_group, K, f.rsf, 1.f, route);
            else
                route_one_token<NV, kCols, kPipeExperts, kPW, true, false>(f.scores, f.bias, 0, E, f.n_group,
                                                                       f.topk_group, K, f.rsf, 1.f, route);
            wave_lds_sync();                             // this wave's selection writes
            const int e = lane < K ? route.sel[lane] : INT_MAX;
            const float w = lane < K ? route.selw[lane] : 0.f;
            int rank = 0;
            for (int k = 0; k < K; ++k) rank += __builtin_amdgcn_readlane(e, k) < e;
            if (lane < K) {
                p_sel[lane] = e;
                p_selw[lane] = w;
                p_eid[rank] = e;
                p_seg[rank] = rank;
                p_asn[rank] = lane;
            } else if (lane < K + S) {
                p_eid[lane] = E + (lane - K);
                p_seg[lane] = lane;
                p_asn[lane] = lane;
            }
            if (lane == 0) {
                p_seg[K + S] = K + S;
                sy.n_slots = K + S;
                sy.n_assign = K + S;
            }
        }
    } else {
        route_select_block<kCols, kPipeExperts, kPW, true, kTopP, true>(f.scores, f.bias, T, E, f.n_group,
                                                                       f.topk_group, K, S, f.rsf, f.top_p, route);
        // the routing outputs the rest of the launch reads, out of the region HB / PART reuse
        const int n_act0 = route.n_active;
        const int A0 = route.n_assign;
        for (int i = threadIdx.x; i < T * K; i += kPT) {
            p_sel[i] = route.sel[i];
            p_selw[i] = route.selw[i];
        }
        for (int i = threadIdx.x; i <= n_act0; i += kPT) {
            if (i < n_act0) p_eid[i] = route.eid[i];
            p_seg[i] = route.seg[i];
        }
        for (int i = threadIdx.x; i < A0; i += kPT) p_asn[i] = route.assign[i];
        if (threadIdx.x == 0) {
            sy.n_slots = n_act0;
            sy.n_assign = A0;
        }
    }
    __syncthreads();
    const int n_act = sy.n_slots;
    const int A = sy.n_assign;
    // HB's padding groups are zero in every staged buffer (staging writes only
    // valid groups); a row of whole K-chunks has none
    if (Pd < 4 * NCHd) {
        zero_pad<BITS, NP>(Pd, NCHd, nc, HB, nhb, hb_bytes, threadIdx.x, kPT);
        __syncthreads();
    }
    g.n = n_act;
    g.lag = nhb >= n_act ? n_act : kLag;             // every slot has a buffer: all gate/up first
    if (wave == 0) PIPE_MARK(tr, 3);

    // assignment of (token t, slot j), or -1
    auto assign_of = [&](int j, int t) {
        const int wi = wl_index(j, S, n_act);
        const int s0 = p_seg[wi], s1 = p_seg[wi + 1];
        int found = -1;
        for (int q = s0; q < s1; ++q)
            if (p_asn[q] / slots == t) found = p_asn[q];
        return found;
    };

    const int nc_gu = NCHg < kSW ? NCHg : kSW;          // streaming waves with chunks of a gate/up tile
    const int nc_dn = rd > 0 ? (NCHd < kSW ? NCHd : kSW) : 0;   // ... of a down unit (none without rows)
    const int ncolT = kPieces * T;                       // B columns in use

    auto staging = [&](bool builder) {
    // ================================================ staging
    // Slots are claimed one at a time from an LDS counter by every staging
    // wave: the stagers, and the finalizer once it has finalized every slot
    // (at one token it is done well before the last slots are staged).  The
    // first stager ("builder") loads the down row scales and lists the rows.
    static_assert(kStg + kNStg == kPW && kFin == kSW && kStg == kFin + 1, "wave roles");
    const int I4 = I >> 2;
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
        f.h, (short)0, (int)((size_t)T * slots * I * sizeof(float)), kBufWord3);
    if (builder) {
        // the down row scales of this workgroup's rows for every slot, to LDS once
        // (the streaming waves read a slot's after its release)
        for (int base = 0; base < n_act * 32; base += 8 * kWave) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {                // every load first, then the stores
                const int idx = min(base + k * kWave + lane, max(n_act * 32 - 1, 0));
                const int j = idx >> 5, r = idx & 31;
                v[k] = a.s_down[(size_t)eid_of(min(j, n_act - 1)) * H + dr0 + min(r, max(rd - 1, 0))];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int idx = base + k * kWave + lane;
                if (idx < n_act * 32) DSC[idx] = (idx & 31) < rd ? v[k] : 0.f;
            }
        }
    }
    const bool one = I4 <= kStageH4 * kWave;            // a row is read once, else twice
    // float4 k of a lane in a piece of the row: int4 codes take 16 consecutive
    // values per lane (4 float4), so each staged operand gets 8-byte writes
    auto c4_of = [&](int c40, int k) {
        return BITS == 4 ? c40 + 4 * ((k >> 2) * kWave + lane) + (k & 3) : c40 + k * kWave + lane;
    };
    auto load_row = [&](int as, int c40, u32x4* v) {
#pragma unroll
        for (int k = 0; k < kStageH4; ++k) {
            const int c4 = c4_of(c40, k);
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(hrs, (as * I4 + min(c4, I4 - 1)) * 16, 0, kCoherent);
        }
    };
    auto any_stale = [&](const u32x4* v) {
        bool st = false;
#pragma unroll
        for (int k = 0; k < kStageH4; ++k)
            st = st || v[k].x == kSentinel || v[k].y == kSentinel || v[k].z == kSentinel || v[k].w == kSentinel;
        return __ballot(st) != 0;
    };
    // loads of a row piece until no sentinel is left (bounded)
    auto settle = [&](int as, int c40, u32x4* v) {
        for (int tries = 0; any_stale(v); ++tries) {
            if (tries >= gates.spin_max) {
                raise_error(f.ws);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            load_row(as, c40, v);
        }
    };
    auto piece_max = [&](const u32x4* v, int c40, float w) {
        float mx = 0.f;
#pragma unroll
        for (int k = 0; k < kStageH4; ++k) {
            if (c4_of(c40, k) < I4) {
                const float m4 = fmaxf(fmaxf(fabsf(__uint_as_float(v[k].x) * w), fabsf(__uint_as_float(v[k].y) * w)),
                                       fmaxf(fabsf(__uint_as_float(v[k].z) * w), fabsf(__uint_as_float(v[k].w) * w)));
                mx = fmaxf(mx, m4);
            }
        }
        return mx;
    };
    // The rows (slot j, token t, assignment as) in slot order, listed once by
    // the builder: x = as, y = j | t << 10 | first << 20 | last << 21
    // (first / last: the slot's first / last row; every slot has one), and
    // slot j's rows are r0[j] .. r0[j + 1] - 1.
    uint2* rl = reinterpret_cast<uint2*>(dyn + f.off_rows);
    int* r0 = reinterpret_cast<int*>(rl + f.max_rows);
    if (builder) {
        int n = 0;
        for (int j = 0; j < n_act; ++j) {
            const int m = lane < T ? assign_of(j, lane) : -1;
            const unsigned long long bal = __ballot(m >= 0);
            const int pos = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
            const int cnt = __builtin_popcountll(bal);
            if (m >= 0)
                rl[n + pos] = make_uint2((uint32_t)m, (uint32_t)j | (uint32_t)lane << 10 |
                                                          (pos == 0 ? 1u << 20 : 0u) |
                                                          (pos == cnt - 1 ? 1u << 21 : 0u));
            if (lane == 0) r0[j] = n;
            n += cnt;
        }
        if (lane == 0) r0[n_act] = n;
        lds_signal_set(&sy.rows_listed, 1);          // (publishes the lanes' list writes)
    } else {
        lds_wait_ge(&sy.rows_listed, 1, f.ws, lds_cap);
    }
    const int nrows = __builtin_amdgcn_readfirstlane(r0[n_act]);
    auto row_at = [&](int r) {                       // (wave-uniform fields)
        const uint2 e = rl[r];
        return make_uint2((uint32_t)__builtin_amdgcn_readfirstlane((int)e.x),
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)e.y));
    };
    // Stage row r, whose first (or only) piece is in v: the slot's buffer is
    // taken on its first row and released on its last.
    auto stage_row = [&](int r, u32x4* v) {
        const uint2 e = row_at(r);
        const int as = (int)e.x, j = e.y & 1023, t = (e.y >> 10) & 1023;
        const bool first = (e.y >> 20) & 1, last = (e.y >> 21) & 1;
        const int hb = j % nhb;
        uint8_t* B = HB + hb * hb_bytes;
        if (first) PIPE_MARK(tr, 35 + j);
        const int sl = as - (as / slots) * slots;
        const float w = sl < K ? p_selw[t * K + sl] : 1.0f;
        float mx = 0.f;
        for (int c40 = 0; c40 < I4; c40 += kStageH4 * kWave) {
            if (c40 > 0) load_row(as, c40, v);
            settle(as, c40, v);
            if (first && c40 == 0) {
                PIPE_MARK(tr, 66 + j);
                lds_wait_ge(&sy.hb_done[hb], (j / nhb) * nc_dn, f.ws, lds_cap);    // its previous slot is consumed
                if (lane < T) sy.dsl[hb][lane] = 0.f;            // tokens not routed here (routed ones below)
                PIPE_MARK(tr, 75 + j);
            }
            mx = fmaxf(mx, piece_max(v, c40, w));
        }
        mx = wave_max(mx);
        const int ex = q24_exponent(mx);
        const float ws = w * ldexpf(1.0f, ex);
        for (int c40 = 0; c40 < I4; c40 += kStageH4 * kWave) {
            if (!one) load_row(as, c40, v);
            if constexpr (BITS == 4) {
                static_assert(kStageH4 % 4 == 0, "whole quads");
#pragma unroll
                for (int k = 0; k < kStageH4; k += 4) {
                    const int c4 = c4_of(c40, k);            // a quad lies wholly inside the row (I % 32 == 0)
                    if (c4 < I4) scatter24_quad4<NP>(v + k, ws, c4 * 4, t, nc, B);
                }
            } else {
#pragma unroll
                for (int k = 0; k < kStageH4; ++k) {
                    const int c4 = c4_of(c40, k);
                    if (c4 < I4) {
                        const float4 hv = make_float4(__uint_as_float(v[k].x) * ws, __uint_as_float(v[k].y) * ws,
                                                      __uint_as_float(v[k].z) * ws, __uint_as_float(v[k].w) * ws);
                        scatter24<BITS, NP>(hv, c4 * 4, t, nc, B);
                    }
                }
            }
        }
        if (lane == 0) sy.dsl[hb][t] = ldexpf(1.0f, -ex - C::kShift);
        if (last) {
            lds_signal_set(&sy.hb_ready[hb], j + 1);
            PIPE_MARK(tr, 45 + j);
        }
    };
    // Rows of one piece alternate between two register buffers: row r + 1
    // is in flight while row r is staged, which keeps most of the long
    // round trip of a load behind the weight stream off the critical path.
    // A row is loaded once this workgroup's own finalizer has stored its
    // slot (every workgroup finalizes a slot at about the same time), so a
    // load seldom returns a sentinel and costs a second trip.  (Past the
    // end the last row is loaded again, so both buffers always have their
    // loads in the same order.)
    auto prefetch = [&](int r, u32x4* P) {
        const uint2 e = row_at(min(r, nrows - 1));
        lds_wait_ge(&sy.fin_done, (int)(e.y & 1023) + 1, f.ws, lds_cap);
        load_row((int)e.x, 0, P);
    };
    // The rows this wave stages, in order: the rest of its current slot,
    // then the first row of the next slot it claims (nrows: no slot left).
    int slot_end = 0;
    auto next_row = [&](int r) {
        if (r + 1 < slot_end) return r + 1;
        int j = 0;
        if (lane == 0) j = __hip_atomic_fetch_add(&sy.next_slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        j = __builtin_amdgcn_readfirstlane(j);
        if (j >= n_act) return nrows;
        slot_end = r0[j + 1];
        return r0[j];
    };
    if (nrows > 0 && one) {
        u32x4 pa[kStageH4], pb[kStageH4];
        int ra = next_row(-1);
        prefetch(ra, pa);
        while (ra < nrows) {
            const int rb = next_row(ra);
            prefetch(rb, pb);
            stage_row(ra, pa);
            if (rb >= nrows) break;
            ra = next_row(rb);
            prefetch(ra, pa);
            stage_row(rb, pb);
        }
    } else if (nrows > 0) {
        u32x4 v[kStageH4];
        for (int r = next_row(-1); r < nrows; r = next_row(r)) {
            load_row((int)row_at(r).x, 0, v);
            stage_row(r, v);
        }
    }
    };

    if (streaming) {
        // ================================================ streaming waves
        // The ring is filled from the start whatever was prefetched before
        // routing (those items come again, now from L2): every slot then has
        // its two loads in a static order and the waits in the loop are
        // static counts.  The wave's item list is read 64 items at a time into
        // a register (lane k holds item base + k).
        const int nitems = build_items(g, wave, 2 * n_act, items, eid_of, I, H, dr0);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");   // the lanes' list writes
        int blk_base = 0, n_issued = 0;
        uint2 blk = items[min(lane, nitems - 1)];
        auto take = [&](uint32_t& d, uint32_t& row) {  // the next item to issue (past the end: the last again)
            const int k = n_issued < nitems ? n_issued : nitems - 1;
            if (k - blk_base >= kWave) {
                blk_base += kWave;
                blk = items[min(blk_base + lane, nitems - 1)];
            }
            d = (uint32_t)__builtin_amdgcn_readlane((int)blk.x, k - blk_base);
            row = (uint32_t)__builtin_amdgcn_readlane((int)blk.y, k - blk_base);
            ++n_issued;
        };
        uint32_t ring_d[kRing];
#pragma unroll
        for (int w = 0; w < kRing; ++w) {
            uint32_t row;
            take(ring_d[w], row);
            issue(ring_d[w], row, ring[w]);
        }
        const i32x4 zero4 = {0, 0, 0, 0};
        i32x4 acc[NP];
        i32x4 dacc[2][NP];
        floatx4 tot[2][NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            acc[p] = zero4;
            dacc[0][p] = dacc[1][p] = zero4;
            tot[0][p] = tot[1][p] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        int hb_cur = -1;                                 // DN unit whose staged h this wave has waited for
        int hb_j = 0;                                    // ... and its staged buffer (hb_cur % nhb)
#ifdef MOEDEC_PIPE_TRACE
        if (wave == 0) PIPE_MARK(tr, 4);
        int mark_u = -1, mark_key = -1;
#endif
        auto compute = [&](uint32_t d, const uint4* cur) {
#ifdef MOEDEC_PIPE_TRACE
            if (wave == 0 && (int)(d & 2047) != mark_key) {
                mark_key = d & 2047;
                ++mark_u;
                PIPE_MARK(tr, 5 + mark_u);
            }
#endif
            if (d & kItemPad) return;
            const int j = item_j(d), c = item_c(d);
            if (item_kind(d) == 0) {
                const bool two = (d & kItemTwo) != 0;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    if (h2 == 1 && !two) break;
                    const uint8_t* B = XB + (size_t)(c + h2) * xb_chunk;
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
#pragma unroll
                        for (int m = 0; m < NM; ++m) {
                            const i32x4 bv = *reinterpret_cast<const i32x4*>(
                                B + (((p * 4 + lq) * NM + m) * nc + min(tcol, nc - 1)) * 16);
                            acc[p] = mma(operand<BITS>(cur[h2], m), bv, acc[p]);
                        }
                    }
                }
                if (d & kItemLast) {                     // this wave's part of the tile: to LDS
                    const int pb = j % kNPB;
                    lds_wait_ge(&sy.gu_free[pb], j - kNPB + 1, f.ws, lds_cap);
                    int* part = PART + ((((size_t)pb * f.ntile_max + item_tile(d)) * kSW + wave) * NP) * 16 * nc;
                    if (tcol < nc) {
#pragma unroll
                        for (int p = 0; p < NP; ++p)
#pragma unroll
                            for (int ii = 0; ii < 4; ++ii) part[(p * 16 + 4 * lq + ii) * nc + tcol] = acc[p][ii];
                    }
#pragma unroll
                    for (int p = 0; p < NP; ++p) acc[p] = zero4;
                    lds_signal_add(&sy.gu_cnt[pb], 1);
                }
            } else {
                if (hb_cur != j) {
                    hb_j = j % nhb;
                    lds_wait_ge(&sy.hb_ready[hb_j], j + 1, f.ws, lds_cap);
                    hb_cur = j;
                }
                const int hb = hb_j;
                const uint8_t* B = HB + hb * hb_bytes + (size_t)c * xb_chunk;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        const i32x4 bv =
                            *reinterpret_cast<const i32x4*>(B + (((p * 4 + lq) * NM + m) * nc + min(tcol, nc - 1)) * 16);
                        dacc[0][p] = mma(operand<BITS>(cur[0], m), bv, dacc[0][p]);
                        dacc[1][p] = mma(operand<BITS>(cur[1], m), bv, dacc[1][p]);
                    }
                }
                if (d & kItemLast) {                     // this wave's part of DN(j): scale and add
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        const int col = 16 * p + tcol;
                        const int t = col / kPieces;
                        const float ds = (col < ncolT && t < T) ? sy.dsl[hb][t] : 0.f;
                        const float pw = (col % kPieces) == 0 ? 65536.f : (col % kPieces) == 1 ? 256.f : 1.f;
#pragma unroll
                        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                            for (int ii = 0; ii < 4; ++ii) {
                                const int r = min(bb * 16 + 4 * lq + ii, 31);
                                tot[bb][p][ii] += (float)dacc[bb][p][ii] * (DSC[j * 32 + r] * ds * pw);
                            }
                        dacc[0][p] = dacc[1][p] = zero4;
                    }
                    lds_signal_add(&sy.hb_done[hb], 1);
                }
            }
        };
        for (int n0 = 0; n0 < nitems; n0 += kRing) {     // rounds of kRing positions
#pragma unroll
            for (int w = 0; w < kRing; ++w) {
                const uint4 cur[2] = {ring[w][0], ring[w][1]};
                const uint32_t dc = ring_d[w];
                uint32_t row;
                take(ring_d[w], row);
                issue(ring_d[w], row, ring[w]);
                if (n0 + w < nitems) compute(dc, cur);
            }
        }
        if (wave == 0) PIPE_MARK(tr, 55);
        __syncthreads();                                 // (A) every wave's stream and task list is done
        // the waves' partial outputs -> LDS (the x region is free now) -> y
        float* red = reinterpret_cast<float*>(XB);       // [kSW][2][NP][16][16]
        if (tcol < nc) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int p = 0; p < NP; ++p)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        red[((((size_t)wave * 2 + bb) * NP + p) * 16 + 4 * lq + ii) * 16 + tcol] = tot[bb][p][ii];
        }
        __syncthreads();                                 // (B)
    } else if (wave == kFin) {
        // ================================================ finalizer
        // the gate/up row scales of this workgroup's tiles of every slot, to LDS
        // once (one round trip, not one per expert behind the streams' loads)
        {
            const int per = f.ntile_max * 16, total = n_act * per;
            for (int base = 0; base < total; base += 8 * kWave) {
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {                // every load first, then the stores
                    const int idx = min(base + k * kWave + lane, total - 1);
                    const int j = f.ntile_max == 1 ? idx >> 4 : idx / per;   // (one tile: per = 16)
                    const int rem = idx - j * per, tile = rem >> 4, r = rem & 15;
                    int i0;
                    const int nt = tiles_of(g, j, i0);
                    const int pair = 8 * (i0 + min(tile, max(nt - 1, 0)) * nwg) + (r & 7);
                    const size_t src = (size_t)eid_of(j) * I + min(pair, I - 1);
                    v[k] = (r & 8) ? a.s_up[src] : a.s_gate[src];
                }
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (base + k * kWave + lane < total) GSC[base + k * kWave + lane] = v[k];
            }
        }
        for (int j = 0; j < n_act; ++j) {
            int i0;
            const int nt = tiles_of(g, j, i0);
            const int pb = j % kNPB;
            const int expect = sy.fin_cum[pb] + nt * nc_gu;     // only this wave touches fin_cum
            if (lane == 0) sy.fin_cum[pb] = expect;
            lds_wait_ge(&sy.gu_cnt[pb], expect, f.ws, lds_cap);
            for (int tile = 0; tile < nt; ++tile) {
                const int i = i0 + tile * nwg;
                const int* part = PART + (((size_t)pb * f.ntile_max + tile) * kSW) * NP * 16 * nc;
                // lanes: pair = lane & 7, token t = lane >> 3 (8 tokens per round)
                for (int t0 = 0; t0 < T; t0 += 8) {
                    const int pr = lane & 7, t = t0 + (lane >> 3);
                    float gv = 0.f, uv = 0.f;
                    if (t < T) {
#pragma unroll
                        for (int q = 0; q < kPieces; ++q) {
                            const int col = kPieces * t + q;
                            const int p = NP > 1 ? col >> 4 : 0, n = NP > 1 ? col & 15 : col;
                            int sg = 0, su = 0;
                            for (int r = 0; r < kSW; ++r) {          // ranges in order: a fixed sum order
                                if ((r + 1) * NCHg / kSW == r * NCHg / kSW) continue;   // empty range
                                const int ww = (r - rot_of(j) + kSW) % kSW;             // the wave that took it
                                const int* pw = part + ((size_t)ww * NP + p) * 16 * nc;
                                sg += pw[pr * nc + n];
                                su += pw[(8 + pr) * nc + n];
                            }
                            const float sc = q == 0 ? 65536.f : q == 1 ? 256.f : 1.f;
                            gv += (float)sg * sc;
                            uv += (float)su * sc;
                        }
                    }
                    const float* gs = GSC + ((size_t)j * f.ntile_max + tile) * 16;
                    const float sgate = gs[pr], sup = gs[8 + pr];
                    if (t < T) {
                        const int as = assign_of(j, t);
                        if (as >= 0) {
                            const float gg = gv * sy.xu[t] * sgate;
                            const float uu = uv * sy.xu[t] * sup;
                            float hv = gg / (1.0f + __expf(-gg)) * uu;
                            if (hv != hv) hv = __uint_as_float(0x7FC00000u);   // never the sentinel
                            store_device(f.h + (size_t)as * I + 8 * i + pr, hv);
                        }
                    }
                }
            }
            lds_signal_set(&sy.gu_free[pb], j + 1);
            lds_signal_set(&sy.fin_done, j + 1);
            PIPE_MARK(tr, 25 + j);
        }
        staging(false);                                  // then it stages the slots still unclaimed
        __syncthreads();                                 // (A)
        __syncthreads();                                 // (B)
    } else {
        staging(wave == kStg);
        __syncthreads();                                 // (A)
        __syncthreads();                                 // (B)
    }

    // ---- the layer output: y = sum over waves and pieces, in a fixed order
    {
        const float* red = reinterpret_cast<const float*>(XB);
        for (int idx = threadIdx.x; idx < rd * T; idx += kPT) {
            const int t = idx / rd, r = idx - t * rd;
            const int bb = r >> 4, r16 = r & 15;
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < kPieces; ++q) {
                const int col = kPieces * t + q;
                const int p = NP > 1 ? col >> 4 : 0, n = NP > 1 ? col & 15 : col;
                for (int w = 0; w < kSW; ++w) s += red[((((size_t)w * 2 + bb) * NP + p) * 16 + r16) * 16 + n];
            }
            const size_t o = (size_t)t * H + dr0 + r;
            f.y[o] = s;
            if (kResid) f.x_out[o] = f.x[o] + s;        // every workgroup read x before its first slot's exchange
        }
    }

#ifdef MOEDEC_PIPE_TRACE
    __syncthreads();
    if (wave == 0) PIPE_MARK(tr, 56);
    __syncthreads();
    if (threadIdx.x < kTraceSlots) g_pipe_trace[(size_t)b * kTraceSlots + threadIdx.x] = tr[threadIdx.x];
#endif
    // Workgroup 0 writes the routing outputs last, from LDS.
    if (b == 0) {
        for (int i = threadIdx.x; i < T * K; i += kPT) {
            f.topk_idx[i] = p_sel[i];
            f.topk_w[i] = p_selw[i];
        }
        if (threadIdx.x == 0) *f.wl_n_active = n_act;
        for (int j = threadIdx.x; j <= n_act; j += kPT) {
            if (j < n_act) f.wl_expert_id[j] = p_eid[j];
            f.wl_seg[j] = p_seg[j];
        }
        for (int i = threadIdx.x; i < A; i += kPT) f.wl_assign[i] = p_asn[i];
    }
}

size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

template <int BITS, int NP>
hipError_t pipe_bits(PipeArgs f, const FusedLayerArgs& l, hipStream_t st) {
    const bool topp = f.top_p < 1.f, resid = f.x_out != nullptr;
    auto k = resid ? (topp ? layer_pipe_kernel<BITS, NP, true, true> : layer_pipe_kernel<BITS, NP, false, true>)
                   : (topp ? layer_pipe_kernel<BITS, NP, true, false> : layer_pipe_kernel<BITS, NP, false, false>);
    static size_t static_cache[2][2] = {{0, 0}, {0, 0}};     // each variant's static LDS, read once
    size_t& static_lds = static_cache[topp][resid];
    if (static_lds == 0) {
        hipFuncAttributes attr;
        hipError_t err = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(k));
        if (err != hipSuccess) return err;
        static_lds = (attr.sharedSizeBytes + 1023) & ~(size_t)1023;
    }
    constexpr int NM = I8Codec<BITS>::NM;
    const int nwg = cu_count();
    const int H = l.ex.H, I = l.ex.I, T = l.T;
    const int rd = (H + nwg - 1) / nwg;
    if (rd > 32) return hipErrorInvalidValue;                   // more output rows than two tiles hold
    if (static_lds + kLdsOnePerCu > kLdsMax) return hipErrorInvalidValue;
    const int nc = NP == 1 ? kPieces * T : 16;
    const int NCHg = ((H * BITS / 8) / 16 + 3) / 4;
    const int NCHd = ((I * BITS / 8) / 16 + 3) / 4;
    const size_t chunk = (size_t)NP * 4 * NM * nc * 16;
    const size_t xb = align16((size_t)NCHg * chunk);
    const size_t red = align16((size_t)kSW * 2 * NP * 16 * 16 * sizeof(float));
    const size_t r0 = xb > red ? xb : red;
    const size_t hb1 = (size_t)NCHd * chunk;             // one staged expert's h
    const int NT = I / 8;
    const int ntile_max = (NT + nwg - 1) / nwg;
    // the item fields' widths: slots < 1024, chunks < 256, tiles < 1024
    if (l.ex.max_active >= 1024 || NCHg > 256 || NCHd > 256 || ntile_max > 1024) return hipErrorInvalidValue;
    const size_t part = align16((size_t)kNPB * ntile_max * kSW * NP * 16 * nc * sizeof(int));
    const size_t route = align16(sizeof(PipeRoute));
    const int K = l.ex.top_k, A = T * l.ex.slots;
    const size_t pers = align16(((size_t)2 * T * K + 2 * l.ex.max_active + 1 + A) * sizeof(int));
    const size_t gsc = align16((size_t)l.ex.max_active * ntile_max * 16 * sizeof(float));
    const size_t dsc = align16((size_t)l.ex.max_active * 32 * sizeof(float));
    const int max_items = max_items_of(l.ex.max_active, ntile_max, NCHg, NCHd);
    const size_t items = align16((size_t)kSW * max_items * sizeof(uint2));
    const size_t rows = align16((size_t)A * sizeof(uint2) + ((size_t)l.ex.max_active + 1) * sizeof(int));
    // as many staged-h buffers as fit (more let the stager run further ahead)
    int nhb = kNHBMax;
    size_t hb = 0, r1 = 0, lds = 0;
    for (;; nhb -= 2) {
        hb = align16((size_t)nhb * hb1);
        r1 = hb + part > route ? hb + part : route;
        lds = r0 + r1 + pers + gsc + dsc + items + rows;
        if (static_lds + lds <= kLdsMax || nhb == 2) break;
    }
    if (static_lds + lds > kLdsMax) return hipErrorInvalidValue;
    f.nc = nc;
    f.nhb = nhb;
    f.ntile_max = ntile_max;
    f.off_hb = (int)r0;
    f.off_part = (int)(r0 + hb);
    f.off_route = (int)r0;
    f.off_pers = (int)(r0 + r1);
    f.off_gsc = (int)(r0 + r1 + pers);
    f.off_dsc = (int)(r0 + r1 + pers + gsc);
    f.off_items = (int)(r0 + r1 + pers + gsc + dsc);
    f.max_items = max_items;
    f.off_rows = (int)(r0 + r1 + pers + gsc + dsc + items);
    f.max_rows = A;
    if (lds < kLdsOnePerCu) lds = kLdsOnePerCu;
    hipError_t err = allow_lds(k, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(nwg), dim3(kPT), lds, st, f);
    return hipGetLastError();
}

}  // namespace

#ifdef MOEDEC_PIPE_TRACE
// The last launch's phase timestamps (trace builds only): workgroups x kTraceSlots.
extern "C" __attribute__((visibility("default"))) int moedec_pipe_trace_read(unsigned long long* host, int n) {
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_pipe_trace), (size_t)n * sizeof(unsigned long long), 0,
                               hipMemcpyDeviceToHost) == hipSuccess ? 0 : 3;
}
#endif

hipError_t launch_layer_pipe(int bits, const FusedLayerArgs& l, hipStream_t st) {
    if (l.T > kCols || l.E > kPipeExperts || l.act8) return hipErrorInvalidValue;
    PipeArgs f{};
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
    f.top_p = l.top_p;
    f.x_out = l.x_out;
    f.eps = l.eps;
    const bool one_pass = kPieces * l.T <= 16;
    switch (bits) {
        case 4: return one_pass ? pipe_bits<4, 1>(f, l, st) : pipe_bits<4, 3>(f, l, st);
        case 8: return one_pass ? pipe_bits<8, 1>(f, l, st) : pipe_bits<8, 3>(f, l, st);
        case 2: return one_pass ? pipe_bits<2, 1>(f, l, st) : pipe_bits<2, 3>(f, l, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moedec
