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
// tens of microseconds.  Every separately started streaming phase pays a
// ramp of a few microseconds (first loads in flight, last loads draining,
// stragglers), so this kernel streams all expert bytes of a workgroup as ONE
// continuous sequence.  One persistent workgroup per compute unit:
//   1. router rows e = b, b + nwg, ...: s = sigmoid(W_r x), stored for all;
//      arrive at the grid barrier; stage x as MFMA B operands in LDS; wait;
//   2. every workgroup routes the batch itself from the scores (route.h), so
//      the worklist needs no second exchange (workgroup 0 writes the routing
//      and worklist outputs from LDS at the very end);
//   3. the stream, through one ring of in-flight 16-byte loads per wave:
//      gate/up of every active expert (this workgroup's rows
//      [b*I/nwg, (b+1)*I/nwg) of each, expert by expert, its h kept in LDS and
//      written out at once after the last block, then counted as done), then
//      down + combine for this workgroup's output rows [b*H/nwg, (b+1)*H/nwg)
//      over every expert, once every workgroup's h is out.
// Inside the stream the workgroup synchronises only through LDS: loads in
// flight are never waited for at a sync.  That matters on this GPU, where a
// wave's loads and stores retire in issue order, so a store waited for in
// the middle of the stream would hold up every load issued after it; hence
// h goes out in one batch, between the gate/up and down segments.
//
// Both exchanges between workgroups (scores before routing, h before down)
// count arrivals on a 64-bit counter in a caller-owned workspace (device
// memory, zeroed once before first use) that only ever grows: each launch
// adds 2*nwg, so this launch's first exchange completes at the next multiple
// of nwg above the count found at the start, and the second nwg later.  The
// data exchanged is written with device-scope stores, which go through to
// the device-coherent level at once, and the h exchange is read with
// device-coherent loads; a workgroup only waits for its own stores to
// complete before it counts itself, so no exchange writes back a cache (with
// eight L2s, one per XCD, a release fence per workgroup would).  All
// workgroups must be resident at once: the grid is one workgroup per compute
// unit and each asks for more than half of a compute unit's LDS.  Every wait
// is bounded: past the spin limit the workgroup sets the workspace's error
// word and goes on, so a launch that cannot be co-resident (the GPU shared
// with other work) ends with garbage outputs and a raised flag instead of
// hanging.
#include "imma.h"
#include "persist.h"
#include "route.h"

namespace moedec {

namespace {

using namespace mfma;
using namespace imma;

constexpr int kFusedExperts = 512;                      // routed experts at most
using FusedRoute = RouteLdsT<kCols, kFusedExperts, kMW>;
constexpr int kRowF4 = MOEDEC_MAX_DIM / 4 / kMT;        // float4 of a router row per thread
constexpr int kSpinDefault = 1 << 21;                   // ~1 us per poll: a couple of seconds
constexpr int kPollRun = 24;                             // pipelined polls before the plain loop
constexpr int kStreamW = 3;                             // stream items in flight per wave (3 measured best)
constexpr int kStageV4 = 10;                            // float4 of h a thread stages at once
constexpr int kStageX4 = 4;                             // float4 of x a thread holds at once
constexpr int kShPref = 8;                              // K-chunks of the shared tile a prefetching wave holds
constexpr int kScaleRegs = 2;                           // row scales a thread fetches early (per kind)
constexpr size_t kDeferLds = 48 * 1024;                 // partial sums of all gate/up blocks at most
constexpr int kBufWord3 = 0x00020000;                   // raw buffer resource: 32-bit data format
constexpr int kCoherent = 16;                           // buffer load cache policy: device-coherent (sc1)

// Workspace: kGates 64-bit arrival counters 256 bytes apart (workgroup b
// counts on counter b % kGates, so arrivals on different counters do not
// queue behind each other), then the error word and the spin cap.
constexpr int kGates = 8, kGateStride = 64;
constexpr int kWsError = MOEDEC_FUSED_WS_ERROR, kWsSpin = MOEDEC_FUSED_WS_SPIN;
static_assert(kGates * kGateStride <= kWsError && kWsSpin < MOEDEC_FUSED_WORKSPACE_INTS, "workspace layout");

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
    float* x_out;                  // residual form: x_out = x + y (x is then the un-normalised stream)
    int32_t* ws;
    int E, n_group, topk_group, n_shared;
    float rsf, top_p, eps;
    int act8;                      // 1: Q8_0-style int8 activations (block scales) instead of int16
    int shp;                       // 1: the shared experts' gate/up rows are fetched during routing
    int qc;                        // assignments staged at once for down
    int rb;                        // gate/up blocks whose partial sums LDS holds at once
    int deferred;                  // 1: every block has its own slot and is finalised after the segment
    int off_gured, off_gsc, off_dsc, off_pairs, off_chunk, off_hprod;   // dynamic LDS layout (bytes)
    int off_shpart;                                                     // shp: the shared tile's partial sums
    int off_qdx;                                                        // kQ8: block scales of the staged x
};

// kQ8: column blocks of a K-chunk (the MFMA columns of one token), blocks
// per column block, whether lane group lq belongs to column block cb, and
// half hf of a lane's B operand (int2: the slots of block 2 cb + hf only).
template <int BITS>
struct Q8Cols {
    static constexpr int NCB = BITS == 8 ? 2 : 4;
    static constexpr int HALVES = BITS == 2 ? 2 : 1;
    __device__ static bool in(int lq, int cb) { return BITS == 8 ? (lq >> 1) == cb : lq == cb; }
    __device__ static i32x4 half(i32x4 v, int hf) {
        if constexpr (BITS == 2) {
            if (hf) v.x = v.y = 0;
            else v.z = v.w = 0;
        }
        return v;
    }
};

// Workgroup barrier for LDS only: loads in flight to registers stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Split-phase grid barrier (see the file comment).  settle(): the
// workgroup's stores have completed; count(): the last wave adds the
// workgroup's arrival (no wait for the add); wait(): the same wave polls the
// counters until every workgroup has arrived, and the workgroup
// resynchronises.  The data exchanged is read afterwards with device-coherent
// loads only, so no cache is invalidated.  A wave's loads complete in
// issue order, so only the counting wave's loads queue behind the add --
// the poll does anyway -- and loads issued before the count do not.  Each launch adds 2 to every counter per member
// workgroup, so a counter's launch index is its count / (2 * members), read
// by each workgroup from its own counter before its first arrival.
struct GridGate {
    int32_t* ws;
    int spin_max;
    unsigned long long launch;      // launches completed on this workspace before this one

    __device__ __forceinline__ static int members(int i) { return ((int)gridDim.x - i + kGates - 1) / kGates; }
    __device__ __forceinline__ unsigned long long* counter(int i) const {
        return reinterpret_cast<unsigned long long*>(ws + i * kGateStride);
    }
    __device__ __forceinline__ void init() {
        const int own = blockIdx.x % kGates;
        const unsigned long long found = __hip_atomic_load(counter(own), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        launch = found / (2ull * members(own));
    }
    __device__ __forceinline__ void settle() {
        __builtin_amdgcn_s_waitcnt(0);     // this wave's stores (device scope) have completed
        __syncthreads();
    }
    __device__ __forceinline__ void count() {
        if ((int)threadIdx.x == kMT - kWave)
            __hip_atomic_fetch_add(counter(blockIdx.x % kGates), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ __forceinline__ void arrive() {
        settle();
        count();
    }
    // exchange x (1 or 2) of this launch is complete
    __device__ __forceinline__ void wait(int x) {
        if ((int)threadIdx.x >= kMT - kWave) {
            const int i = (int)threadIdx.x - (kMT - kWave);
            const int m = i < kGates ? members(i) : 0;
            const unsigned long long target = (2ull * launch + (unsigned long long)x) * (unsigned long long)m;
            // Four polls in flight: each step checks the oldest and issues the
            // next, so the exchange is seen a fraction of a load's latency
            // after it completes instead of up to a whole round trip later.
            // Every lane loads (lanes past the counters re-read the last one):
            // a branch around the loads would make each wait for all of them,
            // and so would a loop back edge -- hence a straight run of steps
            // first, then a plain polling loop for long waits.
            unsigned long long* const cp = counter(i < kGates ? i : kGates - 1);
            auto poll = [&]() -> unsigned long long {
                return __hip_atomic_load(cp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            };
            unsigned long long p[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                p[k] = poll();
                if (k < 3) __builtin_amdgcn_s_sleep(1);
            }
            bool done = false;
#pragma unroll
            for (int k = 0; k < kPollRun; ++k) {
                if (__ballot(m != 0 && p[k & 3] < target) == 0) {
                    done = true;
                    break;
                }
                p[k & 3] = poll();
                __builtin_amdgcn_s_sleep(1);
            }
            int n = kPollRun;
            while (!done) {
                if (__ballot(m != 0 && poll() < target) == 0) break;
                if (++n >= spin_max) {
                    if (i == 0) __hip_atomic_store(ws + kWsError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
    }
};

// Router rows e = part, part + nparts, ... for all T tokens: every thread holds
// its float4s of the row, dots them with each token, the wave sums by DPP and
// the 8 waves' sums are added in wave order.
// Sum of squares of token t's row (kResid): every thread's float4 in k order,
// fmaf chains, then the wave and the waves in fixed order -- the same bits in
// every workgroup, whether or not it also computes router rows.
__device__ __forceinline__ float ssq_part(const float4& v, float ss) {
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    return fmaf(v.w, v.w, ss);
}

template <bool kResid>
__device__ __forceinline__ void router_rows(const FusedArgs& f, int part, int nparts, float (*red)[kMW],
                                            float (*ssq)[kMW], float* xinv) {
    const int H = f.a.H, T = f.a.T, E = f.E;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n4 = H >> 2;
    bool first = true;
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
            float acc = 0.f, ss = 0.f;
#pragma unroll
            for (int k = 0; k < kRowF4; ++k) {
                const int i = threadIdx.x + k * kMT;
                if (i < n4) {
                    const float4 v = x4[i];
                    acc = fmaf(wr[k].x, v.x, acc);
                    acc = fmaf(wr[k].y, v.y, acc);
                    acc = fmaf(wr[k].z, v.z, acc);
                    acc = fmaf(wr[k].w, v.w, acc);
                    if (kResid) ss = ssq_part(v, ss);
                }
            }
            acc = group_sum<kWave>(acc);
            if (lane == 0) red[t][wave] = acc;
            if (kResid && first) {
                ss = group_sum<kWave>(ss);
                if (lane == 0) ssq[t][wave] = ss;
            }
        }
        __syncthreads();
        if ((int)threadIdx.x < T) {
            float z = 0.f;
            for (int w = 0; w < kMW; ++w) z += red[threadIdx.x][w];
            if (kResid) {
                if (first) {
                    float q = 0.f;
                    for (int w = 0; w < kMW; ++w) q += ssq[threadIdx.x][w];
                    xinv[threadIdx.x] = 1.0f / sqrtf(q / (float)H + f.eps);
                }
                z *= xinv[threadIdx.x];                 // W . (x / rms) = (W . x) / rms
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
                const int i = threadIdx.x + k * kMT;
                if (i < n4) ss = ssq_part(x4[i], ss);
            }
            ss = group_sum<kWave>(ss);
            if (lane == 0) ssq[t][wave] = ss;
        }
        __syncthreads();
        if ((int)threadIdx.x < T) {
            float q = 0.f;
            for (int w = 0; w < kMW; ++w) q += ssq[threadIdx.x][w];
            xinv[threadIdx.x] = 1.0f / sqrtf(q / (float)H + f.eps);
        }
        __syncthreads();
    }
}

// Running maximum of non-negative floats in LDS (their bits order as unsigned).
__device__ __forceinline__ void lds_max(unsigned* slot, float v) {
    __hip_atomic_fetch_max(slot, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Maximum of |v| over the values of column t (wave-wide when the whole wave
// holds one column, else per lane) into cmax[t]; invalid lanes pass t < 0.
__device__ __forceinline__ void column_max(unsigned* cmax, int t, float m) {
    const int t0 = __builtin_amdgcn_readfirstlane(t);
    if (t0 < 0) return;                                    // lane 0 holds the smallest index
    if (__ballot(t != t0) == 0) {
        m = wave_max(m);
        if ((threadIdx.x & (kWave - 1)) == 0) lds_max(cmax + t0, m);
    } else if (t >= 0) {
        lds_max(cmax + t, m);
    }
}

// Scatter 4 consecutive columns col0.. (col0 % 4 == 0) of row k, already
// scaled by 2^e, into the int8 B layout: unit ((g*ldn + k)*NM + m) of hi /
// lo, slot s, for column g*CW + col(m, s).  Within a float4 the slots follow
// a fixed pattern per code width, so the bytes go out in whole 16- or 32-bit
// writes where they are adjacent: int4 columns (p, p+2) and (p+1, p+3) are
// slots (s, s+1) of operands 0 and 1; int8 columns are 4 consecutive slots;
// int2 columns are one slot of each of the 4 operands.
__device__ __forceinline__ uint32_t pack_bytes(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) | ((uint32_t)d << 24);
}

template <int BITS>
__device__ __forceinline__ void scatter4(float4 v, float sc, int col0, int k, int ldn, uint8_t* hi, uint8_t* lo) {
    using C = I8Codec<BITS>;
    int h0, h1, h2, h3, l0, l1, l2, l3;
    split16(v.x * sc, h0, l0);
    split16(v.y * sc, h1, l1);
    split16(v.z * sc, h2, l2);
    split16(v.w * sc, h3, l3);
    const int g = col0 / C::CW, p0 = col0 - g * C::CW;
    const int unit = (g * ldn + k) * C::NM * 16;
    if constexpr (BITS == 4) {
        const int s0 = unit + 4 * (p0 >> 3) + ((p0 >> 1) & 3);      // even: 2-byte aligned
        *reinterpret_cast<uint16_t*>(hi + s0) = (uint16_t)pack_bytes(h0, h2, 0, 0);
        *reinterpret_cast<uint16_t*>(hi + s0 + 16) = (uint16_t)pack_bytes(h1, h3, 0, 0);
        *reinterpret_cast<uint16_t*>(lo + s0) = (uint16_t)pack_bytes(l0, l2, 0, 0);
        *reinterpret_cast<uint16_t*>(lo + s0 + 16) = (uint16_t)pack_bytes(l1, l3, 0, 0);
    } else if constexpr (BITS == 8) {
        *reinterpret_cast<uint32_t*>(hi + unit + p0) = pack_bytes(h0, h1, h2, h3);
        *reinterpret_cast<uint32_t*>(lo + unit + p0) = pack_bytes(l0, l1, l2, l3);
    } else {
        const int s0 = unit + 4 * (p0 >> 4) + ((p0 >> 2) & 3);
        hi[s0] = (uint8_t)h0;
        hi[s0 + 16] = (uint8_t)h1;
        hi[s0 + 32] = (uint8_t)h2;
        hi[s0 + 48] = (uint8_t)h3;
        lo[s0] = (uint8_t)l0;
        lo[s0 + 16] = (uint8_t)l1;
        lo[s0 + 32] = (uint8_t)l2;
        lo[s0 + 48] = (uint8_t)l3;
    }
}

// Zero the B units of groups [P, 4*NCH) of n rows (the columns past the row
// end of the last K-chunk).
template <int BITS>
__device__ __forceinline__ void zero_pad(int P, int NCH, int n, int ldn, i32x4* hi, i32x4* lo) {
    constexpr int NM = I8Codec<BITS>::NM;
    const int pad = (NCH * 4 - P) * n * NM;
    for (int uu = threadIdx.x; uu < pad; uu += kMT) {
        const int m = uu % NM;
        const int k = (uu / NM) % n;
        const int g = P + uu / (NM * n);
        hi[(g * ldn + k) * NM + m] = i32x4{0, 0, 0, 0};
        lo[(g * ldn + k) * NM + m] = i32x4{0, 0, 0, 0};
    }
}

// ---- int8 activations in blocks of 32 consecutive columns (Q8_0): d =
// absmax / 127 and q = rint(v / d) in IEEE fp32 (d = 0: all zero; a NaN or
// an infinity in the block: d = NaN, q = 0).  A K-chunk of the B layout (4
// lane groups of CW columns, 512/BITS columns) holds 16/BITS blocks.  Each
// MFMA column stands for one (token, column block) pair, a column block
// being the lane groups of one block (int8: two lane groups) or one lane
// group (int4: one block; int2: two blocks, the lane's dwords 0-1 and 2-3,
// multiplied in two MFMAs, each half with the other zeroed): its B operand
// is the token's codes there and zero elsewhere, so the column's sum is the
// block's exact integer dot product, scaled by the block's d.  The columns
// of a token are added at the end of a tile.  One MFMA per code operand (and
// half) covers 8 tokens with int8 codes, 4 with int4 and int2.

// Largest |value| (and non-finite flag) over the GL lanes of this lane's group.
template <int GL>
__device__ __forceinline__ float group_absmax(float m, bool& bad) {
    float b = bad ? 1.f : 0.f;
#pragma unroll
    for (int o = GL / 2; o >= 1; o >>= 1) {
        m = fmaxf(m, __shfl_xor(m, o, kWave));
        b = fmaxf(b, __shfl_xor(b, o, kWave));
    }
    bad = b != 0.f;
    return m;
}

// The block scale of a group and the int8 codes of 4 of its values.
__device__ __forceinline__ float q8_scale(const float4& v, bool valid, int gl_log2, bool& ok) {
    float m = valid ? fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))) : 0.f;
    bool bad = valid && !(m <= 3.402823466e38f) ;
    bad = bad || (valid && (v.x != v.x || v.y != v.y || v.z != v.z || v.w != v.w));
    if (gl_log2 == 3) m = group_absmax<8>(m, bad);
    else if (gl_log2 == 4) m = group_absmax<16>(m, bad);
    else if (gl_log2 == 5) m = group_absmax<32>(m, bad);
    else m = group_absmax<64>(m, bad);
    const float d = bad ? __uint_as_float(0x7FC00000u) : m / 127.0f;
    ok = !bad && d != 0.f;
    return d;
}

__device__ __forceinline__ int q8_code(float x, float d) {
    return (int)fminf(fmaxf(rintf(x / d), -127.f), 127.f);
}

// Four codes of consecutive columns col0.. of row k into the hi bytes of the
// B layout (the placement of scatter4).
template <int BITS>
__device__ __forceinline__ void place4_q8(int h0, int h1, int h2, int h3, int col0, int k, int ldn, uint8_t* hi) {
    using C = I8Codec<BITS>;
    const int g = col0 / C::CW, p0 = col0 - g * C::CW;
    const int unit = (g * ldn + k) * C::NM * 16;
    if constexpr (BITS == 4) {
        const int s0 = unit + 4 * (p0 >> 3) + ((p0 >> 1) & 3);
        *reinterpret_cast<uint16_t*>(hi + s0) = (uint16_t)pack_bytes(h0, h2, 0, 0);
        *reinterpret_cast<uint16_t*>(hi + s0 + 16) = (uint16_t)pack_bytes(h1, h3, 0, 0);
    } else if constexpr (BITS == 8) {
        *reinterpret_cast<uint32_t*>(hi + unit + p0) = pack_bytes(h0, h1, h2, h3);
    } else {
        const int s0 = unit + 4 * (p0 >> 4) + ((p0 >> 2) & 3);
        hi[s0] = (uint8_t)h0;
        hi[s0 + 16] = (uint8_t)h1;
        hi[s0 + 32] = (uint8_t)h2;
        hi[s0 + 48] = (uint8_t)h3;
    }
}

// Quantise and place one float4 (value i4 of a row-major [rows][cols4]
// layout) whose lane group shares a block: writes the codes, and the group's
// first lane writes the block scale times 2^-kShift to qd[blk * qld + row].
template <int BITS>
__device__ __forceinline__ void stage_q8(float4 v, bool valid, int row, int c4, int ldn, uint8_t* hi, float* qd,
                                         int qld) {
    using C = I8Codec<BITS>;
    constexpr int GL = 8, GLOG = 3;                // float4 per block: 32 columns
    bool ok;
    const float d = q8_scale(v, valid, GLOG, ok);
    if (!valid) return;
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (ok) {
        q0 = q8_code(v.x, d);
        q1 = q8_code(v.y, d);
        q2 = q8_code(v.z, d);
        q3 = q8_code(v.w, d);
    }
    place4_q8<BITS>(q0, q1, q2, q3, c4 * 4, row, ldn, hi);
    if ((c4 & (GL - 1)) == 0) qd[(c4 / GL) * qld + row] = d * (1.0f / (float)(1 << C::kShift));
}

// Stage the T token rows of x (row-major [T][H]) as int8 hi/lo B operands,
// unit ((g*T + t)*NM + m) (kQ8: the codes, and the block scales in
// qdx[blk * T + t]); column t = token t has its own exponent, and
// xu[t] = 2^-(e_t + kShift) undoes it and the code factor.  cmax[0..T) must
// be zero on entry.  When all of x fits the registers (kStageX4 float4 per
// thread) it is read once, else twice (a max pass and a convert pass).
template <int BITS, bool kResid, bool kQ8, typename Hook>
__device__ __forceinline__ void stage_x(const float* __restrict__ x, int H, int T, i32x4* hi, i32x4* lo,
                                        unsigned* cmax, float* xu, const float* xinv, float* qdx,
                                        Hook&& after_loads) {
    using C = I8Codec<BITS>;
    const int H4 = H >> 2, total4 = T * H4;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const bool single = total4 <= kStageX4 * kMT;
    float4 v[kStageX4];
    if constexpr (kQ8) {
        // one pass: each lane group of a block finds its scale and writes its codes
        uint8_t* h8 = reinterpret_cast<uint8_t*>(hi);
        for (int b0 = 0; b0 < total4; b0 += kStageX4 * kMT) {
#pragma unroll
            for (int u = 0; u < kStageX4; ++u) v[u] = x4[min(b0 + (int)threadIdx.x + u * kMT, total4 - 1)];
            if (b0 == 0) {
                __builtin_amdgcn_sched_barrier(0);
                after_loads();
            }
#pragma unroll
            for (int u = 0; u < kStageX4; ++u) {
                const int i4 = b0 + (int)threadIdx.x + u * kMT;
                const bool ok = i4 < total4;
                const int t = ok ? i4 / H4 : 0;
                float4 vv = v[u];
                if (kResid && ok) {
                    const float r = xinv[t];
                    vv = make_float4(vv.x * r, vv.y * r, vv.z * r, vv.w * r);
                }
                stage_q8<BITS>(vv, ok, t, i4 - t * H4, T, h8, qdx, T);
            }
        }
        if ((int)threadIdx.x < T) xu[threadIdx.x] = 1.0f;      // the block scales carry the unscale
        const int P = H / C::CW;
        zero_pad<BITS>(P, (P + 3) / 4, T, T, hi, lo);
        return;
    }
    for (int b0 = 0; b0 < total4; b0 += kStageX4 * kMT) {
#pragma unroll
        for (int u = 0; u < kStageX4; ++u) {           // every load first, then use
            const int i4 = b0 + (int)threadIdx.x + u * kMT;
            v[u] = x4[min(i4, total4 - 1)];
        }
        if (b0 == 0) {
            __builtin_amdgcn_sched_barrier(0);
            after_loads();
        }
#pragma unroll
        for (int u = 0; u < kStageX4; ++u) {
            const int i4 = b0 + (int)threadIdx.x + u * kMT;
            const bool ok = i4 < total4;
            const float m = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
            column_max(cmax, ok ? i4 / H4 : -1, ok ? m : 0.f);
        }
    }
    __syncthreads();
    // kResid: the staged values are x / rms, whose largest magnitude is the
    // largest |x| times 1/rms (rounding is monotonic)
    if (kResid && (int)threadIdx.x < T)
        cmax[threadIdx.x] = __float_as_uint(__uint_as_float(cmax[threadIdx.x]) * xinv[threadIdx.x]);
    if (kResid) __syncthreads();
    if ((int)threadIdx.x < T) xu[threadIdx.x] = ldexpf(1.0f, -q16_exponent(__uint_as_float(cmax[threadIdx.x])) - C::kShift);
    uint8_t* h8 = reinterpret_cast<uint8_t*>(hi);
    uint8_t* l8 = reinterpret_cast<uint8_t*>(lo);
    for (int b0 = 0; b0 < total4; b0 += kStageX4 * kMT) {
        if (!single) {
#pragma unroll
            for (int u = 0; u < kStageX4; ++u) v[u] = x4[min(b0 + (int)threadIdx.x + u * kMT, total4 - 1)];
        }
#pragma unroll
        for (int u = 0; u < kStageX4; ++u) {
            const int i4 = b0 + (int)threadIdx.x + u * kMT;
            if (i4 < total4) {
                const int t = i4 / H4;
                const float sc = ldexpf(1.0f, q16_exponent(__uint_as_float(cmax[t])));
                float4 vv = v[u];
                if (kResid) {
                    const float r = xinv[t];
                    vv = make_float4(vv.x * r, vv.y * r, vv.z * r, vv.w * r);
                }
                scatter4<BITS>(vv, sc, (i4 - t * H4) * 4, t, T, h8, l8);
            }
        }
    }
    const int P = H / C::CW;
    zero_pad<BITS>(P, (P + 3) / 4, T, T, hi, lo);
}

// Stage the down B operands of one chunk: n rows of h (row k = h[qrow[k]],
// times qmul[k]) into hi/lo unit ((g*ldn + k)*NM + m), every row with its own
// exponent; dsl[k] = 2^-(e_k + kShift) undoes it.  h is read once, with
// device-coherent 16-byte loads, consecutive lanes reading consecutive 16
// bytes (all kStageV4 loads of a thread issued before any is used).
// n * I <= kStageV4 * 4 * kMT; cmax[0..n) must be zero on entry.
template <int BITS, bool kQ8>
__device__ __forceinline__ void stage_h(const float* h, int h_bytes, int I, const int* qrow, const float* qmul,
                                        int n, int ldn, i32x4* hi, i32x4* lo, unsigned* cmax, float* dsl,
                                        float* qdh) {
    using C = I8Codec<BITS>;
    const int I4 = I >> 2, total4 = n * I4;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(h), (short)0, h_bytes, kBufWord3);
    u32x4 v[kStageV4];
#pragma unroll
    for (int u = 0; u < kStageV4; ++u) {
        const int i4 = threadIdx.x + u * kMT;
        const int k = min(i4 / I4, n - 1), c4 = i4 - (i4 / I4) * I4;
        const int off = i4 < total4 ? (qrow[k] * I4 + c4) * 16 : 0;
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCoherent);
    }
    if constexpr (kQ8) {
        // blocks of the rows h * weight: qdh[blk * ldn + k] = scale * 2^-kShift
        uint8_t* h8 = reinterpret_cast<uint8_t*>(hi);
#pragma unroll
        for (int u = 0; u < kStageV4; ++u) {
            const int i4 = threadIdx.x + u * kMT;
            const bool ok = i4 < total4;
            const int k = ok ? i4 / I4 : 0;
            const float w = qmul[k];
            const float4 f4 = make_float4(__uint_as_float(v[u].x) * w, __uint_as_float(v[u].y) * w,
                                          __uint_as_float(v[u].z) * w, __uint_as_float(v[u].w) * w);
            stage_q8<BITS>(f4, ok, k, i4 - k * I4, ldn, h8, qdh, ldn);
        }
        const int P = I / C::CW;
        zero_pad<BITS>(P, (P + 3) / 4, n, ldn, hi, lo);
        return;
    }
#pragma unroll
    for (int u = 0; u < kStageV4; ++u) {
        const int i4 = threadIdx.x + u * kMT;
        const bool ok = i4 < total4;
        const int k = ok ? i4 / I4 : 0;
        const float mm = fmaxf(fmaxf(fabsf(__uint_as_float(v[u].x)), fabsf(__uint_as_float(v[u].y))),
                               fmaxf(fabsf(__uint_as_float(v[u].z)), fabsf(__uint_as_float(v[u].w))));
        column_max(cmax, ok ? k : -1, ok ? fabsf(qmul[k]) * mm : 0.f);
    }
    __syncthreads();
    if ((int)threadIdx.x < n) dsl[threadIdx.x] = ldexpf(1.0f, -q16_exponent(__uint_as_float(cmax[threadIdx.x])) - C::kShift);
    uint8_t* h8 = reinterpret_cast<uint8_t*>(hi);
    uint8_t* l8 = reinterpret_cast<uint8_t*>(lo);
#pragma unroll
    for (int u = 0; u < kStageV4; ++u) {
        const int i4 = threadIdx.x + u * kMT;
        if (i4 < total4) {
            const int k = i4 / I4;
            const float sk = qmul[k] * ldexpf(1.0f, q16_exponent(__uint_as_float(cmax[k])));
            const float4 f4 = make_float4(__uint_as_float(v[u].x), __uint_as_float(v[u].y), __uint_as_float(v[u].z),
                                          __uint_as_float(v[u].w));
            scatter4<BITS>(f4, sk, (i4 - k * I4) * 4, k, ldn, h8, l8);
        }
    }
    const int P = I / C::CW;
    zero_pad<BITS>(P, (P + 3) / 4, n, ldn, hi, lo);
}

// Phase 3 (see the file comment).  Items of a wave, all waves alike:
//   gate/up: for each active expert j, each 16-row block of this workgroup's
//            rows, each of the wave's K-chunks -> loads of gate and up;
//   down:    for each (expert, staging chunk) pair, each of the wave's
//            K-chunks -> loads of the two 16-row blocks of output rows.
// A wave's K-chunks are c = wave*nk + k, k < nk; chunks past the row end are
// computed against zero activations.  Every load is issued at a clamped
// (valid) address, so every item issues exactly two loads and the wait
// counts before each use are static.
// The shared experts (always active, known before routing) need not wait for
// it: with shp, workgroup b takes the pairs [b*SP/nwg, (b+1)*SP/nwg) of the
// SP = S*I (gate row, up row) pairs, at most 8, as one 16-row tile -- rows
// 0-7 the pairs' gate rows, rows 8-15 their up rows -- and the waves that
// neither route a token nor poll the grid counters (waves T .. kMW-2) load
// its K-chunks, kShPref each, right after staging x.  Those waves issue no
// other loads before the stream, so the loads stay in flight through the
// routing; the tile is multiplied once the routing is done.
struct SharedTile {
    uint4 pref[kShPref];
    float scale;                   // first prefetching wave, lanes 0-15: the tile's gate (0-7) / up row scale
    int pw;                        // this wave's index among the prefetching waves, or -1
};

__device__ __forceinline__ void shared_pairs(int S, int I, int& p0, int& np) {
    const long long SP = (long long)S * I;
    p0 = (int)(SP * blockIdx.x / gridDim.x);
    np = (int)(SP * (blockIdx.x + 1) / gridDim.x) - p0;
}

template <int BITS>
__device__ __forceinline__ void shared_prefetch(const FusedArgs& f, SharedTile& st) {
    const ExpertArgs& a = f.a;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int ln = lane & 15, lq = lane >> 4;
    const int T = a.T, I = a.I, H = a.H;
    st.pw = (wave >= T && wave < kMW - 1) ? wave - T : -1;
    if (st.pw < 0) return;
    int p0, np;
    shared_pairs(f.n_shared, I, p0, np);
    const int pair = p0 + min(ln & 7, max(np - 1, 0));          // spare rows repeat a real one
    const int j = pair / I, row = pair - j * I;
    const size_t rbg = (size_t)H * BITS / 8;
    const uint8_t* base = (ln < 8 ? a.w_gate : a.w_up) + ((size_t)(f.E + j) * I + row) * rbg;
    const int Pg = (int)(rbg >> 4), NCHg = (Pg + 3) >> 2;
#pragma unroll
    for (int k = 0; k < kShPref; ++k) {
        const int ch = min(st.pw * kShPref + k, NCHg - 1);
        const int grp = min(ch * 4 + lq, Pg - 1);
        st.pref[k] = ld16(base + (size_t)grp * 16);
    }
    if (st.pw == 0 && lane < 16) {
        const size_t src = (size_t)(f.E + j) * I + row;            // lane l < 16 has pair p0 + min(l & 7, np - 1)
        st.scale = lane < 8 ? a.s_gate[src] : a.s_up[src];
    }
}

// kPass (kQ8): passes of MFMA token columns compiled in (1: up to 16 / NCB
// tokens; more: up to kCols, at the cost of a larger loop body).
template <int BITS, bool kResid, bool kQ8, int kPass>
__device__ __forceinline__ void stream(const FusedArgs& f, const FusedRoute& r, unsigned char* dyn, const float* xu,
                                       const float* qdx, GridGate& gate, const SharedTile& shtile) {
    using C = I8Codec<BITS>;
    constexpr int NM = C::NM;
    constexpr int W = kStreamW;
    const ExpertArgs& a = f.a;
    const int H = a.H, I = a.I, T = a.T, K = a.top_k, slots = a.slots;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int ln = lane & 15, lq = lane >> 4;
    const int nwg = gridDim.x, b = blockIdx.x;
    const int n_act = r.n_active;
    const int A = r.seg[n_act];
    const int* eid = r.eid;
    const int* seg = r.seg;
    const int* asn = r.assign;
    // gate/up geometry: every active expert's rows as one list (entry j*I + r
    // is row r of expert j); this workgroup takes the contiguous stretch
    // [g0, g0 + NR) of it -- one or two runs of consecutive code rows, which
    // stream faster than a few rows of every expert -- cut into 16-row
    // blocks; a block may hold rows of two experts: B carries every token,
    // and each row keeps only the columns of tokens routed to its expert
    const int rbg = H * BITS / 8, Pg = rbg >> 4, NCHg = (Pg + 3) >> 2, nkg = (NCHg + kMW - 1) / kMW;
    const int n_gu = f.shp ? n_act - f.n_shared : n_act;       // experts in the gate/up stretch
    const long long NRT = (long long)n_gu * I;
    const int g0 = (int)(NRT * b / nwg);
    const int NR = (int)(NRT * (b + 1) / nwg) - g0;
    const int nbg = (NR + 15) >> 4;
    // down geometry: output rows [dr0, dr0 + rd), rd <= 32
    const int rbd = I * BITS / 8, Pd = rbd >> 4, NCHd = (Pd + 3) >> 2, nkd = (NCHd + kMW - 1) / kMW;
    const int dr0 = b * H / nwg;
    const int rd = (b + 1) * H / nwg - dr0;
    const int qc = f.qc;
    // LDS
    const i32x4* xhi = reinterpret_cast<const i32x4*>(dyn);
    const i32x4* xlo = xhi + (size_t)NCHg * 4 * T * NM;
    i32x4* hhi = reinterpret_cast<i32x4*>(dyn);                   // replaces x once gate/up is done
    i32x4* hlo = hhi + (size_t)NCHd * 4 * qc * NM;
    float* dred = reinterpret_cast<float*>(dyn);                  // replaces h at the very end
    float* gred = reinterpret_cast<float*>(dyn + f.off_gured);    // [rb][kMW][2][16][T] + counters
    // per partial-sum slot: waves arrived at its block, and blocks finalised through it
    const int rb = f.rb;
    int* slot_cnt = reinterpret_cast<int*>(gred + (size_t)rb * kMW * 2 * 16 * T);
    int* slot_done = slot_cnt + rb;
    float* gsc = reinterpret_cast<float*>(dyn + f.off_gsc);       // [NR][2]: gate, up row scales
    float* hprod = reinterpret_cast<float*>(dyn + f.off_hprod);   // [NR][T]: this workgroup's h
    float* shpart = reinterpret_cast<float*>(dyn + f.off_shpart); // shp: [prefetching wave][16][T] + 16 scales
    float* dsc = reinterpret_cast<float*>(dyn + f.off_dsc);       // [n_act][rd]
    int* pstart = reinterpret_cast<int*>(dyn + f.off_pairs);      // [n_act + 1]
    int* qrow = reinterpret_cast<int*>(dyn + f.off_chunk);        // [qc]
    float* qmul = reinterpret_cast<float*>(qrow + qc);            // [qc]
    unsigned* qmax = reinterpret_cast<unsigned*>(qmul + qc);      // [qc]
    float* dsl = reinterpret_cast<float*>(qmax + qc);             // [qc]
    int* amap = reinterpret_cast<int*>(dsl + qc);                 // [qc][16]
    int* ctab = amap + qc * kCols;                                 // [chunks + 1][3]
    // kQ8: block scales of the staged h rows, [I / 32][qc], after the chunk tables

    // Positions: the gate/up items, then each down chunk's items, every segment
    // padded to a multiple of W, so a segment starts at ring slot 0 and its
    // start (h out, chunk staging) runs between rounds, outside the unrolled
    // ring body.  Padding positions issue loads of a real item and compute
    // nothing.
    const int Ngu = nbg * nkg;
    const int Gpad = (Ngu + W - 1) / W * W;
    const int nchunk = rd > 0 ? (A + qc - 1) / qc : 0;
    float* qdh = reinterpret_cast<float*>(ctab + 3 * ((T * slots + qc - 1) / qc + 1));

    // Two cursors walk the positions in order, one W positions ahead issuing
    // loads, one computing; a cursor advances by counting (no division or
    // search per item) and reads LDS only when its expert changes.  All
    // fields are uniform over the workgroup.
    struct Cursor {
        int kind;                   // 0 gate/up, 1 down
        int pos;                    // position within the segment
        int q;                      // down chunk
        bool valid;                 // a real item (not padding)
        int j, blk, k;              // expert, gate/up block, K-chunk of the wave
        int pair, pend;             // down pair; first pair of the next expert
    };
    auto enter_chunk = [&](Cursor& c, int q) {
        c.kind = 1;
        c.pos = 0;
        c.q = q;
        c.pair = ctab[3 * q + 2];
        c.j = mw_upper_index(pstart, n_act, c.pair);
        c.pend = pstart[c.j + 1];
        c.k = 0;
        c.valid = ctab[3 * q + 1] > 0;
    };
    auto start = [&](Cursor& c) {
        c.blk = c.k = c.j = 0;
        c.pair = c.pend = c.q = 0;
        if (Gpad > 0) {
            c.kind = 0;
            c.pos = 0;
            c.valid = true;
        } else {
            enter_chunk(c, 0);
        }
    };
    auto advance = [&](Cursor& c) {
        ++c.pos;
        if (c.kind == 0) {
            c.valid = c.pos < Ngu;
            if (c.valid && ++c.k == nkg) {
                c.k = 0;
                ++c.blk;
            }
            if (c.pos == Gpad && nchunk > 0) enter_chunk(c, 0);
        } else {
            c.valid = c.pos < ctab[3 * c.q + 1];
            if (c.valid && ++c.k == nkd) {
                c.k = 0;
                if (++c.pair == c.pend) {
                    ++c.j;
                    c.pend = pstart[c.j + 1];
                }
            }
            const int padded = (ctab[3 * c.q + 1] + W - 1) / W * W;
            if (c.pos == padded && c.q + 1 < nchunk) enter_chunk(c, c.q + 1);
        }
    };
    // (past the last position a cursor stays on the last real item: loads stay valid)

    // this lane's row of the issuing cursor's gate/up block (recomputed when the block changes)
    int iblk = -1;
    size_t irow_off = 0;
    auto issue = [&](const Cursor& c, uint4* dst) {
        if (c.kind == 0) {
            if (c.blk != iblk) {
                iblk = c.blk;
                const int rho = min(iblk * 16 + ln, NR - 1);
                const int g = g0 + rho, j = g / I;
                irow_off = ((size_t)eid[j] * I + (g - j * I)) * rbg;
            }
            const int cc = min(wave * nkg + c.k, NCHg - 1);
            const int grp = min(cc * 4 + lq, Pg - 1);
            const size_t off = irow_off + grp * 16;
            dst[0] = ld16(a.w_gate + off);
            dst[1] = ld16(a.w_up + off);
        } else {
            const int cc = min(wave * nkd + c.k, NCHd - 1);
            const int grp = min(cc * 4 + lq, Pd - 1);
            const uint8_t* base = a.w_down + ((size_t)eid[c.j] * H + dr0) * rbd + grp * 16;
            dst[0] = ld16(base + (size_t)min(ln, rd - 1) * rbd);
            dst[1] = ld16(base + (size_t)min(16 + ln, rd - 1) * rbd);
        }
    };

    const i32x4 zero4 = {0, 0, 0, 0};
    const floatx4 zerof4 = {0.f, 0.f, 0.f, 0.f};
    i32x4 gh = zero4, gl = zero4, uh = zero4, ul = zero4;     // gate / up, hi / lo parts
    i32x4 ah[kNBD], al[kNBD];
    // kQ8: block-scaled sums per pass of TPP tokens (MFMA column ln = token
    // p * TPP + ln / NCB of pass p, column block ln % NCB of the K-chunk)
    using QC = Q8Cols<BITS>;
    constexpr int NCB = kQ8 ? QC::NCB : 1;                    // column blocks of a K-chunk
    constexpr int NHF = QC::HALVES;                           // blocks of a column block
    constexpr int NBC = NCB * NHF;                            // blocks of a K-chunk
    constexpr int TPP = 16 / NCB;                             // tokens of a pass
    constexpr int NPS = kQ8 ? kPass : 1;                      // passes at most
    static_assert(!kQ8 || kPass == 1 || kPass * TPP >= kCols, "passes for every token");
    const int bc = ln % NCB, tp = ln / NCB;
    const bool bq_on = QC::in(lq, bc);                        // this lane's K slots are column block bc's
    const int npass = (T + TPP - 1) / TPP;
    // tot[p]: the layer output of pass p's tokens (kQ8: in lanes bc = 0 of
    // each token's columns; else pass 0 only, column = token)
    floatx4 gf[NPS], uf[NPS], af[NPS][kNBD], tot[NPS][kNBD];
#pragma unroll
    for (int p = 0; p < NPS; ++p) {
        gf[p] = uf[p] = zerof4;
#pragma unroll
        for (int bb = 0; bb < kNBD; ++bb) af[p][bb] = tot[p][bb] = zerof4;
    }
#pragma unroll
    for (int bb = 0; bb < kNBD; ++bb) ah[bb] = al[bb] = zero4;
    int cbqp[NPS];                  // kQ8: per pass, the staged slot of this lane's B token, or -1
    // kQ8: a pass's sums of this lane's column added over the token's NCB
    // columns (lanes tp * NCB .. + NCB - 1 of a quad: DPP); every lane gets it
    auto q8_token_sum = [&](float v) { return group_sum<NCB>(v); };
    // kQ8: leave a finished gate/up tile's sums in LDS (token t's column)
    auto q8_part_out = [&](float* part) {
#pragma unroll
        for (int p = 0; p < NPS; ++p) {
            if (p < npass) {
                const int tt = p * TPP + tp;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const float g = q8_token_sum(gf[p][ii]), u = q8_token_sum(uf[p][ii]);
                    if (bc == 0 && tt < T) {
                        part[((wave * 2 + 0) * 16 + 4 * lq + ii) * T + tt] = g;
                        part[((wave * 2 + 1) * 16 + 4 * lq + ii) * T + tt] = u;
                    }
                }
            }
            gf[p] = uf[p] = zerof4;
        }
    };
    int chunk_first = 0;            // first expert of the staged chunk
    // per-expert state of the computing cursor: this lane's staged column and its unscale
    int cj = -1, cbq = -1;
    float du = 0.f;

    // Columns of the MFMA output that no token uses hold garbage and are never
    // read, so B operands need no zeroing; chunks past the row end are skipped.
    const int tcol = min(ln, T - 1);              // this lane's token column in B
    auto gu_item = [&](const Cursor& c, const uint4* cur) {
        const int ch = wave * nkg + c.k;
        if (kQ8 && ch < NCHg) {
#pragma unroll
            for (int p = 0; p < NPS; ++p) {
                if (p < npass) {
                    const int tt = p * TPP + tp;
                    const bool on = tt < T;
                    i32x4 bx[NM];
#pragma unroll
                    for (int m = 0; m < NM; ++m) bx[m] = on && bq_on ? xhi[((ch * 4 + lq) * T + tt) * NM + m] : zero4;
#pragma unroll
                    for (int hf = 0; hf < NHF; ++hf) {
                        i32x4 g8 = zero4, u8 = zero4;
#pragma unroll
                        for (int m = 0; m < NM; ++m) {
                            const i32x4 bq = QC::half(bx[m], hf);
                            g8 = mma(operand<BITS>(cur[0], m), bq, g8);
                            u8 = mma(operand<BITS>(cur[1], m), bq, u8);
                        }
                        const int blk = ch * NBC + bc * NHF + hf;     // this column's block of the row
                        const float dq = on && blk < H / 32 ? qdx[blk * T + tt] : 0.f;   // padding groups: none
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii) {
                            gf[p][ii] = fmaf(dq, (float)g8[ii], gf[p][ii]);
                            uf[p][ii] = fmaf(dq, (float)u8[ii], uf[p][ii]);
                        }
                    }
                }
                if constexpr (BITS == 2) __builtin_amdgcn_sched_barrier(0);   // one pass's operands live at a time
            }
        } else if (!kQ8 && ch < NCHg) {
            i32x4 bh[NM], bl[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int src = ((ch * 4 + lq) * T + tcol) * NM + m;
                bh[m] = xhi[src];
                bl[m] = xlo[src];
            }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const i32x4 ag = operand<BITS>(cur[0], m);
                gh = mma(ag, bh[m], gh);
                gl = mma(ag, bl[m], gl);
                const i32x4 au = operand<BITS>(cur[1], m);
                uh = mma(au, bh[m], uh);
                ul = mma(au, bl[m], ul);
            }
        }
        if (c.k == nkg - 1 && f.deferred) {
            // every block has a slot of its own: leave the partial sums there;
            // all blocks are finalised together after the gate/up segment
            float* part = gred + (size_t)c.blk * kMW * 2 * 16 * T;
            if constexpr (kQ8) {
                q8_part_out(part);
            } else if (ln < T) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    part[((wave * 2 + 0) * 16 + 4 * lq + ii) * T + ln] = combine(gh[ii], gl[ii]);
                    part[((wave * 2 + 1) * 16 + 4 * lq + ii) * T + ln] = combine(uh[ii], ul[ii]);
                }
            }
            gh = gl = uh = ul = zero4;
        } else if (c.k == nkg - 1) {
            // This wave's part of the block is done.  No workgroup barrier here
            // (every one would wait for the slowest wave's loads): the wave leaves
            // its partial sums in the block's LDS slot and counts itself; the
            // last of the 8 waves to arrive adds them up, in wave order, and
            // writes h = silu(g) * v for the block.  A slot is reused rb blocks
            // later, once its block is finalised.
            const int bidx = c.blk;
            const int slot = bidx % rb;
            float* part = gred + (size_t)slot * kMW * 2 * 16 * T;
            if (bidx >= rb) {
                int n = 0;
                while (__hip_atomic_load(slot_done + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) <
                       bidx - rb + 1) {
                    if (++n > (1 << 24)) {
                        __hip_atomic_store(f.ws + kWsError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if constexpr (kQ8) {
                q8_part_out(part);
            } else if (ln < T) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    part[((wave * 2 + 0) * 16 + 4 * lq + ii) * T + ln] = combine(gh[ii], gl[ii]);
                    part[((wave * 2 + 1) * 16 + 4 * lq + ii) * T + ln] = combine(uh[ii], ul[ii]);
                }
            }
            gh = gl = uh = ul = zero4;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            int arrived = 0;
            if (lane == 0)
                arrived = __hip_atomic_fetch_add(slot_cnt + slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            arrived = __shfl(arrived, 0, kWave);
            if (arrived == kMW - 1) {   // the last wave: finalise the block
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                const int rows_blk = min(16, NR - bidx * 16);
                for (int idx = lane; idx < rows_blk * T; idx += kWave) {
                    const int rr = idx / T, t = idx - rr * T;
                    const int rho = bidx * 16 + rr;
                    const int j = (g0 + rho) / I;
                    const int s0 = seg[j], nc = seg[j + 1] - s0;
                    int n = 0;
                    while (n < nc && asn[s0 + n] / slots != t) ++n;     // token t's column of expert j
                    if (n < nc) {
                        float gs = 0.f, vs = 0.f;
                        for (int w = 0; w < kMW; ++w) {
                            gs += part[((w * 2 + 0) * 16 + rr) * T + t];
                            vs += part[((w * 2 + 1) * 16 + rr) * T + t];
                        }
                        const float gv = gs * xu[t] * gsc[rho * 2 + 0];
                        const float uv = vs * xu[t] * gsc[rho * 2 + 1];
                        hprod[rho * T + n] = gv / (1.0f + __expf(-gv)) * uv;
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                if (lane == 0) {
                    __hip_atomic_store(slot_cnt + slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_store(slot_done + slot, bidx + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
        }
    };

    auto dn_item = [&](const Cursor& c, const uint4* cur) {
        if (c.j != cj) {
            cj = c.j;
            cbq = amap[(cj - chunk_first) * kCols + ln];      // staged slot of this lane's token, or -1
            du = cbq >= 0 ? dsl[cbq] : 0.f;
            if constexpr (kQ8) {
#pragma unroll
                for (int p = 0; p < NPS; ++p)                 // (tokens < kCols: the map holds -1 past T)
                    cbqp[p] = amap[(cj - chunk_first) * kCols + min(p * TPP + tp, kCols - 1)];
            }
        }
        const int ch = wave * nkd + c.k;
        if (kQ8 && ch < NCHd) {
#pragma unroll
            for (int p = 0; p < NPS; ++p) {
                if (p < npass) {
                    const int slot = cbqp[p];
                    i32x4 bx[NM];
#pragma unroll
                    for (int m = 0; m < NM; ++m)
                        bx[m] = slot >= 0 && bq_on ? hhi[((ch * 4 + lq) * qc + slot) * NM + m] : zero4;
#pragma unroll
                    for (int hf = 0; hf < NHF; ++hf) {
                        const int blk = ch * NBC + bc * NHF + hf;
                        const float dq = slot >= 0 && blk < I / 32 ? qdh[blk * qc + slot] : 0.f;
#pragma unroll
                        for (int bb = 0; bb < kNBD; ++bb) {
                            i32x4 a8 = zero4;
#pragma unroll
                            for (int m = 0; m < NM; ++m) a8 = mma(operand<BITS>(cur[bb], m), QC::half(bx[m], hf), a8);
#pragma unroll
                            for (int i2 = 0; i2 < 4; ++i2) af[p][bb][i2] = fmaf(dq, (float)a8[i2], af[p][bb][i2]);
                        }
                    }
                }
                if constexpr (BITS == 2) __builtin_amdgcn_sched_barrier(0);   // one pass's operands live at a time
            }
        } else if (!kQ8 && ch < NCHd) {
            const int slot = max(cbq, 0);
            i32x4 bh[NM], bl[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int src = ((ch * 4 + lq) * qc + slot) * NM + m;
                bh[m] = hhi[src];
                bl[m] = hlo[src];
            }
#pragma unroll
            for (int bb = 0; bb < kNBD; ++bb) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const i32x4 av = operand<BITS>(cur[bb], m);
                    ah[bb] = mma(av, bh[m], ah[bb]);
                    al[bb] = mma(av, bl[m], al[bb]);
                }
            }
        }
        if (c.k == nkd - 1) {         // this pair is complete: scale rows, add (tokens routed here only)
            if constexpr (kQ8) {
                // token p * TPP + tp: its sum over its columns, added where it is routed here
#pragma unroll
                for (int p = 0; p < NPS; ++p) {
                    if (p < npass) {
#pragma unroll
                        for (int bb = 0; bb < kNBD; ++bb) {
#pragma unroll
                            for (int i2 = 0; i2 < 4; ++i2) {
                                const float v = q8_token_sum(af[p][bb][i2]);
                                const int rr = min(bb * 16 + 4 * lq + i2, rd - 1);
                                if (cbqp[p] >= 0) tot[p][bb][i2] += dsc[cj * rd + rr] * v;
                            }
                        }
                    }
#pragma unroll
                    for (int bb = 0; bb < kNBD; ++bb) af[p][bb] = zerof4;
                }
            } else if (cbq >= 0) {
#pragma unroll
                for (int bb = 0; bb < kNBD; ++bb) {
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2) {
                        const int rr = min(bb * 16 + 4 * lq + i2, rd - 1);
                        tot[0][bb][i2] += (dsc[cj * rd + rr] * du) * combine(ah[bb][i2], al[bb][i2]);
                    }
                }
            }
#pragma unroll
            for (int bb = 0; bb < kNBD; ++bb) ah[bb] = al[bb] = zero4;
        }
    };

    // segment starts, between rounds
    auto flush_h = [&]() {            // all of this workgroup's h: out at once (device scope), then counted
        for (int idx = threadIdx.x; idx < NR * T; idx += kMT) {
            const int rho = idx / T, n = idx - rho * T;
            const int g = g0 + rho, jj = g / I;
            if (n < seg[jj + 1] - seg[jj]) store_device(f.h + (size_t)asn[seg[jj] + n] * I + (g - jj * I), hprod[idx]);
        }
        gate.arrive();
    };
    // Down chunk q's tables (they depend on the routing only): rows of h to
    // stage and their weights, and each expert's column map; the caller
    // synchronises before the map is read.
    auto dn_prep = [&](int q) {
        const int q0 = q * qc, q1 = min(A, q0 + qc), nq = q1 - q0;
        const int jf = mw_upper_index(seg, n_act, q0);
        const int jl = mw_upper_index(seg, n_act, q1 - 1);
        for (int ql = threadIdx.x; ql < nq; ql += kMT) {
            const int as = asn[q0 + ql];
            const int t = as / slots, sl = as - t * slots;
            qrow[ql] = as;
            qmul[ql] = sl < K ? r.selw[t * K + sl] : 1.0f;
        }
        for (int i = threadIdx.x; i < (jl - jf + 1) * kCols; i += kMT) amap[i] = -1;
        for (int i = threadIdx.x; i < nq; i += kMT) qmax[i] = 0u;
        __syncthreads();
        for (int ql = threadIdx.x; ql < nq; ql += kMT) {
            const int jj = mw_upper_index(seg, n_act, q0 + ql);
            amap[(jj - jf) * kCols + qrow[ql] / slots] = ql;
        }
    };
    auto dn_stage = [&](int q) {
        lds_barrier();                // everyone is done with the previous chunk
        dn_prep(q);                   // chunk 0's: after this workgroup's h is out, during the exchange
        const int q0 = q * qc, nq = min(A, q0 + qc) - q0;
        if (q == 0) gate.wait(2);     // every workgroup's h is out
        // h rows are assignment indices t * slots + slot (< T * slots; A is fewer under top-p)
        stage_h<BITS, kQ8>(f.h, T * slots * I * (int)sizeof(float), I, qrow, qmul, nq, qc, hhi, hlo, qmax, dsl, qdh);
        __syncthreads();
        chunk_first = mw_upper_index(seg, n_act, q0);
        cj = -1;                      // the computing cursor reloads its expert's column map
    };

    // The stream's first loads go out before the down chunk tables are built
    // (only down items read them) when the gate/up segment holds more than a
    // ring's worth of items, so the filling cursor stays inside it.
    Cursor ci, cc_;
    uint4 ring[W][2];
    auto fill = [&]() {
        start(ci);
        start(cc_);
#pragma unroll
        for (int w = 0; w < W; ++w) {
            issue(ci, ring[w]);
            advance(ci);
        }
    };
    const bool early = Gpad > W;
    // Nothing issued earlier is still in flight (routing consumed its
    // loads); saying so here keeps later register reuse from waiting for
    // the ring's loads.
    __builtin_amdgcn_s_waitcnt(0);

    // shp: multiply the prefetched shared tile (its loads are complete: the
    // wait above; only the waves that loaded it work here, the others go on
    // to issue the ring at once); partial sums to LDS
    const int npw = kMW - 1 - T;                                   // prefetching waves
    float* ssc = shpart + (size_t)kMW * 16 * T;                    // the tile's 8 gate and 8 up row scales
    int sh_p0 = 0, sh_np = 0;
    if (f.shp) {
        shared_pairs(f.n_shared, I, sh_p0, sh_np);
        if (shtile.pw >= 0) {
            i32x4 sh = zero4, sl = zero4;
#pragma unroll
            for (int k = 0; k < kShPref; ++k) {
                const int ch = shtile.pw * kShPref + k;
                if (ch < NCHg) {
                    i32x4 bh[NM], bl[NM];
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        const int src = ((ch * 4 + lq) * T + tcol) * NM + m;
                        bh[m] = xhi[src];
                        bl[m] = xlo[src];
                    }
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        const i32x4 av = operand<BITS>(shtile.pref[k], m);
                        sh = mma(av, bh[m], sh);
                        sl = mma(av, bl[m], sl);
                    }
                }
            }
            if (ln < T) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    shpart[(shtile.pw * 16 + 4 * lq + ii) * T + ln] = combine(sh[ii], sl[ii]);
            }
            if (shtile.pw == 0 && lane < 16) ssc[lane] = shtile.scale;
        }
    }
    if (early) fill();
    // The row scales of this workgroup's gate/up rows and down rows, into
    // registers now (their loads queue right behind the ring's), to LDS just
    // before the stream starts: kScaleRegs per thread, the rest loaded there.
    float gs_r[kScaleRegs], us_r[kScaleRegs], ds_r[kScaleRegs];
    const int n_dsc = n_act * rd;
    if (NR > 0) {
#pragma unroll
        for (int u = 0; u < kScaleRegs; ++u) {
            const int i = min((int)threadIdx.x + u * kMT, NR - 1);
            const int g = g0 + i, j = g / I;
            const size_t src = (size_t)eid[j] * I + (g - j * I);
            gs_r[u] = a.s_gate[src];
            us_r[u] = a.s_up[src];
        }
    }
    if (n_dsc > 0) {
#pragma unroll
        for (int u = 0; u < kScaleRegs; ++u) {
            const int i = min((int)threadIdx.x + u * kMT, n_dsc - 1);
            const int j = i / rd, rr = i - j * rd;
            ds_r[u] = a.s_down[(size_t)eid[j] * H + dr0 + rr];
        }
    }

    // (expert, chunk) pairs: expert j spans chunks seg[j]/qc .. (seg[j+1]-1)/qc.
    // The pair starts and the chunk table are built by the last wave alone
    // (it polls the grid counters and has no other work here), so the only
    // barrier before the stream is the one that publishes them.
    if (wave == kMW - 1) {
        int carry = 0;
        for (int j0 = 0; j0 <= n_act; j0 += kWave) {       // pstart[0 .. n_act], exclusive
            const int j = j0 + lane;
            const int cnt = j < n_act ? (seg[j + 1] - 1) / qc - seg[j] / qc + 1 : 0;
            int inc = cnt;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int u = __shfl_up(inc, off, kWave);
                if (lane >= off) inc += u;
            }
            if (j <= n_act) pstart[j] = carry + inc - cnt;
            carry += __shfl(inc, kWave - 1, kWave);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane == 0) {
            int run = 0;
            for (int q = 0; q < nchunk; ++q) {
                const int jf = mw_upper_index(seg, n_act, q * qc);
                const int jl = mw_upper_index(seg, n_act, min(A, (q + 1) * qc) - 1);
                const int p0 = pstart[jf] + (q - seg[jf] / qc), p1 = pstart[jl] + (q - seg[jl] / qc);
                ctab[3 * q] = run;                        // first position (after Gpad)
                ctab[3 * q + 1] = (p1 - p0 + 1) * nkd;    // items
                ctab[3 * q + 2] = p0;                     // first pair
                run += (ctab[3 * q + 1] + W - 1) / W * W;
            }
            ctab[3 * nchunk] = run;
        }
    }
    __syncthreads();
    // shp: h of the shared pairs, straight to global memory with device-scope
    // stores, which complete before this workgroup's h-exchange arrival
    auto shared_finalize = [&]() {
        if (!f.shp) return;
        for (int idx = threadIdx.x; idx < sh_np * T; idx += kMT) {
            const int i = idx / T, t = idx - i * T;
            float gs = 0.f, vs = 0.f;
            for (int w = 0; w < npw; ++w) {
                gs += shpart[(w * 16 + i) * T + t];
                vs += shpart[(w * 16 + 8 + i) * T + t];
            }
            const float gv = gs * xu[t] * ssc[i];
            const float uv = vs * xu[t] * ssc[8 + i];
            const int pair = sh_p0 + i, j = pair / I, row = pair - j * I;
            store_device(f.h + (size_t)(t * slots + K + j) * I + row, gv / (1.0f + __expf(-gv)) * uv);
        }
    };
    // The row scales to LDS, from the registers (and past kScaleRegs per
    // thread, loaded here): gate/up ones before the stream when the blocks
    // are finalised in it, else, and the down ones always, after it.
    auto scales_to_lds = [&](bool gu, bool dn) {
#pragma unroll
        for (int u = 0; u < kScaleRegs; ++u) {
            const int i = (int)threadIdx.x + u * kMT;
            if (gu && i < NR) {
                gsc[i * 2 + 0] = gs_r[u];
                gsc[i * 2 + 1] = us_r[u];
            }
            if (dn && i < n_dsc) dsc[i] = ds_r[u];
        }
        for (int i = threadIdx.x + kScaleRegs * kMT; gu && i < NR; i += kMT) {
            const int g = g0 + i, j = g / I;
            const size_t src = (size_t)eid[j] * I + (g - j * I);
            gsc[i * 2 + 0] = a.s_gate[src];
            gsc[i * 2 + 1] = a.s_up[src];
        }
        for (int i = threadIdx.x + kScaleRegs * kMT; dn && i < n_dsc; i += kMT) {
            const int j = i / rd, rr = i - j * rd;
            dsc[i] = a.s_down[(size_t)eid[j] * H + dr0 + rr];
        }
    };
    const int Np = Gpad + (nchunk > 0 ? ctab[3 * nchunk] : 0);
    if (Ngu == 0) {                   // no gate/up rows here: the shared pairs' h, then counted as done
        shared_finalize();
        gate.arrive();
    }
    if (Np == 0) return;
    if (!early) fill();
    if (!f.deferred) {                // blocks finalised in the stream need their counters and scales now
        for (int i = threadIdx.x; i < 2 * rb; i += kMT) slot_cnt[i] = 0;
        scales_to_lds(true, false);
        __syncthreads();
    }
    // gate/up segment, then the down chunks: two loops, so each hot loop holds
    // one kind of item (the ring and both cursors carry over, Gpad % W == 0)
    for (int base = 0; base < Gpad; base += W) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const uint4 cur[2] = {ring[w][0], ring[w][1]};
            issue(ci, ring[w]);
            advance(ci);
            if (cc_.valid) gu_item(cc_, cur);
            advance(cc_);
        }
    }
    scales_to_lds(f.deferred != 0, true);
    __syncthreads();                  // every block's partial sums are in (and, ring slots: finalised)
    if (f.deferred) {                 // h = silu(g) * v of every row and routed token, in parallel
        for (int idx = threadIdx.x; idx < NR * T; idx += kMT) {
            const int rho = idx / T, t = idx - rho * T;
            const int j = (g0 + rho) / I;
            const int s0 = seg[j], nc = seg[j + 1] - s0;
            int n = 0;
            while (n < nc && asn[s0 + n] / slots != t) ++n;     // token t's column of expert j
            if (n < nc) {
                const float* part = gred + (size_t)(rho >> 4) * kMW * 2 * 16 * T;
                const int rr = rho & 15;
                float gs = 0.f, vs = 0.f;
                for (int w = 0; w < kMW; ++w) {
                    gs += part[((w * 2 + 0) * 16 + rr) * T + t];
                    vs += part[((w * 2 + 1) * 16 + rr) * T + t];
                }
                const float gv = gs * xu[t] * gsc[rho * 2 + 0];
                const float uv = vs * xu[t] * gsc[rho * 2 + 1];
                hprod[rho * T + n] = gv / (1.0f + __expf(-gv)) * uv;
            }
        }
        __syncthreads();
    }
    if (Ngu > 0) {
        shared_finalize();
        flush_h();
    }
    cj = -1;
    int next_chunk = 0;
    for (int base = Gpad; base < Np; base += W) {
        if (next_chunk < nchunk && base == Gpad + ctab[3 * next_chunk]) dn_stage(next_chunk++);
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const uint4 cur[2] = {ring[w][0], ring[w][1]};
            issue(ci, ring[w]);
            advance(ci);
            if (cc_.valid) dn_item(cc_, cur);
            advance(cc_);
        }
    }

    // the waves' partial sums -> LDS -> y, summed in wave order
    if (nchunk == 0) return;
    lds_barrier();
    if constexpr (kQ8) {
#pragma unroll
        for (int p = 0; p < NPS; ++p) {
            const int tt = p * TPP + tp;
            if (p < npass && bc == 0 && tt < T) {
#pragma unroll
                for (int bb = 0; bb < kNBD; ++bb)
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2)
                        dred[((wave * kNBD + bb) * 16 + 4 * lq + i2) * 16 + tt] = tot[p][bb][i2];
            }
        }
    } else if (ln < T) {
#pragma unroll
        for (int bb = 0; bb < kNBD; ++bb)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) dred[((wave * kNBD + bb) * 16 + 4 * lq + i2) * 16 + ln] = tot[0][bb][i2];
    }
    lds_barrier();
    for (int idx = threadIdx.x; idx < rd * T; idx += kMT) {
        const int t = idx / rd, rr = idx - t * rd;
        const int bb = rr >> 4, r16 = rr & 15;
        float s = 0.f;
        for (int w = 0; w < kMW; ++w) s += dred[((w * kNBD + bb) * 16 + r16) * 16 + t];
        const size_t o = (size_t)t * H + dr0 + rr;
        f.y[o] = s;
        if (kResid) f.x_out[o] = f.x[o] + s;            // every workgroup read x before the h exchange
    }
}

template <int BITS, bool kTopP, bool kResid, bool kQ8, int kPass>
__global__ __launch_bounds__(kMT) void layer_fused_kernel(const FusedArgs f) {
    constexpr int NM = I8Codec<BITS>::NM;
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ FusedRoute r;
    __shared__ float gemv_red[kCols][kMW];
    __shared__ float gemv_ssq[kResid ? kCols : 1][kMW];
    __shared__ unsigned xmax[kCols];
    __shared__ float xu[kCols];
    __shared__ float xinv[kCols];                     // kResid: 1 / rms of each token's x

    const ExpertArgs& a = f.a;
    const int T = a.T, H = a.H, K = a.top_k, S = f.n_shared, E = f.E;
    const int NCHg = ((H * BITS / 8) / 16 + 3) / 4;
    i32x4* xhi = reinterpret_cast<i32x4*>(dyn);
    i32x4* xlo = xhi + (size_t)NCHg * 4 * T * NM;
    float* qdx = reinterpret_cast<float*>(dyn + f.off_qdx);   // kQ8: block scales of the staged x, [H / 32][T]
    if (threadIdx.x < kCols) xmax[threadIdx.x] = 0u;
    GridGate gate{f.ws, f.ws[kWsSpin] > 0 ? f.ws[kWsSpin] : kSpinDefault, 0ull};
    gate.init();

    // ---- phase 1
    router_rows<kResid>(f, blockIdx.x, gridDim.x, gemv_red, gemv_ssq, xinv);
    gate.settle();
    stage_x<BITS, kResid, kQ8>(f.x, H, T, xhi, xlo, xmax, xu, xinv, qdx, [&] { gate.count(); });   // loads, then count
    SharedTile shtile;
    shtile.pw = -1;
    if (!kQ8 && f.shp) shared_prefetch<BITS>(f, shtile);   // in flight through the routing
    gate.wait(1);

    // ---- phase 2: routing (every workgroup, identically)
    route_select_block<kCols, kFusedExperts, kMW, true, kTopP>(f.scores, f.bias, T, E, f.n_group, f.topk_group, K, S,
                                                             f.rsf, f.top_p, r);

    // ---- phase 3: the stream
    stream<BITS, kResid, kQ8, kPass>(f, r, dyn, xu, qdx, gate, shtile);

    // Workgroup 0 writes the routing outputs last, from LDS: stores issued
    // earlier would make the compiler wait for the stream's first loads
    // wherever it reuses their registers.
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
        for (int i = threadIdx.x; i < r.n_assign; i += kMT) f.wl_assign[i] = r.assign[i];
    }
}

size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

// Dynamic LDS of a launch: [staging: x, then each down chunk's h, then the
// final reduction][gate/up reduction][gate/up scales][down scales][pair
// starts][chunk tables]; the chunk size qc is the largest that fits.
template <int BITS>
hipError_t layer_fused_bits(FusedArgs f, const FusedLayerArgs& l, hipStream_t st) {
    // only the int8-activation form is launched here (the other calls run the
    // pipelined kernel); it has no residual form
    const bool topp = f.top_p < 1.f, resid = f.x_out != nullptr, q8 = f.act8 != 0;
    if (!q8 || resid) return hipErrorInvalidValue;
    // one pass of token columns where the batch fits it, else all passes
    constexpr int kNCB = Q8Cols<BITS>::NCB, kFull = (kCols * kNCB + 15) / 16;
    const bool one = l.T * kNCB <= 16;
    auto k = one ? (topp ? layer_fused_kernel<BITS, true, false, true, 1> : layer_fused_kernel<BITS, false, false, true, 1>)
                 : (topp ? layer_fused_kernel<BITS, true, false, true, kFull>
                         : layer_fused_kernel<BITS, false, false, true, kFull>);
    static size_t static_cache[2][2] = {{0, 0}, {0, 0}};            // each variant's static LDS, read once
    size_t& static_lds = static_cache[one][topp];
    if (static_lds == 0) {
        hipFuncAttributes attr;
        hipError_t err = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(k));
        if (err != hipSuccess) return err;
        static_lds = (attr.sharedSizeBytes + 1023) & ~(size_t)1023;
    }
    const int nwg = cu_count();
    const int H = l.ex.H, I = l.ex.I, T = l.T;
    const int rd = (H + nwg - 1) / nwg;
    if (rd > kNBD * 16) return hipErrorInvalidValue;             // more output rows than a pass holds
    if (q8 && (H % 32 || I % 32)) return hipErrorInvalidValue;   // whole activation blocks
    const int A = T * l.ex.slots;
    const int max_active = l.ex.max_active;
    if (static_lds + kLdsOnePerCu > kLdsMax) return hipErrorInvalidValue;
    const size_t avail = kLdsMax - static_lds;
    const size_t x_bytes = align16(staged_row_bytes_i8<BITS>(H) * T);
    const size_t dred_bytes = (size_t)kMW * kNBD * 256 * sizeof(float);
    const int nr_max = (int)(((long long)max_active * I + nwg - 1) / nwg);   // gate/up rows of a workgroup
    const int n_blocks = (nr_max + 15) / 16;
    // partial-sum slots: one per block when they fit kDeferLds (finalised
    // after the segment), else a ring of 8 reused in order
    const size_t slot_bytes = (size_t)kMW * 2 * 16 * T * sizeof(float);
    const bool deferred = n_blocks >= 1 && (size_t)n_blocks * slot_bytes <= kDeferLds;
    const int rb = deferred ? n_blocks : (n_blocks < 8 ? (n_blocks < 1 ? 1 : n_blocks) : 8);
    const size_t gured = align16((size_t)rb * kMW * 2 * 16 * T * sizeof(float) + 2 * rb * sizeof(int));
    const size_t gsc = align16((size_t)nr_max * 2 * sizeof(float));
    const size_t dsc = align16((size_t)max_active * rd * sizeof(float));
    const size_t pairs = align16((size_t)(max_active + 1) * sizeof(int));
    const size_t hprod = align16((size_t)nr_max * T * sizeof(float));
    // the shared tile during routing: free waves to load it, whole pairs per workgroup
    const int NCHg = ((H * BITS / 8) / 16 + 3) / 4;
    const bool shp = !q8 && l.n_shared >= 1 && T <= kMW - 2 && (long long)l.n_shared * I <= 8LL * nwg &&
                     (kMW - 1 - T) * kShPref >= NCHg;
    const size_t shpart = shp ? align16(((size_t)kMW * 16 * T + 16) * sizeof(float)) : 0;
    const size_t qdx = q8 ? align16((size_t)(H / 32) * T * sizeof(float)) : 0;   // block scales of the staged x
    const size_t fixed = gured + gsc + dsc + pairs + hprod + shpart + qdx;
    auto staging = [&](int q) {
        size_t s = align16(staged_row_bytes_i8<BITS>(I) * q);
        if (s < x_bytes) s = x_bytes;
        if (s < dred_bytes) s = dred_bytes;
        return s;
    };
    auto total = [&](int q) {
        const size_t chunks = (size_t)(A + q - 1) / q;
        const size_t q8_scales = q8 ? (size_t)q * (I / 32) : 0;   // the staged h rows' block scales
        const size_t all_chunks = (size_t)(T * l.ex.slots + q - 1) / q;
        return staging(q) + fixed +
               align16(((size_t)q * (4 + kCols) + 3 * ((q8 ? all_chunks : chunks) + 1) + q8_scales) * sizeof(int));
    };
    int qc = A;
    if ((size_t)qc * I > (size_t)kStageV4 * 4 * kMT) qc = kStageV4 * 4 * kMT / I;   // a chunk's h fits registers
    while (qc > 0 && total(qc) > avail) --qc;
    if (qc < 1) return hipErrorInvalidValue;
    const size_t stg = staging(qc);
    f.qc = qc;
    f.rb = rb;
    f.deferred = deferred ? 1 : 0;
    f.off_gured = (int)stg;
    f.off_gsc = (int)(stg + gured);
    f.off_dsc = (int)(stg + gured + gsc);
    f.off_pairs = (int)(stg + gured + gsc + dsc);
    f.off_hprod = (int)(stg + gured + gsc + dsc + pairs);
    f.off_shpart = (int)(stg + gured + gsc + dsc + pairs + hprod);
    f.off_qdx = (int)(stg + gured + gsc + dsc + pairs + hprod + shpart);
    f.shp = shp ? 1 : 0;
    f.off_chunk = (int)(stg + fixed);
    size_t lds = total(qc);
    if (lds < kLdsOnePerCu) lds = kLdsOnePerCu;
    hipError_t err = allow_lds(k, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(nwg), dim3(kMT), lds, st, f);
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
    f.top_p = l.top_p;
    f.x_out = l.x_out;
    f.eps = l.eps;
    f.act8 = l.act8;
    switch (bits) {
        case 4: return layer_fused_bits<4>(f, l, st);
        case 8: return layer_fused_bits<8>(f, l, st);
        case 2: return layer_fused_bits<2>(f, l, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moedec
