// Matrix-core building blocks of the split expert kernels: code -> f16
// conversion, MFMA, activation staging, and the gate/up and down row loops of
// a persistent 8-wave workgroup (the pieces the fused layer kernel shares
// with them are in persist.h).
//
// Codes are dequantised on use (Show HN page "धीमे कंप्यूटर पर GLM 5.2
// चलाना", section "implemented features": int8, packed int4, packed int2 with
// one scale per row).  The vector ALUs only turn codes into exact f16 integers;
// the dot products run on v_mfma_f32_16x16x32_f16 with 16 weight rows as M,
// the batch's tokens as N (up to 16) and 32 input columns per call as K.
// Activations enter as an f16 hi/lo pair under one power-of-two scale (x ~= hi
// + lo to about 22 bits), so each product is two MFMAs accumulated in fp32.
//
// Code -> f16: a field q of b bits at bit s of a 32-bit word w, together with
// the field 16 bits higher, is isolated by ((w >> s) & mask), has its sign bit
// flipped (two's complement -> q + 2^(b-1)) and the exponent of 1024 ORed in
// by the same XOR, giving the half2 (1024 + 2^(b-1) + q, ...); one packed f16
// subtract of that bias leaves q exactly.  The pairs come out in the column
// order (s, s + 16/b); the staged activations use the same order.
//
// MFMA A operand: lane l supplies row l % 16 and K-values 8*(l/16) .. +7, so
// the 4 lanes of a row read 4 consecutive 16-byte groups of it (a 64-byte
// "chunk") and one wave-wide load covers 16 rows x 64 bytes.  The waves of a
// workgroup split the K dimension into chunks; their partial sums meet in LDS
// in a fixed order, so results are deterministic.
#pragma once

#include "persist.h"

namespace moedec {
namespace mfma {


// Per code width: MFMA calls per 16-byte group, mask / magic / bias of the
// conversion, and the column (within the group) of element e of call c.
template <int BITS>
struct MfmaCodec;

template <>
struct MfmaCodec<4> {
    static constexpr int NCALL = 4;
    static constexpr int NB = 3;          // 16-row blocks per gate/up group (5 ran 3-4 % slower)
    static constexpr int NBE = 5;         // ... per expert-major down group (3 ran 5 % slower)
    static constexpr uint32_t kMask = 0x000F000Fu, kMagic = 0x64086408u, kBias = 0x64086408u;   // 1032
    __device__ static int col(int c, int e) { return 8 * c + (e >> 1) + 4 * (e & 1); }
    __device__ static void place(int p, int& c, int& e) {      // col(c, e) == p
        c = p >> 3;
        e = 2 * (p & 3) + ((p >> 2) & 1);
    }
};
template <>
struct MfmaCodec<8> {
    static constexpr int NCALL = 2;
    static constexpr int NB = 5;
    static constexpr int NBE = 5;
    static constexpr uint32_t kMask = 0x00FF00FFu, kMagic = 0x64806480u, kBias = 0x64806480u;   // 1152
    __device__ static int col(int c, int e) { return 8 * c + 4 * (e >> 2) + ((e >> 1) & 1) + 2 * (e & 1); }
    __device__ static void place(int p, int& c, int& e) {      // col(c, e) == p
        c = p >> 3;
        e = 4 * ((p >> 2) & 1) + 2 * (p & 1) + ((p >> 1) & 1);
    }
};
template <>
struct MfmaCodec<2> {
    static constexpr int NCALL = 8;
    static constexpr int NB = 3;          // wider B operands: fewer blocks fit in registers
    static constexpr int NBE = 3;
    static constexpr uint32_t kMask = 0x00030003u, kMagic = 0x64026402u, kBias = 0x64026402u;   // 1026
    // call c = 2*dword + half; element e = 2*s + t is field 4*half + s + 8*t of the dword
    __device__ static int col(int c, int e) { return 16 * (c >> 1) + 4 * (c & 1) + (e >> 1) + 8 * (e & 1); }
    __device__ static void place(int p, int& c, int& e) {      // col(c, e) == p
        c = 2 * (p >> 4) + ((p >> 2) & 1);
        e = 2 * (p & 3) + ((p >> 3) & 1);
    }
};

__device__ __forceinline__ uint32_t q_pair(uint32_t w, int sh, uint32_t mask, uint32_t magic, uint32_t bias) {
    const half2v v = __builtin_bit_cast(half2v, ((w >> sh) & mask) ^ magic) - __builtin_bit_cast(half2v, bias);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t dword(const uint4& q, int d) {
    return d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
}

// A operand of call c (0 <= c < NCALL) from this lane's 16-byte group.
template <int BITS>
__device__ __forceinline__ half8 a_operand(const uint4& q, int c) {
    using M = MfmaCodec<BITS>;
    u32x4 p;
    if constexpr (BITS == 4) {
        const uint32_t w = dword(q, c);
        p = u32x4{q_pair(w, 0, M::kMask, M::kMagic, M::kBias), q_pair(w, 4, M::kMask, M::kMagic, M::kBias),
                  q_pair(w, 8, M::kMask, M::kMagic, M::kBias), q_pair(w, 12, M::kMask, M::kMagic, M::kBias)};
    } else if constexpr (BITS == 8) {
        const uint32_t w0 = dword(q, 2 * c), w1 = dword(q, 2 * c + 1);
        p = u32x4{q_pair(w0, 0, M::kMask, M::kMagic, M::kBias), q_pair(w0, 8, M::kMask, M::kMagic, M::kBias),
                  q_pair(w1, 0, M::kMask, M::kMagic, M::kBias), q_pair(w1, 8, M::kMask, M::kMagic, M::kBias)};
    } else {
        const uint32_t w = dword(q, c >> 1);
        const int s0 = 8 * (c & 1);
        p = u32x4{q_pair(w, s0 + 0, M::kMask, M::kMagic, M::kBias), q_pair(w, s0 + 2, M::kMask, M::kMagic, M::kBias),
                  q_pair(w, s0 + 4, M::kMask, M::kMagic, M::kBias), q_pair(w, s0 + 6, M::kMask, M::kMagic, M::kBias)};
    }
    return __builtin_bit_cast(half8, p);
}

__device__ __forceinline__ floatx4 mfma(const half8& a, const half8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ small helpers

__device__ __forceinline__ int mw_load_worklist(const ExpertArgs& a, int* eid, int* seg) {
    __shared__ int n_s;
    if (threadIdx.x == 0) n_s = *a.n_active;
    __syncthreads();
    const int n = n_s;
    for (int j = threadIdx.x; j <= n; j += kMT) {
        if (j < n) eid[j] = a.expert_id[j];
        seg[j] = a.seg[j];
    }
    __syncthreads();
    return n;
}

// Maximum over the workgroup.
__device__ __forceinline__ float block_max(float v, float* scratch) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    float m = scratch[0];
    for (int w = 1; w < kMW; ++w) m = fmaxf(m, scratch[w]);
    return m;
}

// Power-of-two exponent k with max|v| * 2^k in [2^14, 2^15): the activations
// then use the upper part of the f16 range without overflow.
__device__ __forceinline__ int f16_exponent(float m) {
    if (!(m > 0.f) || !isfinite(m)) return 0;
    int e;
    frexpf(m, &e);
    int k = 15 - e;
    return k > 100 ? 100 : k < -100 ? -100 : k;
}

// cpre[j] = segments (chunks of up to `cmax` tokens) of experts 0..j-1, j in [0, n].
__device__ __forceinline__ void mw_segment_prefix(const int* seg, int n, int cmax, int* cpre) {
    __shared__ int wtot[kMW];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int per = (n + 1 + kMT - 1) / kMT;
    const int j0 = threadIdx.x * per, j1 = min(j0 + per, n);
    int local = 0;
    for (int j = j0; j < j1; ++j) local += (seg[j + 1] - seg[j] + cmax - 1) / cmax;
    int inc = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += u;
    }
    if (lane == kWave - 1) wtot[wave] = inc;
    __syncthreads();
    int run = inc - local;
    for (int w = 0; w < wave; ++w) run += wtot[w];
    for (int j = j0; j < min(j0 + per, n + 1); ++j) {
        cpre[j] = run;
        if (j < n) run += (seg[j + 1] - seg[j] + cmax - 1) / cmax;
    }
    __syncthreads();
}

// x = v * s rounded to fp32, then split into f16 hi + lo (hi + lo = x to
// about 2^-22 relative).  The product is pinned in a register first: left
// free, the compiler may round it straight to f16 for one use of hi (a mixed
// fma) and through fp32 for the other, and where fp32 rounding lands on an
// f16 tie the stored pair is then one hi-ulp off.
struct F16Pair {
    _Float16 hi, lo;
};
__device__ __forceinline__ F16Pair split_f16(float v, float s) {
    float x = v * s;
    asm volatile("" : "+v"(x));
    const _Float16 hx = (_Float16)x;
    return {hx, (_Float16)(x - (float)hx)};
}

// Stage n activation rows (row k of src = src + row_off[k] * ld, times mul[k])
// into the B-operand layout: hi/lo[((ch*4 + q)*ldn + k)*NCALL + c] (half8),
// with one power-of-two scale 2^kexp for all of them; groups past the row end
// are zero.  Returns kexp.  A thread takes whole 16-byte-code groups (the CW
// activations one A-operand group multiplies): when every group fits in
// registers (IPT per thread) all loads are issued at once and each value is
// read once; otherwise a max pass and a convert pass read the rows twice.
template <int BITS>
__device__ __forceinline__ int stage_b(const float* __restrict__ src, int ld, int ncols, const int* row_off,
                                       const float* mul, int n, int ldn, half8* hi, half8* lo, float* scratch) {
    using M = MfmaCodec<BITS>;
    constexpr int CW = 16 * (8 / BITS);          // activations per code group
    constexpr int F4 = CW / 4;
    constexpr int IPT = BITS == 2 ? 1 : 2;       // groups per thread held in registers
    const int P = ncols / CW;                    // 16-byte groups of a row
    const int NCH = (P + 3) / 4;
    const int items = n * P;
    int kexp;
    if (items <= IPT * kMT) {
        float v[IPT][CW];
#pragma unroll
        for (int it = 0; it < IPT; ++it) {      // every load first, at clamped (valid) items
            const int idx = min((int)threadIdx.x + it * kMT, items - 1);
            const int k = idx / P, g = idx - k * P;
            const float4* p4 = reinterpret_cast<const float4*>(src + (size_t)row_off[k] * ld + g * CW);
#pragma unroll
            for (int q = 0; q < F4; ++q) {
                const float4 t = p4[q];
                v[it][4 * q] = t.x;
                v[it][4 * q + 1] = t.y;
                v[it][4 * q + 2] = t.z;
                v[it][4 * q + 3] = t.w;
            }
        }
        float m = 0.f;
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int idx = threadIdx.x + it * kMT;
            if (idx < items) {
                const float sm = mul ? fabsf(mul[idx / P]) : 1.f;
                float mm = 0.f;
#pragma unroll
                for (int i = 0; i < CW; ++i) mm = fmaxf(mm, fabsf(v[it][i]));
                m = fmaxf(m, sm * mm);
            }
        }
        kexp = f16_exponent(block_max(m, scratch));
        const float sc = ldexpf(1.0f, kexp);
#pragma unroll
        for (int it = 0; it < IPT; ++it) {
            const int idx = threadIdx.x + it * kMT;
            if (idx < items) {
                const int k = idx / P, g = idx - k * P;
                const float sk = (mul ? mul[k] : 1.f) * sc;
#pragma unroll
                for (int c = 0; c < M::NCALL; ++c) {
                    half8 vh, vl;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const F16Pair p = split_f16(v[it][M::col(c, e)], sk);
                        vh[e] = p.hi;
                        vl[e] = p.lo;
                    }
                    const int dst = (g * ldn + k) * M::NCALL + c;
                    hi[dst] = vh;
                    lo[dst] = vl;
                }
            }
        }
        const int pad = (NCH * 4 - P) * n * M::NCALL;   // zero groups past the row end
        for (int u = threadIdx.x; u < pad; u += kMT) {
            const int c = u % M::NCALL;
            const int k = (u / M::NCALL) % n;
            const int g = P + u / (M::NCALL * n);
            half8 z;
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = (_Float16)0.f;
            hi[(g * ldn + k) * M::NCALL + c] = z;
            lo[(g * ldn + k) * M::NCALL + c] = z;
        }
        return kexp;
    }
    float m = 0.f;
    for (int idx = threadIdx.x; idx < n * (ncols / 4); idx += kMT) {
        const int k = idx / (ncols / 4), c4 = idx - k * (ncols / 4);
        const float4 t = reinterpret_cast<const float4*>(src + (size_t)row_off[k] * ld)[c4];
        const float sm = mul ? fabsf(mul[k]) : 1.f;
        m = fmaxf(m, sm * fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))));
    }
    kexp = f16_exponent(block_max(m, scratch));
    const float sc = ldexpf(1.0f, kexp);
    const int units = NCH * 4 * n * M::NCALL;
    for (int u = threadIdx.x; u < units; u += kMT) {
        const int c = u % M::NCALL;
        const int k = (u / M::NCALL) % n;
        const int g = u / (M::NCALL * n);        // group = ch * 4 + q
        half8 vh, vl;
        if (g < P) {
            const float* row = src + (size_t)row_off[k] * ld + g * CW;
            const float sk = (mul ? mul[k] : 1.f) * sc;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const F16Pair p = split_f16(row[M::col(c, e)], sk);
                vh[e] = p.hi;
                vl[e] = p.lo;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vh[e] = vl[e] = (_Float16)0.f;
        }
        const int dst = (g * ldn + k) * M::NCALL + c;
        hi[dst] = vh;
        lo[dst] = vl;
    }
    return kexp;
}



// ------------------------------------------------------------------ gate / up
//
// Rows [rlo, rhi) of expert e's gate and up matrices against nc token columns
// (column n uses B slot colslot[n] of the staged activations and writes
// assignment asg[n]; colslot and asg in LDS).  Rows are taken in groups of up
// to NB 16-row blocks; for each group the waves walk their K-chunks (gate and
// up codes of all the group's blocks per chunk, the next chunk's loads in
// flight during the current one's MFMAs), reduce over waves in LDS and write
// h[a][r] = silu(g) * v.  Every load is issued unconditionally at a clamped
// (valid) address so the wait counts before each use are static: rows past
// the group re-read its last row (their outputs are never written) and groups
// past the row end meet zero activations.  red: LDS [kMW][NB][2][16][ns];
// sg_s / su_s: LDS [NB*16].  Returns with the workgroup synchronised.
// kDeviceStore: h is read by other workgroups of the launch (store_device).
template <int BITS, bool kDeviceStore = false>
__device__ __forceinline__ void gate_up_rows(const ExpertArgs& a, float* __restrict__ h, int e, int rlo, int rhi, int nc,
                             const int* colslot, const int* asg, const half8* xhi, const half8* xlo, int ns,
                             float unscale, float* red, float* sg_s, float* su_s) {
    using M = MfmaCodec<BITS>;
    constexpr int NCALL = M::NCALL;
    constexpr int kNB = M::NB;
    const int H = a.H, I = a.I;
    const int row_bytes = H * BITS / 8;
    const int P = row_bytes >> 4;
    const int NCH = (P + 3) / 4;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int ln = lane & 15, lq = lane >> 4;       // MFMA column (token) and K-slice of this lane
    const int cw0 = wave * NCH / kMW, cw1 = (wave + 1) * NCH / kMW;   // this wave's K-chunks
    const int nk = cw1 - cw0;
    const int bslot = ln < nc ? colslot[ln] : -1;
    const uint8_t* gb = a.w_gate + (size_t)e * I * row_bytes;
    const uint8_t* ub = a.w_up + (size_t)e * I * row_bytes;

    constexpr int G = kNB * 16;
    // chunk ch of the group starting at row gs
    auto issue_at = [&](int gs, int ch, uint4* dg, uint4* du) {
        const int grp = min(ch * 4 + lq, P - 1);
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            const int r = min(gs + b * 16 + ln, rhi - 1);
            const size_t off = (size_t)r * row_bytes + grp * 16;
            dg[b] = ld16(gb + off);
            du[b] = ld16(ub + off);
        }
    };
    // With an even chunk count per wave, chunks go in pairs t, t + 1: the two
    // 64-byte halves of each row's 128-byte line, issued back to back so the
    // second half meets the first one's fill (issued apart, under load about
    // a third of the lines were fetched twice).  Gate and up pairs alternate:
    // one matrix's pair streams while the other's is multiplied, and the next
    // group's first pairs go out ahead of this group's reduction.
    const bool ahead = nk > 0 && (nk & 1) == 0;
    uint4 g0b[kNB], u0b[kNB], g1b[kNB], u1b[kNB];
    auto issue_m = [&](int gs, int ch, uint4* d, const uint8_t* mb) {
        const int grp = min(ch * 4 + lq, P - 1);
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            const int r = min(gs + b * 16 + ln, rhi - 1);
            d[b] = ld16(mb + (size_t)r * row_bytes + grp * 16);
        }
    };
    if (ahead) {
        issue_m(rlo, cw0, g0b, gb);
        issue_m(rlo, cw0 + 1, g1b, gb);
        issue_m(rlo, cw0, u0b, ub);
        issue_m(rlo, cw0 + 1, u1b, ub);
    }
    for (int g0 = rlo; g0 < rhi; g0 += G) {
        const int gn = min(rhi - g0, G);                 // rows in this group
        const int nb = (gn + 15) >> 4;
        // row scales: loaded now, used after the K loop (to LDS only then, so
        // nothing waits for them before the code loads are issued)
        const int sr = min((int)threadIdx.x, gn - 1);
        const float sgv = a.s_gate[(size_t)e * I + g0 + sr];
        const float suv = a.s_up[(size_t)e * I + g0 + sr];
        floatx4 accg[kNB], accu[kNB];
#pragma unroll
        for (int b = 0; b < kNB; ++b) accg[b] = accu[b] = floatx4{0.f, 0.f, 0.f, 0.f};
        auto issue = [&](int ch, uint4* dg, uint4* du) { issue_at(g0, ch, dg, du); };
        auto compute = [&](int ch, const uint4* dg, const uint4* du) {
            half8 bh[NCALL], bl[NCALL];
#pragma unroll
            for (int c = 0; c < NCALL; ++c) {
                if (bslot >= 0) {
                    const int src = ((ch * 4 + lq) * ns + bslot) * NCALL + c;
                    bh[c] = xhi[src];
                    bl[c] = xlo[src];
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
                        const half8 ag = a_operand<BITS>(dg[b], c);
                        accg[b] = mfma(ag, bh[c], accg[b]);
                        accg[b] = mfma(ag, bl[c], accg[b]);
                        const half8 au = a_operand<BITS>(du[b], c);
                        accu[b] = mfma(au, bh[c], accu[b]);
                        accu[b] = mfma(au, bl[c], accu[b]);
                    }
                }
            }
        };
        if (ahead) {
            const int gnx = g0 + G < rhi ? g0 + G : g0;
            auto compute_m = [&](int ch, const uint4* d, floatx4* acc) {
                half8 bh[NCALL], bl[NCALL];
#pragma unroll
                for (int c = 0; c < NCALL; ++c) {
                    if (bslot >= 0) {
                        const int src = ((ch * 4 + lq) * ns + bslot) * NCALL + c;
                        bh[c] = xhi[src];
                        bl[c] = xlo[src];
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
                            const half8 av = a_operand<BITS>(d[b], c);
                            acc[b] = mfma(av, bh[c], acc[b]);
                            acc[b] = mfma(av, bl[c], acc[b]);
                        }
                    }
                }
            };
            for (int t = 0; t < nk; t += 2) {          // gate chunks t, t+1 in g0b, g1b; up in u0b, u1b
                compute_m(cw0 + t, g0b, accg);
                compute_m(cw0 + t + 1, g1b, accg);
                const bool in0 = t + 2 < nk, more = in0 || g0 + G < rhi;
                const int ng = in0 ? g0 : gnx, nc0 = in0 ? cw0 + t + 2 : cw0;
                if (more) {
                    issue_m(ng, nc0, g0b, gb);
                    issue_m(ng, nc0 + 1, g1b, gb);
                }
                compute_m(cw0 + t, u0b, accu);
                compute_m(cw0 + t + 1, u1b, accu);
                if (more) {
                    issue_m(ng, nc0, u0b, ub);
                    issue_m(ng, nc0 + 1, u1b, ub);
                }
            }
        } else if (nk > 0) {
            issue(cw0, g0b, u0b);
            for (int t = 0; t < nk; t += 2) {          // two register buffers, alternating
                issue(cw0 + min(t + 1, nk - 1), g1b, u1b);
                compute(cw0 + t, g0b, u0b);
                issue(cw0 + min(t + 2, nk - 1), g0b, u0b);
                if (t + 1 < nk) compute(cw0 + t + 1, g1b, u1b);
            }
        }
        if ((int)threadIdx.x < gn) {
            sg_s[threadIdx.x] = sgv;
            su_s[threadIdx.x] = suv;
        }
        // partial sums of this wave's K-chunks -> LDS; lane holds rows 4*lq + i, column ln
        if (ln < nc) {
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                if (b < nb) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * lq + i;
                        red[(((wave * kNB + b) * 2 + 0) * 16 + r) * ns + ln] = accg[b][i];
                        red[(((wave * kNB + b) * 2 + 1) * 16 + r) * ns + ln] = accu[b][i];
                    }
                }
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < gn * nc; idx += kMT) {
            const int r = idx / nc, n = idx - r * nc;
            const int b = r >> 4, rr = r & 15;
            float gs = 0.f, vs = 0.f;
            for (int w = 0; w < kMW; ++w) {
                gs += red[(((w * kNB + b) * 2 + 0) * 16 + rr) * ns + n];
                vs += red[(((w * kNB + b) * 2 + 1) * 16 + rr) * ns + n];
            }
            const int row = g0 + r;
            const float gv = gs * unscale * sg_s[r];
            const float uv = vs * unscale * su_s[r];
            const float hv = gv / (1.0f + __expf(-gv)) * uv;
            if constexpr (kDeviceStore) store_device(h + (size_t)asg[n] * I + row, hv);
            else h[(size_t)asg[n] * I + row] = hv;
        }
        __syncthreads();
    }
}

// Per-workgroup LDS of gate_up_units (besides the dynamic staging).
struct GateUpLds {
    int cpre[kMaxActive + 1];                // segments of experts 0..j-1
    int tok[kCols], asg[kCols], col[kCols], staged[kCols];
    float scratch[kMW];
    float sg[kNBMax * 16], su[kNBMax * 16];
    int kexp;
};

// Stage all T tokens of x once (B slot = token index); sets s.kexp and
// s.staged.  Used when T <= ns.
template <int BITS>
__device__ __forceinline__ void stage_tokens(const float* __restrict__ x, int T, int H, int ns, half8* xhi, half8* xlo,
                             GateUpLds& s) {
    if (threadIdx.x < kCols) s.tok[threadIdx.x] = threadIdx.x;
    __syncthreads();
    const int k = stage_b<BITS>(x, H, H, s.tok, nullptr, T, ns, xhi, xlo, s.scratch);
    if (threadIdx.x == 0) s.kexp = k;
    __syncthreads();
}

// Gate/up + SwiGLU over the experts j < n_exp of a worklist (eid ascending,
// seg offsets into assign; LDS or global).  Work units are (segment, row):
// segment = (expert j, a chunk of up to ns of its tokens), enumerated
// expert-ascending; this workgroup takes share `part` of `nparts` equal
// contiguous shares.  With stage_all the tokens were staged by stage_tokens
// and a segment's columns point at their tokens' slots; otherwise each
// segment stages its own tokens (skipped when they are already staged).
template <int BITS, bool kDeviceStore = false>
__device__ __forceinline__ void gate_up_units(const ExpertArgs& a, const float* __restrict__ x, float* __restrict__ h,
                              const int* eid, const int* seg, const int* assign, int n_exp, int ns, bool stage_all,
                              int part, int nparts, half8* xhi, half8* xlo, float* red, GateUpLds& s) {
    const int H = a.H, I = a.I;
    if (threadIdx.x < kCols && !stage_all) s.staged[threadIdx.x] = -1;
    mw_segment_prefix(seg, n_exp, ns, s.cpre);
    const int n_seg = s.cpre[n_exp];
    const long long n_units = (long long)n_seg * I;
    const long long u0 = n_units * part / nparts;
    const long long u1 = n_units * (part + 1) / nparts;
    if (u0 >= u1) return;                        // uniform over the workgroup
    for (int sidx = (int)(u0 / I); (long long)sidx * I < u1; ++sidx) {
        const int rlo = (int)max(u0 - (long long)sidx * I, 0LL);
        const int rhi = (int)min(u1 - (long long)sidx * I, (long long)I);
        const int j = mw_upper_index(s.cpre, n_exp, sidx);
        const int e = eid[j];
        const int first = seg[j] + (sidx - s.cpre[j]) * ns;
        const int nc = min(ns, seg[j + 1] - first);
        __syncthreads();   // everyone is done with the previous segment's LDS
        if ((int)threadIdx.x < nc) {
            const int as = assign[first + threadIdx.x];
            s.asg[threadIdx.x] = as;
            s.tok[threadIdx.x] = as / a.slots;
            s.col[threadIdx.x] = stage_all ? as / a.slots : (int)threadIdx.x;
        }
        __syncthreads();
        if (!stage_all) {
            bool same = true;
            for (int k = 0; k < nc; ++k) same = same && s.staged[k] == s.tok[k];
            if (!same) {
                const int k = stage_b<BITS>(x, H, H, s.tok, nullptr, nc, ns, xhi, xlo, s.scratch);
                if (threadIdx.x == 0) s.kexp = k;
                if (threadIdx.x < kCols) s.staged[threadIdx.x] = (int)threadIdx.x < nc ? s.tok[threadIdx.x] : -1;
                __syncthreads();
            }
        }
        gate_up_rows<BITS, kDeviceStore>(a, h, e, rlo, rhi, nc, s.col, s.asg, xhi, xlo, ns, ldexpf(1.0f, -s.kexp), red, s.sg,
                           s.su);
    }
}

// LDS bytes gate_up_rows needs besides the staged activations, per staged token.
template <int BITS>
constexpr size_t gate_up_red_bytes_per_token() {
    return (size_t)kMW * MfmaCodec<BITS>::NB * 2 * 16 * sizeof(float);
}

// Bytes of one staged activation row (hi + lo B operands) of `ncols` columns.
template <int BITS>
__host__ __device__ constexpr size_t staged_row_bytes(int ncols) {
    return (size_t)((ncols * BITS / 8 / 16 + 3) / 4) * 4 * MfmaCodec<BITS>::NCALL * 2 * 16;
}

// LDS per staged token of gate_up_units: hi + lo B operands and the reduction.
template <int BITS>
__host__ __device__ constexpr size_t gate_up_lds_per_token(int H) {
    return staged_row_bytes<BITS>(H) + gate_up_red_bytes_per_token<BITS>();
}

// ------------------------------------------------------------ down + combine
//
// Output rows [r0, r1) (at most kNBD blocks of 16) for the whole batch of at
// most 16 tokens (one MFMA column each), over every expert of the worklist
// (eid / seg / assign, experts ascending, in LDS or global memory).  The
// assignments are walked in chunks of up to qc; each chunk's h times its
// routing weight is staged as f16 hi/lo in LDS, and for every expert the waves
// accumulate Qd . h' over their K-chunks, scale by the expert's row scales and
// add to a running sum; at the end the waves' sums meet in LDS in a fixed order
// and y is written.  No atomics: deterministic.  `dyn` holds the chunk's
// staging (down_lds_bytes).  Returns with the workgroup synchronised.
//
// `gate` lets a caller overlap a wait for h with the first weight loads:
// gate.arrive() runs before the first chunk's weight loads are issued and
// gate.wait() after, before h is first read (both once, by the whole
// workgroup).  NoGate does nothing.
struct NoGate {
    __device__ void arrive() {}
    __device__ void wait() {}
};
constexpr int kDownW = 4;                      // items (expert, chunk) in flight per wave

template <int BITS>
__host__ __device__ constexpr size_t down_lds_bytes_per_assignment(int I) {
    return staged_row_bytes<BITS>(I) + sizeof(int) + sizeof(float) + kCols * sizeof(int) + 32 * sizeof(float);
}
__host__ __device__ constexpr size_t down_lds_fixed_bytes() { return (size_t)kMW * kNBD * 256 * sizeof(float); }

template <int BITS, typename Gate>
__device__ __forceinline__ void down_rows(const float* h, const float* topk_w, const ExpertArgs& a, float* __restrict__ y, int r0,
                          int r1, int qc, unsigned char* dyn, const int* eid, const int* seg, const int* assign,
                          int n_act, float* scratch, Gate& gate) {
    using M = MfmaCodec<BITS>;
    constexpr int NCALL = M::NCALL;
    constexpr int W = kDownW;
    const int H = a.H, I = a.I, T = a.T, K = a.top_k, slots = a.slots;
    const int row_bytes = I * BITS / 8;
    const int P = row_bytes >> 4;
    const int NCH = (P + 3) / 4;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int ln = lane & 15, lq = lane >> 4;
    const int nrows = r1 - r0;
    const int nb = (nrows + 15) >> 4;

    half8* hhi = reinterpret_cast<half8*>(dyn);                 // [NCH*4][qc][NCALL]
    half8* hlo = hhi + (size_t)NCH * 4 * qc * NCALL;
    float* red = reinterpret_cast<float*>(hlo + (size_t)NCH * 4 * qc * NCALL);   // [kMW][kNBD][16][16]
    int* qrow = reinterpret_cast<int*>(red + (size_t)kMW * kNBD * 256);          // [qc] assignment
    float* qmul = reinterpret_cast<float*>(qrow + qc);                            // [qc] routing weight
    int* amap = reinterpret_cast<int*>(qmul + qc);                                // [qc][16] expert x token -> slot
    float* sd_s = reinterpret_cast<float*>(amap + (size_t)qc * kCols);           // [qc][32] row scales

    const int A = seg[n_act];
    const int cw0 = wave * NCH / kMW, cw1 = (wave + 1) * NCH / kMW;
    const int nk = cw1 - cw0;                    // this wave's K-chunks
    floatx4 tot[kNBD];
#pragma unroll
    for (int b = 0; b < kNBD; ++b) tot[b] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint8_t* wbase = a.w_down + (size_t)r0 * row_bytes;

    for (int q0 = 0; q0 < A; q0 += qc) {
        const int q1 = min(A, q0 + qc);
        const int nq = q1 - q0;
        const int j_first = mw_upper_index(seg, n_act, q0);
        const int j_last = mw_upper_index(seg, n_act, q1 - 1);
        const int nj = j_last - j_first + 1;
        const int n_items = nj * nk;

        uint4 ring[W][kNBD];
        // every load unconditional at a clamped address (static wait counts):
        // rows past the block re-read the last row, items past the end the last item
        auto issue = [&](int i, uint4* dst) {
            i = min(i, n_items - 1);
            const int jj = j_first + i / nk, ch = cw0 + i % nk;
            const int grp = min(ch * 4 + lq, P - 1);
            const uint8_t* base = wbase + (size_t)eid[jj] * H * row_bytes + grp * 16;
#pragma unroll
            for (int b = 0; b < kNBD; ++b) dst[b] = ld16(base + (size_t)min(b * 16 + ln, nrows - 1) * row_bytes);
        };
        // weights first: these loads fly while h is staged
        if (q0 == 0) gate.arrive();
        if (n_items > 0) {
#pragma unroll
            for (int w = 0; w < W; ++w) issue(w, ring[w]);
        }
        if (q0 == 0) gate.wait();

        __syncthreads();   // the previous chunk's readers are done with LDS
        for (int ql = threadIdx.x; ql < nq; ql += kMT) {
            const int as = assign[q0 + ql];
            const int t = as / slots, slot = as - t * slots;
            qrow[ql] = as;
            qmul[ql] = slot < K ? topk_w[t * K + slot] : 1.0f;
        }
        for (int i = threadIdx.x; i < nj * kCols; i += kMT) amap[i] = -1;
        for (int i = threadIdx.x; i < nj * 32; i += kMT) {        // row scales of the chunk's experts
            const int jq = i >> 5, rl = min(i & 31, nrows - 1);
            sd_s[i] = a.s_down[(size_t)eid[j_first + jq] * H + r0 + rl];
        }
        __syncthreads();
        for (int ql = threadIdx.x; ql < nq; ql += kMT) {
            const int jj = mw_upper_index(seg, n_act, q0 + ql);
            amap[(jj - j_first) * kCols + qrow[ql] / slots] = ql;
        }
        const int kexp = stage_b<BITS>(h, I, I, qrow, qmul, nq, qc, hhi, hlo, scratch);
        __syncthreads();
        const float unscale = ldexpf(1.0f, -kexp);

        floatx4 acc[kNBD];
#pragma unroll
        for (int b = 0; b < kNBD; ++b) acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int base = 0; base < n_items; base += W) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const int i = base + w;
                uint4 cq[kNBD];
#pragma unroll
                for (int b = 0; b < kNBD; ++b) cq[b] = ring[w][b];
                issue(i + W, ring[w]);
                if (i < n_items) {
                    const int jq = i / nk, ch = cw0 + i % nk;
                    const int bq = amap[jq * kCols + ln];                 // this lane's token column
                    half8 bh[NCALL], bl[NCALL];
#pragma unroll
                    for (int c = 0; c < NCALL; ++c) {
                        if (bq >= 0) {
                            const int src = ((ch * 4 + lq) * qc + bq) * NCALL + c;
                            bh[c] = hhi[src];
                            bl[c] = hlo[src];
                        } else {
#pragma unroll
                            for (int e2 = 0; e2 < 8; ++e2) bh[c][e2] = bl[c][e2] = (_Float16)0.f;
                        }
                    }
#pragma unroll
                    for (int b = 0; b < kNBD; ++b) {
                        if (b < nb) {
#pragma unroll
                            for (int c = 0; c < NCALL; ++c) {
                                const half8 av = a_operand<BITS>(cq[b], c);
                                acc[b] = mfma(av, bh[c], acc[b]);
                                acc[b] = mfma(av, bl[c], acc[b]);
                            }
                        }
                    }
                    if (i % nk == nk - 1) {          // expert done for this wave: scale rows, add
#pragma unroll
                        for (int b = 0; b < kNBD; ++b) {
#pragma unroll
                            for (int i2 = 0; i2 < 4; ++i2)
                                tot[b][i2] += (sd_s[jq * 32 + b * 16 + 4 * lq + i2] * unscale) * acc[b][i2];
                            acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
                        }
                    }
                }
            }
        }
    }
    if (A == 0) {          // no chunk ran: the gate still opens once
        gate.arrive();
        gate.wait();
    }
    // the waves' partial sums -> LDS -> y, summed in wave order
    if (ln < T) {
#pragma unroll
        for (int b = 0; b < kNBD; ++b)
            if (b < nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[((wave * kNBD + b) * 16 + 4 * lq + i) * 16 + ln] = tot[b][i];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nrows * T; idx += kMT) {
        const int t = idx / nrows, r = idx - t * nrows;
        const int b = r >> 4, rr = r & 15;
        float s = 0.f;
        for (int w = 0; w < kMW; ++w) s += red[((w * kNBD + b) * 16 + rr) * 16 + t];
        y[(size_t)t * H + r0 + r] = s;
    }
    __syncthreads();
}

}  // namespace mfma
}  // namespace moedec
