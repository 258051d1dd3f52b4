"""CPU oracle for the routed Mixture-of-Experts decode step (TEST INFRASTRUCTURE).

Plain, slow, obviously-correct numpy.  Only the test suite, the package's
smoke() entry and the benchmark's CPU-baseline leg may import or call this
module; the product path never does, and this module imports nothing from the
HIP library or its package.  It shares no code with the GPU side: no kernels,
no packing helpers, no tables.

What it computes, with the passages it follows (pages are cited by title and
section; every unstated point is a reading, listed as R-numbers):

[HN]    "Show HN: धीमे कंप्यूटर पर GLM 5.2 चलाना" (hi.news.hada.io), section
        "implement किए गए मुख्य features" (implemented features): the
        DeepSeek-V3-style sigmoid router item (noaux_tc, routed_scaling_factor,
        shared expert); the quantisation-kernel item (int8, packed int4, packed
        int2, one scale per row, dequantised on use); the batch-union item (each
        unique expert of a batch is read once and applied to all positions
        routed to it).
[NEWS]  ideipro.ru, "Энтузиаст запустил GLM-5.2 на ноутбуке с 25 ГБ RAM",
        body: each token consults 8 experts in each MoE layer; int8/int4/int2
        kernels with a per-row scale whose packing was checked bit for bit.
[HN-S]  same Show HN page, section "disk streaming आधारित MoE execution
        तरीका": 256 routed experts per layer, about 19 MB per int4 expert;
        shared experts belong to the always-resident dense part.

Readings (the pages are silent on these):
 R1  group score = sum of the two largest bias-corrected scores of the group
     (DeepSeek-V3's noaux_tc rule, which the router item names).
 R2  bias-corrected scores c = s + b select groups and experts; the unbiased
     sigmoid scores s give the weights.
 R3  experts outside the kept groups are not candidates (strictly group-limited).
 R4  ties go to the lower group index, then the lower expert index.
 R5  weights: w_k = (s_k / sum_j s_j) * routed_scaling_factor, the sum taken in
     slot order; slot order = c descending, ties to the lower index.
 R6  a NaN corrected score (from a NaN activation or bias), or a NaN group
     score (+inf and -inf in one group), ranks below every number, as -inf
     does, with ties to the lower index: the selection stays a well-defined
     set of distinct experts.
 R7  expert FFN = SwiGLU without biases: h = silu(Wg x) * (Wu x), o = Wd h,
     silu(g) = g / (1 + exp(-g)).
 R8  int4 code = two's-complement nibble; byte j of a row holds column 2j in
     bits 0-3 and column 2j+1 in bits 4-7 (low nibble first).
 R9  int2 code = two's-complement 2-bit field; byte j holds columns 4j..4j+3 in
     bits (0-1, 2-3, 4-5, 6-7); int8 = one two's-complement byte.
 R10 a "row" is an output row; matrices are [out, in] row-major, packed along
     the input dimension; one fp32 scale per row, symmetric, no zero point.
 R14 shared experts have weight 1 (not scaled by routed_scaling_factor).
 R15 the multi-layer stack is x <- x + MoE(rmsnorm(x)) with a weightless
     RMSNorm (eps 1e-6).
 R20 requantising fp32 rows: s = absmax(row) / qmax, qmax = 2^(bits-1) - 1
     (7 / 127 / 1), q = rint(w / s) half to even, clamped to the field; a
     zero row gets s = 0 and codes 0.  Decided in fp32.
 R21 a row holding a NaN or an infinity gets s = NaN and codes 0, so that the
     problem shows in every output computed from it.
 R23 Q8_0-style int8 activations (the integer-dot item): the activations that
     meet the weights -- each token's x, and each assignment's h times its
     routing weight (fp32) -- are quantised in blocks of 32 consecutive
     input columns, Q8_0's block (whatever the weights' code width), by
     R20's rule with qmax 127 (d = absmax / 127, q = rint(v / d) half to
     even); the dot products are then exact integer sums scaled by d.
 R22 adaptive expert top-p (the run options' --topp): after the top-k
     selection, order the K chosen experts by unbiased score s descending
     (a NaN s last, ties to the lower index), add their s in that order in
     fp32 and keep the shortest prefix whose sum reaches fp32(p * total),
     total being the slot-order fp32 sum of R5 (at least one expert; p >= 1
     keeps all K).  The kept experts stay in slot order in the first slots
     (the rest hold index -1 and weight 0) and are reweighted by R5 over the
     kept set alone.  Dropped slots have no assignment in the batch union.

Precision.  Routing decisions are taken in fp32, as the kernel takes them
(scores rounded to fp32, c = s + b and the group sums in fp32, weights in
fp32).  The expert arithmetic runs in fp64 over explicitly dequantised weights
(code * scale is exact in fp64), so it is the exact value of the quantised
layer up to fp64 rounding.

Pins (tests/test_oracle_*.py, run without a GPU): exhaustive pack/unpack
round trips and hand-derived byte fixtures; brute-force subset enumeration of
group and expert selection; the one-group case against a library sort; the
all-tied case; the weights-sum invariant; the one-hot-input and all-equal
closed forms of the FFN; the RMSNorm closed form; the ~19 MB expert size of
[HN-S]; for the row quantiser, hand-worked rows, the exact round trip of code
rows that reach +-qmax, the nearest-code brute force over the whole code
alphabet, and the sign and power-of-two scaling symmetries.  The pages
print no worked example, so the group-score rule R1, the code layouts
R8-R10, the quantiser rule R20-R21, the top-p rule R22 and the activation
blocks R23 are readings: the tests pin each function to its reading's own
mathematics (brute force, closed forms, exhaustive tables), and the
readings themselves are choices, listed with their reasons.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable

import numpy as np

SUPPORTED_BITS = (8, 4, 2)


# ----------------------------------------------------------- codes and packing
# [NEWS], [HN] quantisation item; layout readings R8-R10.

def code_range(bits: int) -> tuple[int, int]:
    """Smallest and largest two's-complement code of a `bits`-wide field."""
    return -(1 << (bits - 1)), (1 << (bits - 1)) - 1


def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    """Integer codes [rows, n] -> packed bytes [rows, n*bits/8].

    Field j of byte k (bits j*b .. j*b+b-1) holds column k*(8/b) + j, stored as
    the low b bits of the code's two's complement (R8, R9)."""
    assert bits in SUPPORTED_BITS
    codes = np.asarray(codes)
    lo, hi = code_range(bits)
    assert codes.min(initial=0) >= lo and codes.max(initial=0) <= hi, "code out of range"
    per = 8 // bits
    rows, n = codes.shape
    assert n % per == 0
    field = codes.astype(np.int64) & ((1 << bits) - 1)
    out = np.zeros((rows, n // per), dtype=np.int64)
    for j in range(per):
        out |= field[:, j::per] << (j * bits)
    return out.astype(np.uint8)


def unpack_rows(packed: np.ndarray, bits: int) -> np.ndarray:
    """Packed bytes [rows, nb] -> int8 codes [rows, nb*8/bits] (sign-extended)."""
    assert bits in SUPPORTED_BITS
    per = 8 // bits
    p = np.asarray(packed, dtype=np.uint8)
    rows, nb = p.shape
    out = np.empty((rows, nb * per), dtype=np.int16)
    for j in range(per):
        f = ((p >> (j * bits)) & ((1 << bits) - 1)).astype(np.int16)
        f[f >= (1 << (bits - 1))] -= (1 << bits)            # sign-extend
        out[:, j::per] = f
    return out.astype(np.int8)


def act8_block(bits: int) -> int:
    """Input columns per activation block for weights of `bits` (R23: Q8_0's
    block of 32, the same for every code width)."""
    return 32


def dequantize(packed: np.ndarray, scales: np.ndarray, bits: int) -> np.ndarray:
    """W[r, c] = code[r, c] * scale[r], exact in fp64 (dequant-on-use, R10)."""
    w = unpack_rows(packed, bits).astype(np.float64)
    w *= np.asarray(scales, dtype=np.float64)[:, None]
    return w


# ------------------------------------------------------------- row quantiser
# [HN] implemented features: the offline converter item (dequantise from
# 128x128 block scales, then requantise into the engine's container) and the
# quantisation item (one scale per row).  The rule is reading R20; R21 covers
# rows that hold a NaN or an infinity.

def quantize_rows(w: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """fp32 rows [rows, n] -> (int8 codes [rows, n], fp32 scales [rows]).

    Per row, in fp32 (the precision of the input, and the one the kernel
    decides the codes in): s = absmax / qmax with qmax = 2^(bits-1) - 1, and
    q = rint(w / s) (round half to even) clamped to the field's range (R20).
    A zero row (absmax 0, or s rounding to 0) gets s = 0 and codes 0; a row
    holding a NaN or an infinity gets s = NaN and codes 0 (R21)."""
    assert bits in SUPPORTED_BITS
    w32 = np.asarray(w, dtype=np.float32)
    assert w32.ndim == 2
    rows, n = w32.shape
    lo, hi = code_range(bits)
    qmax = np.float32(hi)
    codes = np.zeros((rows, n), dtype=np.int8)
    scales = np.zeros(rows, dtype=np.float32)
    for r in range(rows):
        row = w32[r]
        if not np.all(np.isfinite(row)):
            scales[r] = np.float32(np.nan)
            continue
        absmax = np.max(np.abs(row)) if n else np.float32(0.0)
        s = np.float32(absmax / qmax)                      # one fp32 division
        if s == 0:
            continue
        scales[r] = s
        ratio = (row / s).astype(np.float32)               # fp32 division per element
        q = np.rint(ratio)                                 # half to even
        codes[r] = np.clip(q, lo, hi).astype(np.int8)
    return codes, scales


def quantize_act8(v: np.ndarray, block: int) -> np.ndarray:
    """fp32 activation rows [rows, n] -> the values q * d they stand for after
    Q8_0-style quantisation in blocks of `block` columns (R23; R20's rule with
    qmax 127 applied to each block), exact in fp64."""
    v32 = np.asarray(v, dtype=np.float32)
    rows, n = v32.shape
    assert n % block == 0
    q, d = quantize_rows(v32.reshape(rows * n // block, block), 8)
    return (q.astype(np.float64) * d.astype(np.float64)[:, None]).reshape(rows, n)


# --------------------------------------------------------------------- router
# [HN] router item: sigmoid affinities, noaux_tc correction, group-limited
# top-k, renormalised weights times routed_scaling_factor; [NEWS]: top-8.

def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def router_scores(x: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """s[t, e] = sigmoid(sum_h W_r[e, h] x[t, h]) in fp64."""
    z = np.asarray(x, np.float64) @ np.asarray(router_w, np.float64).T
    return sigmoid(z)


def _top2_sum32(vals: np.ndarray) -> np.float32:
    order = sorted(range(len(vals)), key=lambda j: (-vals[j], j))
    with np.errstate(invalid="ignore"):
        g = np.float32(vals[order[0]] + vals[order[1]])
    return np.float32(-np.inf) if np.isnan(g) else g          # R6


def select_experts(scores: np.ndarray, bias: np.ndarray, n_group: int, topk_group: int,
                   top_k: int, rsf: float):
    """Group-limited top-k from fp32 sigmoid scores [T, E] and fp32 bias [E].

    Returns (idx int32 [T, K], w float32 [T, K]) in slot order (R1-R5)."""
    s = np.asarray(scores, dtype=np.float32)
    b = np.asarray(bias, dtype=np.float32)
    T, E = s.shape
    per = E // n_group
    assert per * n_group == E and per >= 2 and topk_group <= n_group
    assert top_k <= topk_group * per
    idx = np.zeros((T, top_k), dtype=np.int32)
    w = np.zeros((T, top_k), dtype=np.float32)
    rsf32 = np.float32(rsf)
    for t in range(T):
        c = s[t] + b                                         # fp32 (R2)
        c = np.where(np.isnan(c), np.float32(-np.inf), c)    # R6
        gs = [_top2_sum32(c[g * per:(g + 1) * per]) for g in range(n_group)]  # R1
        kept = sorted(range(n_group), key=lambda g: (-gs[g], g))[:topk_group]  # R4
        cand = [e for e in range(E) if e // per in kept]      # R3
        chosen = sorted(cand, key=lambda e: (-c[e], e))[:top_k]  # R4, R6
        total = np.float32(0.0)
        for e in chosen:                                     # R5: slot order
            total = np.float32(total + s[t, e])
        for k, e in enumerate(chosen):
            idx[t, k] = e
            w[t, k] = np.float32(np.float32(s[t, e] / total) * rsf32)
    return idx, w


def select_experts_topp(scores: np.ndarray, bias: np.ndarray, n_group: int, topk_group: int,
                        top_k: int, rsf: float, top_p: float):
    """Group-limited top-k, then the adaptive top-p prefix (R22).

    Returns (idx int32 [T, K], w float32 [T, K], kept int32 [T]); slots past
    kept[t] hold idx -1 and w 0."""
    idx, w = select_experts(scores, bias, n_group, topk_group, top_k, rsf)
    T = idx.shape[0]
    kept = np.full(T, top_k, dtype=np.int32)
    if not top_p < 1.0:
        return idx, w, kept
    s = np.asarray(scores, dtype=np.float32)
    rsf32, p32 = np.float32(rsf), np.float32(top_p)
    out_idx = np.full_like(idx, -1)
    out_w = np.zeros_like(w)
    for t in range(T):
        chosen = [int(e) for e in idx[t]]
        sv = {e: s[t, e] for e in chosen}
        total = np.float32(0.0)
        for e in chosen:                                       # slot order, as R5
            total = np.float32(total + sv[e])
        thr = np.float32(p32 * total)
        by_weight = sorted(chosen, key=lambda e: (np.isnan(sv[e]), -sv[e] if not np.isnan(sv[e]) else 0.0, e))
        cum, m = np.float32(0.0), top_k
        for i, e in enumerate(by_weight):
            cum = np.float32(cum + sv[e])
            if cum >= thr:
                m = i + 1
                break
        keep = set(by_weight[:m])
        kept_slots = [e for e in chosen if e in keep]          # slot order
        total2 = np.float32(0.0)
        for e in kept_slots:
            total2 = np.float32(total2 + sv[e])
        for k, e in enumerate(kept_slots):
            out_idx[t, k] = e
            with np.errstate(invalid="ignore", divide="ignore"):
                out_w[t, k] = np.float32(np.float32(sv[e] / total2) * rsf32)
        kept[t] = m
    return out_idx, out_w, kept


def selection_margin(scores64: np.ndarray, bias: np.ndarray, n_group: int, topk_group: int,
                     top_k: int) -> np.ndarray:
    """Per token, the smallest fp64 gap that decides the selected set: between
    the topk_group-th and next group score, and between the top_k-th and next
    candidate.  Where it exceeds the fp32 error of the scores, any correct fp32
    implementation must select the same experts."""
    s = np.asarray(scores64, np.float64)
    b = np.asarray(bias, np.float64)
    T, E = s.shape
    per = E // n_group
    out = np.full(T, np.inf)
    for t in range(T):
        with np.errstate(invalid="ignore"):
            c = s[t] + b
            c = np.where(np.isnan(c), -np.inf, c)                # R6: NaN ranks as -inf
            gs = np.array([np.sort(c[g * per:(g + 1) * per])[-2:].sum() for g in range(n_group)])
        gs = np.where(np.isnan(gs), -np.inf, gs)                 # R6: +inf + -inf ranks as -inf
        order = np.argsort(-gs, kind="stable")
        m = np.inf
        with np.errstate(invalid="ignore"):
            if topk_group < n_group:
                m = gs[order[topk_group - 1]] - gs[order[topk_group]]
            kept = order[:topk_group]
            cand = np.sort(np.concatenate([c[g * per:(g + 1) * per] for g in kept]))[::-1]
            if top_k < len(cand):
                m = min(m, cand[top_k - 1] - cand[top_k])
        out[t] = m if not np.isnan(m) else 0.0       # inf - inf: ties between infinities decide by index
    return out


def order_margin(scores64: np.ndarray, bias: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Per token, the smallest fp64 gap between the corrected scores of
    consecutive chosen slots (infinite for one slot): where it is wide, the
    slot order is the same for any correct fp32 implementation."""
    with np.errstate(invalid="ignore"):
        c = np.asarray(scores64, np.float64) + np.asarray(bias, np.float64)
    c = np.where(np.isnan(c), -np.inf, c)                         # R6
    out = np.full(idx.shape[0], np.inf)
    for t in range(idx.shape[0]):
        v = c[t, idx[t][idx[t] >= 0]]
        if len(v) > 1:
            with np.errstate(invalid="ignore"):
                d = v[:-1] - v[1:]
            out[t] = float(np.min(np.where(np.isnan(d), 0.0, d)))   # equal infinities: no margin
    return out


def topp_margin(scores64: np.ndarray, idx_topk: np.ndarray, top_p: float) -> np.ndarray:
    """Per token, the smallest fp64 distance between a prefix sum of the
    top-k experts' scores (in score order) and p times their total, relative to
    the total, and between consecutive scores in that order: where both are
    wide, any correct fp32 implementation keeps the same prefix (R22)."""
    out = np.full(idx_topk.shape[0], np.inf)
    if not top_p < 1.0:
        return out
    s = np.asarray(scores64, np.float64)
    for t in range(idx_topk.shape[0]):
        v = np.sort(s[t, idx_topk[t]])[::-1]
        total = v.sum()
        cum = np.cumsum(v)
        m = np.min(np.abs(cum - top_p * total)) / max(total, 1e-300)
        if len(v) > 1:
            m = min(m, float(np.min(v[:-1] - v[1:])))
        out[t] = m
    return out


# ---------------------------------------------------------- batch union
# [HN] batch-union item: each unique expert of the batch once, with every
# (token, slot) routed to it.

@dataclass
class Worklist:
    expert_id: np.ndarray   # int32 [n_active], ascending; shared j is E + j
    seg: np.ndarray         # int32 [n_active + 1], offsets into assign
    assign: np.ndarray      # int32 [T * (K + S)], entries t * (K + S) + slot


def batch_union(idx: np.ndarray, n_experts: int, n_shared: int) -> Worklist:
    T, K = idx.shape
    slots = K + n_shared
    owner = {}
    for t in range(T):
        for k in range(K):
            if idx[t, k] >= 0:                             # R22: a dropped slot has no assignment
                owner[t * slots + k] = int(idx[t, k])
        for j in range(n_shared):
            owner[t * slots + K + j] = n_experts + j
    experts = sorted(set(owner.values()))
    seg, assign = [0], []
    for e in experts:
        assign.extend(a for a in sorted(owner) if owner[a] == e)
        seg.append(len(assign))
    return Worklist(np.array(experts, np.int32), np.array(seg, np.int32),
                    np.array(assign, np.int32))


# ---------------------------------------------------------------- experts
# [HN-S] expert size; R7 SwiGLU; R14 shared weight 1.

def silu(g):
    with np.errstate(over="ignore"):
        return np.asarray(g, np.float64) / (1.0 + np.exp(-np.asarray(g, np.float64)))


def swiglu_expert(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    """One expert on one token, fp64: returns (o [H], h [I])."""
    x = np.asarray(x, np.float64)
    h = silu(wg @ x) * (wu @ x)
    return wd @ h, h


def expert_bytes(hidden: int, inter: int, bits: int) -> int:
    """Bytes of one expert record: three packed matrices plus fp32 row scales."""
    return 3 * hidden * inter * bits // 8 + 4 * (2 * inter + hidden)


@dataclass
class LayerResult:
    scores64: np.ndarray    # [T, E] fp64 sigmoid scores
    idx: np.ndarray         # [T, K] int32
    w: np.ndarray           # [T, K] float32
    worklist: Worklist
    h: np.ndarray           # [T * (K + S), I] fp64, row = assignment index
    y: np.ndarray           # [T, H] fp64
    margin: np.ndarray      # [T] fp64 selection margin (decides the set)
    order: np.ndarray       # [T] fp64 gap between consecutive slots (decides the order)
    topp: np.ndarray | None = None   # [T] fp64 top-p prefix margin (R22); inf without top-p


def moe_layer(x: np.ndarray, router_w: np.ndarray, bias: np.ndarray,
              expert: Callable[[int], dict], *, n_group: int, topk_group: int, top_k: int,
              n_shared: int, rsf: float, bits: int, top_p: float = 1.0, act8: bool = False) -> LayerResult:
    """One routed-MoE layer on T tokens.

    expert(e) returns the packed codes and row scales of expert e
    ({q_gate, q_up, q_down, s_gate, s_up, s_down}); routed experts are
    0..E-1, shared ones E..E+S-1.  The selection is taken on the fp64 scores
    rounded to fp32.  top_p < 1 adds the adaptive top-p prefix (R22); act8
    quantises the activations that meet the weights (R23): x before gate/up,
    and fp32(h) times the slot's fp32 weight before down."""
    x = np.asarray(x, np.float32)
    T = x.shape[0]
    E = router_w.shape[0]
    s64 = router_scores(x, router_w)
    idx, w, _ = select_experts_topp(s64.astype(np.float32), bias, n_group, topk_group, top_k, rsf, top_p)
    wl = batch_union(idx, E, n_shared)
    slots = top_k + n_shared
    blk = act8_block(bits)
    xin = quantize_act8(x, blk) if act8 else x
    y = np.zeros((T, router_w.shape[1]), np.float64)
    h_all = None
    for j, e in enumerate(wl.expert_id):
        d = expert(int(e))
        wg = dequantize(d["q_gate"], d["s_gate"], bits)
        wu = dequantize(d["q_up"], d["s_up"], bits)
        wd = dequantize(d["q_down"], d["s_down"], bits)
        if h_all is None:
            h_all = np.zeros((T * slots, wg.shape[0]), np.float64)
        for a in wl.assign[wl.seg[j]:wl.seg[j + 1]]:
            t, slot = divmod(int(a), slots)
            o, h = swiglu_expert(xin[t], wg, wu, wd)
            h_all[a] = h
            coef = float(w[t, slot]) if slot < top_k else 1.0
            if act8:
                hw = (h.astype(np.float32) * np.float32(coef)).astype(np.float32)
                y[t] += wd @ quantize_act8(hw[None, :], blk)[0]
            else:
                y[t] += coef * o
    margin = selection_margin(s64, bias, n_group, topk_group, top_k)
    idx_k, _ = select_experts(s64.astype(np.float32), bias, n_group, topk_group, top_k, rsf) if top_p < 1.0 \
        else (idx, None)
    return LayerResult(s64, idx, w, wl, h_all, y, margin, order_margin(s64, bias, idx),
                       topp_margin(s64, idx_k, top_p))


def rmsnorm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Weightless RMSNorm over the last axis (R15), fp64."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def moe_stack(x0: np.ndarray, layers: list[tuple], **kw) -> list[LayerResult]:
    """x_{l+1} = x_l + MoE_l(rmsnorm(x_l)) over the given layers (R15).

    layers[l] = (router_w, bias, expert_fn).  Each layer's input is rounded to
    fp32, as the device keeps activations in fp32.  Returns one LayerResult per
    layer with .y replaced by the layer's output stream x_{l+1} (fp64)."""
    x = np.asarray(x0, np.float64)
    out = []
    for rw, b, ex in layers:
        xn = rmsnorm(x).astype(np.float32)
        r = moe_layer(xn, rw, b, ex, **kw)
        x = x + r.y
        r.y = x.copy()
        out.append(r)
    return out
