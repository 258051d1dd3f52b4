"""Pins of the oracle's adaptive expert top-p (a variant of the top-k selection
that keeps only as many of the chosen experts as the probability mass p needs).

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "model download और run"
(run options: --topp, adaptive expert top-p, fewer expert reads) and section
"community benchmarks" (the measured effect).  The rule is a reading (score
order, shortest prefix reaching p of the total, reweighting over the kept
set): these tests pin the oracle to it with hand-worked rows, brute force over
every subset of the chosen experts, the limits p >= 1 and p = 0, and
invariants of the kept set and its weights.
"""
import itertools
import os

import numpy as np
import pytest

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    out = []
    with open(os.path.join(GOLDEN, "route_topp.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            shape, s, b, idx, w = (p.strip() for p in line.split("|"))
            E, G, TG, K, rsf, p = shape.split()
            out.append((int(E), int(G), int(TG), int(K), float(rsf), float(p),
                        [float(v) for v in s.split(",")], [float(v) for v in b.split(",")],
                        [int(v) for v in idx.split(",")], [float(v) for v in w.split(",")]))
    return out


@pytest.mark.parametrize("case", _golden())
def test_worked_rows(case):
    E, G, TG, K, rsf, p, s, b, idx, w = case
    gi, gw, kept = orc.select_experts_topp(np.array([s], np.float32), np.array(b, np.float32), G, TG, K, rsf, p)
    assert gi[0].tolist() == idx
    assert np.allclose(gw[0], w, rtol=2e-7, atol=0)
    assert kept[0] == sum(1 for i in idx if i >= 0)


def _random(seed, T, E):
    rng = np.random.default_rng(seed)
    s = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, E)) * 2.0))).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    return s, b


@pytest.mark.parametrize("seed", range(6))
def test_prefix_is_the_smallest_subset_reaching_p(seed):
    """Brute force over every subset of the chosen experts, in exact
    arithmetic: the kept count is the smallest size of any subset whose score
    sum reaches p of the total, and the kept set has the largest sum among
    subsets of that size (cases within fp32 rounding of p are skipped)."""
    T, E, G, TG, K = 12, 16, 4, 2, 5
    s, b = _random(seed, T, E)
    for p in (0.3, 0.55, 0.7, 0.9):
        idx_k, _ = orc.select_experts(s, b, G, TG, K, 2.5)
        gi, gw, kept = orc.select_experts_topp(s, b, G, TG, K, 2.5, p)
        for t in range(T):
            v = {int(e): float(s[t, e]) for e in idx_k[t]}
            total = sum(v.values())
            sums = {}
            for r in range(1, K + 1):
                sums[r] = max(sum(v[e] for e in c) for c in itertools.combinations(v, r))
            if min(abs(x - p * total) for x in sums.values()) < 1e-5 * total:
                continue
            m_star = min(r for r in sums if sums[r] >= p * total)
            assert kept[t] == m_star
            ks = [int(e) for e in gi[t] if e >= 0]
            assert len(ks) == m_star and abs(sum(v[e] for e in ks) - sums[m_star]) < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_p_one_is_plain_topk_and_p_zero_keeps_the_top_score(seed):
    T, E, G, TG, K = 16, 32, 4, 2, 6
    s, b = _random(100 + seed, T, E)
    ik, wk = orc.select_experts(s, b, G, TG, K, 2.5)
    for p in (1.0, 1.5):
        ip, wp, kept = orc.select_experts_topp(s, b, G, TG, K, 2.5, p)
        assert np.array_equal(ip, ik) and np.array_equal(wp, wk) and (kept == K).all()
    ip, wp, kept = orc.select_experts_topp(s, b, G, TG, K, 2.5, 0.0)
    assert (kept == 1).all()
    for t in range(T):
        best = max(ik[t], key=lambda e: (s[t, e], -e))
        assert ip[t, 0] == best and wp[t, 0] == np.float32(2.5)        # s / s = 1 exactly
        assert (ip[t, 1:] == -1).all() and (wp[t, 1:] == 0).all()


@pytest.mark.parametrize("seed", range(3))
def test_kept_set_invariants(seed):
    T, E, G, TG, K = 20, 64, 8, 4, 8
    s, b = _random(200 + seed, T, E)
    ik, _ = orc.select_experts(s, b, G, TG, K, 2.5)
    c = s + b
    prev = np.zeros(T, np.int32)
    for p in np.linspace(0.05, 0.99, 12):
        ip, wp, kept = orc.select_experts_topp(s, b, G, TG, K, 2.5, float(p))
        assert (kept >= prev).all()                                     # monotone in p
        prev = kept
        for t in range(T):
            ks = ip[t, :kept[t]]
            assert set(ks.tolist()) <= set(ik[t].tolist())              # a subset of the top-k
            assert (ip[t, kept[t]:] == -1).all()
            assert all(c[t, ks[i]] >= c[t, ks[i + 1]] for i in range(len(ks) - 1))   # slot order kept
            assert abs(float(wp[t, :kept[t]].astype(np.float64).sum()) - 2.5) < 8 * 2.5 * 2 ** -23
            ratio = wp[t, :kept[t]].astype(np.float64) / s[t, ks].astype(np.float64)
            assert np.allclose(ratio, ratio[0], rtol=1e-6)              # weights proportional to s
            # the kept experts are the highest-scored ones
            dropped = [e for e in ik[t] if e not in set(ks.tolist())]
            if dropped:
                assert s[t, ks].min() >= s[t, dropped].max()


def test_batch_union_skips_dropped_slots():
    idx = np.array([[3, -1, -1], [5, 3, -1]], np.int32)
    wl = orc.batch_union(idx, 8, 1)
    assert wl.expert_id.tolist() == [3, 5, 8]
    assert wl.assign.tolist() == [0, 5, 4, 3, 7]                        # slots = 4: token 1 slot 1 is 5
    assert wl.seg.tolist() == [0, 2, 3, 5]


def test_layer_with_p_zero_is_top_one_plus_shared():
    """p = 0 keeps exactly the highest-scored expert with weight rsf: the layer
    output is rsf times that expert's output plus the shared expert's."""
    rng = np.random.default_rng(7)
    H, I, E, bits = 64, 32, 8, 4
    experts = {}
    lo, hi = orc.code_range(bits)
    for e in range(E + 1):
        experts[e] = {k: orc.pack_rows(rng.integers(lo, hi + 1, size=shp), bits)
                      for k, shp in (("q_gate", (I, H)), ("q_up", (I, H)), ("q_down", (H, I)))}
        experts[e].update({"s_gate": rng.uniform(0.005, 0.02, I), "s_up": rng.uniform(0.005, 0.02, I),
                           "s_down": rng.uniform(0.005, 0.02, H)})
    x = rng.standard_normal((1, H)).astype(np.float32)
    rw = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    r = orc.moe_layer(x, rw, b, experts.__getitem__, n_group=2, topk_group=1, top_k=3, n_shared=1, rsf=2.5,
                      bits=bits, top_p=0.0)
    assert r.idx[0, 1:].tolist() == [-1, -1] and r.w[0, 0] == np.float32(2.5)

    def out(e):
        d = experts[e]
        return orc.swiglu_expert(x[0], orc.dequantize(d["q_gate"], d["s_gate"], bits),
                                 orc.dequantize(d["q_up"], d["s_up"], bits),
                                 orc.dequantize(d["q_down"], d["s_down"], bits))[0]
    want = 2.5 * out(int(r.idx[0, 0])) + out(E)
    assert np.allclose(r.y[0], want, rtol=1e-12, atol=1e-12)
    assert r.worklist.expert_id.tolist() == sorted([int(r.idx[0, 0]), E])
