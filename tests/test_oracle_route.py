"""Pins of the oracle's router: sigmoid scores, noaux_tc-corrected group-limited
top-k, renormalised weights times routed_scaling_factor, and the batch union.

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
router item (DeepSeek-V3 style, noaux_tc, routed_scaling_factor, shared expert)
and batch-union item; ideipro.ru article: 8 experts per token.
"""
import itertools
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    out = []
    with open(os.path.join(GOLDEN, "route_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, shape, s, b, idx, w = (p.strip() for p in line.split("|"))
            E, G, TG, K, rsf = shape.split()
            out.append((name, int(E), int(G), int(TG), int(K), float(rsf),
                        [float(v) for v in s.split(",")], [float(v) for v in b.split(",")],
                        [int(v) for v in idx.split(",")], [float(v) for v in w.split(",")]))
    return out


@pytest.mark.parametrize("case", _worked(), ids=lambda c: c[0])
def test_worked_routing_cases(case):
    name, E, G, TG, K, rsf, s, b, idx, w = case
    got_i, got_w = orc.select_experts(np.array([s], np.float32), np.array(b, np.float32),
                                      G, TG, K, rsf)
    assert got_i[0].tolist() == idx
    np.testing.assert_allclose(got_w[0], w, rtol=2e-7)


def test_sigmoid_matches_library():
    z = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(orc.sigmoid(z), expit(z), rtol=1e-15, atol=0)
    assert orc.sigmoid(0.0) == 0.5


def test_router_scores_closed_form():
    """One-hot token picks a column of the router: s = sigmoid(W_r[:, j] * a)."""
    g = np.random.default_rng(0)
    W = g.standard_normal((16, 32)).astype(np.float32)
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = 1.5
    np.testing.assert_allclose(orc.router_scores(x, W)[0], expit(1.5 * W[:, 5].astype(np.float64)),
                               rtol=1e-15)


def _brute_select(s, b, G, TG, K, rsf):
    """Selection by enumerating subsets: the kept groups are the one subset of
    size TG whose every member beats every non-member on (group score, -index);
    the chosen experts likewise among the kept groups' members."""
    s = np.asarray(s, np.float32)
    c = s + np.asarray(b, np.float32)
    E = len(c)
    per = E // G
    gs = []
    for g in range(G):
        m = c[g * per:(g + 1) * per]
        pairs = [np.float32(m[i] + m[j]) for i in range(per) for j in range(per) if i != j]
        gs.append(max(pairs))       # the largest sum over pairs of members
    key_g = lambda g: (float(gs[g]), -g)
    kept = [S for S in itertools.combinations(range(G), TG)
            if all(key_g(a) > key_g(o) for a in S for o in range(G) if o not in S)]
    assert len(kept) == 1
    cand = [e for e in range(E) if e // per in kept[0]]
    key_e = lambda e: (float(c[e]), -e)
    chosen = [S for S in itertools.combinations(cand, K)
              if all(key_e(a) > key_e(o) for a in S for o in cand if o not in S)]
    assert len(chosen) == 1
    order = sorted(chosen[0], key=key_e, reverse=True)
    tot = float(sum(float(s[e]) for e in order))
    return order, [float(s[e]) / tot * rsf for e in order]


@pytest.mark.parametrize("seed", range(40))
def test_selection_matches_subset_enumeration(seed):
    g = np.random.default_rng(seed)
    G, per = [(4, 4), (4, 2), (3, 3), (2, 4)][seed % 4]
    E = G * per
    TG = int(g.integers(1, G + 1))
    K = int(g.integers(1, min(TG * per, 5) + 1))
    s = expit(g.standard_normal((3, E))).astype(np.float32)
    if seed % 5 == 0:               # force exact ties in scores
        s = np.round(s * 4) / 4
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    if seed % 7 == 0:
        b[:] = 0
    idx, w = orc.select_experts(s, b, G, TG, K, 2.5)
    for t in range(3):
        order, ww = _brute_select(s[t], b, G, TG, K, 2.5)
        assert idx[t].tolist() == order
        np.testing.assert_allclose(w[t], ww, rtol=3e-7)


@pytest.mark.parametrize("seed", range(6))
def test_nan_scores_rank_last(seed):
    """Reading R6: a NaN corrected score selects as -inf does (ties by index);
    the brute-force enumerator, given -inf there, is the reference."""
    g = np.random.default_rng(100 + seed)
    G, per, TG, K = 4, 4, 2, 4
    s = expit(g.standard_normal((2, G * per))).astype(np.float32)
    b = g.uniform(-0.1, 0.1, G * per).astype(np.float32)
    holes = g.choice(G * per, size=5 + seed, replace=False)
    b_nan, b_inf = b.copy(), b.copy()
    b_nan[holes] = np.nan
    b_inf[holes] = -np.inf
    idx, _ = orc.select_experts(s, b_nan, G, TG, K, 2.5)
    for t in range(2):
        order, _ = _brute_select(s[t], b_inf, G, TG, K, 2.5)
        assert idx[t].tolist() == order
        assert len(set(idx[t].tolist())) == K


def test_inf_minus_inf_group_ranks_last():
    """Reading R6: a group whose top two corrected scores are +inf and -inf has
    a NaN sum, ranked as -inf: with three finite groups and two kept, it is
    never kept, as if all its members were -inf."""
    g = np.random.default_rng(7)
    s = expit(g.standard_normal((3, 16))).astype(np.float32)
    b = g.uniform(-0.1, 0.1, 16).astype(np.float32)
    b_odd, b_ref = b.copy(), b.copy()
    b_odd[4:8] = [np.inf, -np.inf, -np.inf, -np.inf]
    b_ref[4:8] = -np.inf
    idx, _ = orc.select_experts(s, b_odd, 4, 2, 4, 2.5)
    for t in range(3):
        order, _ = _brute_select(s[t], b_ref, 4, 2, 4, 2.5)
        assert idx[t].tolist() == order
        assert not any(4 <= e < 8 for e in idx[t])


def test_single_group_is_plain_topk():
    """n_group = topk_group = 1 reduces to a stable top-k of s + b."""
    g = np.random.default_rng(3)
    s = expit(g.standard_normal((20, 16))).astype(np.float32)
    s[::3, 2] = s[::3, 9]                      # ties
    b = g.uniform(-0.1, 0.1, 16).astype(np.float32)
    idx, _ = orc.select_experts(s, b, 1, 1, 4, 2.5)
    for t in range(20):
        c = s[t] + b
        want = np.argsort(-c, kind="stable")[:4]
        assert idx[t].tolist() == want.tolist()


def test_all_tied_scores():
    """x = 0 and b = 0: every score is 0.5, so the lowest groups and indices win
    and every weight is rsf / K exactly."""
    x = np.zeros((2, 256), np.float32)
    W = np.random.default_rng(0).standard_normal((16, 256)).astype(np.float32)
    s = orc.router_scores(x, W).astype(np.float32)
    assert np.all(s == 0.5)
    idx, w = orc.select_experts(s, np.zeros(16, np.float32), 4, 2, 4, 2.5)
    assert idx.tolist() == [[0, 1, 2, 3]] * 2
    assert np.all(w == np.float32(0.625))


@pytest.mark.parametrize("K", [1, 4, 8])
def test_weights_sum_to_scaling_factor(K):
    g = np.random.default_rng(K)
    s = expit(3.9 * g.standard_normal((50, 64))).astype(np.float32)
    b = g.uniform(-0.1, 0.1, 64).astype(np.float32)
    _, w = orc.select_experts(s, b, 8, 4, K, 2.5)
    tot = w.astype(np.float64).sum(axis=1)
    np.testing.assert_allclose(tot, 2.5, rtol=K * 2.4e-7)
    if K == 1:
        assert np.all(w == np.float32(2.5))


def test_selection_margin_certifies():
    """Wherever the fp64 margin is wide, perturbing the scores by far less than
    the margin never changes the selected set."""
    g = np.random.default_rng(11)
    s64 = expit(3.9 * g.standard_normal((30, 64)))
    b = g.uniform(-0.1, 0.1, 64).astype(np.float32)
    m = orc.selection_margin(s64, b, 8, 4, 8)
    i0, _ = orc.select_experts(s64.astype(np.float32), b, 8, 4, 8, 2.5)
    for t in range(30):
        eps = m[t] / 8
        pert = (s64[t] + g.uniform(-eps, eps, 64)).astype(np.float32)[None]
        i1, _ = orc.select_experts(pert, b, 8, 4, 8, 2.5)
        assert sorted(i1[0]) == sorted(i0[t])


def test_batch_union_invariants():
    g = np.random.default_rng(5)
    T, K, E, S = 7, 4, 16, 1
    idx = np.stack([g.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    wl = orc.batch_union(idx, E, S)
    assert list(wl.expert_id) == sorted(set(idx.ravel().tolist()) | {E})
    assert wl.seg[0] == 0 and wl.seg[-1] == T * (K + S)
    assert sorted(wl.assign.tolist()) == list(range(T * (K + S)))
    for j, e in enumerate(wl.expert_id):
        seg = wl.assign[wl.seg[j]:wl.seg[j + 1]]
        assert list(seg) == sorted(seg)
        for a in seg:
            t, slot = divmod(int(a), K + S)
            assert (idx[t, slot] == e) if slot < K else (e == E)


def test_margins_follow_the_nonfinite_reading():
    """The certificates rank NaN and +inf + -inf group scores as -inf (R6),
    as the selection itself does: worked rows."""
    s = np.array([[0.9, 0.8, 0.7, 0.6, 0.5, 0.4, 0.3, 0.2]])
    b = np.array([np.nan, 0, 0, 0, 0, 0, 0, 0], np.float32)
    idx, _ = orc.select_experts(s.astype(np.float32), b, 1, 1, 3, 2.5)
    assert idx.tolist() == [[1, 2, 3]]                          # expert 0 ranks as -inf
    assert abs(orc.selection_margin(s, b, 1, 1, 3)[0] - 0.1) < 1e-12   # c[3] - c[4]
    assert abs(orc.order_margin(s, b, idx)[0] - 0.1) < 1e-12
    # group 0 = experts {0, 1} holds +inf and -inf: its score is NaN and ranks last
    b2 = np.zeros(8, np.float32)
    b2[0], b2[1] = np.inf, -np.inf
    idx2, _ = orc.select_experts(s.astype(np.float32), b2, 4, 2, 2, 2.5)
    assert idx2.tolist() == [[2, 3]]                            # groups 1 (1.3) and 2 (0.9) kept
    m = orc.selection_margin(s, b2, 4, 2, 2)[0]
    assert abs(m - 0.1) < 1e-12                                 # min(gs[2] - gs[3] = 0.4, c[3] - c[4] = 0.1)
