"""Shared helpers of the GPU parity tests: run a layer through the C ABI, run
the oracle on the same seeded inputs, and compare.

The oracle takes its own routing (its fp64 scores rounded to fp32, the
decision in fp32 as the kernel takes it); nothing it computes is fed from
the GPU side.  Tolerances:
  * sigmoid scores: 2e-6 absolute against the fp64 oracle;
  * expert ids: equal as sets wherever the oracle's fp64 selection margin is
    at least 1e-5, and equal in slot order (with weights within 2e-6
    relative) wherever the gaps between consecutive chosen experts are too;
    below those margins fp32 rounding may legitimately flip a near-tie, and
    the GPU's choice is then only checked to be valid: its own fp32 scores,
    which lie within 2e-6 of the oracle's, select exactly that set;
  * with adaptive top-p, a token's set also needs the oracle's top-p margin
    (prefix sums and score gaps away from the cut by 1e-5 of the total);
  * worklist (batch union): bit-exact when every token's order is
    certified; otherwise checked to be the batch union of the GPU's ids;
  * h rows and y rows: max|gpu - oracle| / max|oracle| <= 1e-3 per row
    (fp32 accumulation against fp64), the bar the workload states, on every
    certified token.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from quantized_moe_decode_route_amd import ops

TOL = 1e-3
SCORE_ATOL = 2e-6
W_RTOL = 2e-6
MARGIN = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def experts_dev(cfg, lay) -> ops.Experts:
    return ops.Experts.from_layer(lay, cfg.n_experts, cfg.n_shared, cfg.bits)


def run_layer(cfg, lay, x: np.ndarray, fused: bool | None = None, top_p: float | None = None,
              act8: bool = False) -> dict:
    """One layer on the GPU (fused: the single-launch call; False: route +
    gate/up + down; None: whichever moe_layer picks; top_p: the adaptive
    top-p calls); results on the host."""
    dev = lay["router_w"].device
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    ex = experts_dev(cfg, lay)
    try:
        buf = ops.moe_layer(xt, lay["router_w"], lay["bias"], ex, n_group=cfg.n_group, topk_group=cfg.topk_group,
                            top_k=cfg.top_k, rsf=cfg.rsf, fused=fused, top_p=top_p, act8=act8)
    except ops.MoedecError as err:
        if (fused or act8) and err.status == ops.MOEDEC_ERR_UNSUPPORTED:
            pytest.skip("the activations of this batch do not fit the fused call's LDS plan")
        raise
    torch.cuda.synchronize()
    assert not buf.fused_error(), "a grid barrier of the fused launch timed out"
    wl = buf.route.worklist
    n = int(wl.n_active.item())
    seg = wl.seg[:n + 1].cpu().numpy()
    return dict(scores=buf.route.scores.cpu().numpy(), idx=buf.route.topk_idx.cpu().numpy(),
                w=buf.route.topk_w.cpu().numpy(), n_active=n, expert_id=wl.expert_id[:n].cpu().numpy(),
                seg=seg, assign=wl.assign[:int(seg[-1])].cpu().numpy(), h=buf.h.cpu().numpy(),
                y=buf.y.cpu().numpy(), top_p=top_p, act8=act8)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the last axis, worst row."""
    got = np.atleast_2d(got).astype(np.float64)
    ref = np.atleast_2d(ref).astype(np.float64)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((np.abs(got - ref).max(axis=-1) / den).max())


def oracle_layer(cfg, x: np.ndarray, router_w: np.ndarray, bias: np.ndarray, expert_fn,
                 top_p: float | None = None, act8: bool = False) -> orc.LayerResult:
    return orc.moe_layer(x, router_w, bias, expert_fn, n_group=cfg.n_group, topk_group=cfg.topk_group,
                         top_k=cfg.top_k, n_shared=cfg.n_shared, rsf=cfg.rsf, bits=cfg.bits,
                         top_p=1.0 if top_p is None else top_p, act8=act8)


def oracle_layer_c(cfg, x: np.ndarray, router_w: np.ndarray, bias: np.ndarray, expert_fn) -> orc.LayerResult:
    """The same LayerResult from the plain-C oracle (oracle/moe_ref.c, on
    every host thread; a second implementation, cross-checked against the
    NumPy one on the CPU), for the full-size sweeps the NumPy oracle is too
    slow for.  The selection certificates come from the NumPy oracle's margin
    functions on the C oracle's fp64 scores; the routing of the two must
    agree.  Plain top-k, fp32 activations only."""
    from oracle import moe_ref
    x = np.asarray(x, np.float32)
    E, S, K = router_w.shape[0], cfg.n_shared, cfg.top_k
    s64 = orc.router_scores(x, router_w)
    idx, w = orc.select_experts(s64.astype(np.float32), bias, cfg.n_group, cfg.topk_group, K, cfg.rsf)
    wl = orc.batch_union(idx, E, S)
    experts = {int(e): expert_fn(int(e)) for e in wl.expert_id}
    c = moe_ref.layer(x, router_w, bias, experts, n_group=cfg.n_group, topk_group=cfg.topk_group, top_k=K,
                      n_shared=S, rsf=cfg.rsf, bits=cfg.bits, threads=moe_ref.max_threads())
    np.testing.assert_array_equal(c.idx, idx)                  # the two oracles route alike
    assert np.abs(c.scores64 - s64).max() <= 1e-12
    margin = orc.selection_margin(s64, bias, cfg.n_group, cfg.topk_group, K)
    return orc.LayerResult(s64, idx, c.w, wl, c.h, c.y, margin, orc.order_margin(s64, bias, idx),
                           np.full(x.shape[0], np.inf))


def check_routing(cfg, g: dict, r: orc.LayerResult, bias: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Returns (set_certified, order_certified) per token after checking."""
    d = np.abs(g["scores"].astype(np.float64) - r.scores64)
    both_nan = np.isnan(g["scores"]) & np.isnan(r.scores64)     # a token whose x holds a NaN
    err = float(np.where(both_nan, 0.0, np.where(np.isnan(d), np.inf, d)).max())
    assert err <= SCORE_ATOL, f"scores off by {err}"
    set_ok = (r.margin >= MARGIN) & (r.topp >= MARGIN)       # top-p: the kept prefix is certified too
    order_ok = set_ok & (r.order >= MARGIN)
    for t in range(len(set_ok)):
        if set_ok[t]:
            assert sorted(g["idx"][t]) == sorted(r.idx[t]), f"token {t}: {g['idx'][t]} vs {r.idx[t]}"
        if order_ok[t]:
            np.testing.assert_array_equal(g["idx"][t], r.idx[t])
            np.testing.assert_allclose(g["w"][t], r.w[t], rtol=W_RTOL)
        if not order_ok[t]:
            # near-tie: the GPU's choice must be what its own (checked) scores select
            i_v, w_v, _ = orc.select_experts_topp(g["scores"][t:t + 1], bias, cfg.n_group, cfg.topk_group,
                                                  cfg.top_k, cfg.rsf, 1.0 if g["top_p"] is None else g["top_p"])
            np.testing.assert_array_equal(g["idx"][t], i_v[0])
            np.testing.assert_array_equal(g["w"][t], w_v[0])
    if order_ok.all():
        wl = r.worklist
    else:
        wl = orc.batch_union(g["idx"], cfg.n_experts, cfg.n_shared)
    assert g["n_active"] == len(wl.expert_id)
    np.testing.assert_array_equal(g["expert_id"], wl.expert_id)
    np.testing.assert_array_equal(g["seg"], wl.seg)
    np.testing.assert_array_equal(g["assign"], wl.assign)
    say(f"  routing: score err {err:.2e}; certified sets {int(set_ok.sum())}/{len(set_ok)}, "
        f"orders {int(order_ok.sum())}/{len(set_ok)}")
    return set_ok, order_ok


def check_layer(cfg, g: dict, r: orc.LayerResult, set_ok: np.ndarray, order_ok: np.ndarray) -> tuple[float, float]:
    """h rows of order-certified tokens and y rows of set-certified tokens."""
    assert set_ok.any(), "no token has a certified selection"
    slots = cfg.top_k + cfg.n_shared
    # rows of the slots that hold an expert (top-p leaves dropped slots unwritten)
    rows = [t * slots + s for t in range(len(order_ok)) if order_ok[t] for s in range(slots)
            if s >= cfg.top_k or r.idx[t, s] >= 0]
    eh = rel_err(g["h"][rows], r.h[rows]) if rows else 0.0
    ey = rel_err(g["y"][set_ok], r.y[set_ok])
    say(f"  outputs: h err {eh:.2e} ({len(rows)} rows), y err {ey:.2e} ({int(set_ok.sum())} tokens)")
    assert eh <= TOL and ey <= TOL
    return eh, ey


def check_all(cfg, g: dict, x, router_w, bias, expert_fn, c_oracle: bool = False) -> orc.LayerResult:
    if c_oracle:
        assert g.get("top_p") is None and not g.get("act8", False)
        r = oracle_layer_c(cfg, x, router_w, bias, expert_fn)
    else:
        r = oracle_layer(cfg, x, router_w, bias, expert_fn, g.get("top_p"), g.get("act8", False))
    set_ok, order_ok = check_routing(cfg, g, r, bias)
    check_layer(cfg, g, r, set_ok, order_ok)
    return r
