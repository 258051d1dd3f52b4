"""GPU parity of the pre-norm residual form: one fused launch per layer
(moe_layer_fused_resid_q*, x_out = x + MoE(rmsnorm(x)) with the norm inside
the launch) and stacks of layers through ops.stack_forward, against the
oracle's moe_stack.

The pages describe one MoE layer; x <- x + MoE(rmsnorm(x)) with a weightless
RMSNorm is the reading used to chain layers.  The oracle normalises in fp64
and rounds the normalised tokens to fp32; the launch scales x by its own fp32
1/rms, so the scores differ in the last bits and near-ties are certified by
the oracle's margins as in the single-layer tests.
"""
import gc

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from quantized_moe_decode_route_amd import ops, synth

from _parity import MARGIN, TOL, check_all, rel_err, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name: (T, H, I, E, G, TG, K, S, bits)
SHAPES = {
    "tiny": (1, 256, 128, 16, 4, 2, 4, 1, 4),
    "t3_ragged_rows_s2": (3, 2048, 544, 64, 8, 3, 6, 2, 4),
    "t5_q8_noshared": (5, 1536, 320, 16, 2, 1, 2, 0, 8),
    "t2_q2_small": (2, 512, 256, 32, 4, 2, 4, 1, 2),
}


def _cfg(name, seed=21, layers=1):
    T, H, I, E, G, TG, K, S, b = SHAPES[name]
    return synth.MoEConfig(name, T, H, I, E, G, TG, K, S, b, layers=layers, seed=seed)


def _kw(cfg):
    return dict(n_group=cfg.n_group, topk_group=cfg.topk_group, top_k=cfg.top_k, rsf=cfg.rsf)


def _resid_layer(cfg, lay, x: np.ndarray, top_p=None, in_place=False):
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    ex = ops.Experts.from_layer(lay, cfg.n_experts, cfg.n_shared, cfg.bits)
    buf = ops.LayerBuffers.allocate(cfg.tokens, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared, DEV)
    xo = xt if in_place else torch.empty_like(xt)
    ops.layer_fused(xt, lay["router_w"], lay["bias"], ex, buf=buf, top_p=top_p, x_out=xo, **_kw(cfg))
    torch.cuda.synchronize()
    assert not buf.fused_error()
    wl = buf.route.worklist
    n = int(wl.n_active.item())
    seg = wl.seg[:n + 1].cpu().numpy()
    return dict(scores=buf.route.scores.cpu().numpy(), idx=buf.route.topk_idx.cpu().numpy(),
                w=buf.route.topk_w.cpu().numpy(), n_active=n, expert_id=wl.expert_id[:n].cpu().numpy(), seg=seg,
                assign=wl.assign[:int(seg[-1])].cpu().numpy(), h=buf.h.cpu().numpy(), y=buf.y.cpu().numpy(),
                x_out=xo.cpu().numpy(), top_p=top_p)


def _gdict(buf, top_p=None) -> dict:
    wl = buf.route.worklist
    n = int(wl.n_active.item())
    seg = wl.seg[:n + 1].cpu().numpy()
    return dict(scores=buf.route.scores.cpu().numpy(), idx=buf.route.topk_idx.cpu().numpy(),
                w=buf.route.topk_w.cpu().numpy(), n_active=n, expert_id=wl.expert_id[:n].cpu().numpy(), seg=seg,
                assign=wl.assign[:int(seg[-1])].cpu().numpy(), h=buf.h.cpu().numpy(), y=buf.y.cpu().numpy(),
                top_p=top_p)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("top_p", [None, 0.7])
def test_resid_layer_matches_oracle(name, top_p):
    cfg = _cfg(name)
    say(f"case {name} resid top_p={top_p}: {SHAPES[name]}")
    lay = synth.layer_device(cfg, 0, DEV)
    # an un-normalised residual stream: tokens at a scale far from 1
    x = synth.token_pool(cfg, cfg.tokens) * np.float32(7.5)
    g = _resid_layer(cfg, lay, x, top_p=top_p)
    np.testing.assert_array_equal(g["x_out"], x + g["y"])           # x_out = x + y in fp32
    xn = orc.rmsnorm(x).astype(np.float32)                            # the oracle's normalised tokens
    rw, b = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
    check_all(cfg, g, xn, rw, b, synth.expert_loader(cfg, 0))


def test_resid_in_place_is_identical():
    cfg = _cfg("t3_ragged_rows_s2", seed=23)
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens) * np.float32(3.0)
    a = _resid_layer(cfg, lay, x)
    b = _resid_layer(cfg, lay, x, in_place=True)
    for k in ("scores", "idx", "w", "h", "y", "x_out"):
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "split"])
def test_stack_matches_oracle(fused):
    """Four layers through stack_forward (fused: one resid launch per layer;
    split: the separate calls and the norm kernel) against the oracle's stack,
    token by token while every layer's routing is certified."""
    cfg = _cfg("t3_ragged_rows_s2", seed=29, layers=4)
    L, T = cfg.layers, cfg.tokens
    lays = [synth.layer_device(cfg, l, DEV) for l in range(L)]
    layers = [(l["router_w"], l["bias"], ops.Experts.from_layer(l, cfg.n_experts, cfg.n_shared, cfg.bits))
              for l in lays]
    bufs = [ops.LayerBuffers.allocate(T, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared, DEV)
            for _ in range(L)]
    x0 = synth.token_pool(cfg, T) * np.float32(4.0)
    x = torch.from_numpy(x0).to(DEV)
    ran_fused = ops.stack_forward(x, layers, bufs, fused=fused, **_kw(cfg))
    assert ran_fused == fused
    got = x.cpu().numpy()
    ref = orc.moe_stack(x0, [(synth.router_weight(cfg, l), synth.router_bias(cfg, l), synth.expert_loader(cfg, l))
                             for l in range(L)], n_group=cfg.n_group, topk_group=cfg.topk_group, top_k=cfg.top_k,
                        n_shared=cfg.n_shared, rsf=cfg.rsf, bits=cfg.bits)
    ok = np.ones(T, bool)
    for r in ref:
        ok &= (r.margin >= MARGIN) & (r.order >= MARGIN)
    say(f"  certified tokens {int(ok.sum())}/{T}")
    assert ok.any()
    err = rel_err(got[ok], ref[-1].y[ok])
    say(f"  x after {L} layers: err {err:.2e}")
    # an end-to-end bar only: each layer's y is held to 1e-3 of its own row
    # maximum below, and those errors (and their effect on later layers'
    # inputs) add up over the L layers, so the stream gets L * 1e-3
    assert err <= L * TOL
    # every layer on its own: the layers again one at a time from x0 (the
    # same bits as the whole stack), the oracle on the device's stream
    # before each layer, h and y at 1e-3
    x = torch.from_numpy(x0).to(DEV)
    for l in range(L):
        xin = x.cpu().numpy().copy()
        ops.stack_forward(x, [layers[l]], [bufs[l]], fused=fused, **_kw(cfg))
        torch.cuda.synchronize()
        say(f"  layer {l}:")
        check_all(cfg, _gdict(bufs[l]), orc.rmsnorm(xin).astype(np.float32), synth.router_weight(cfg, l),
                  synth.router_bias(cfg, l), synth.expert_loader(cfg, l))
    np.testing.assert_array_equal(x.cpu().numpy(), got)


def test_glm_resid_layer_full_size():
    """The full GLM-5.2 layer (every expert resident) in the residual form."""
    cfg = synth.CONFIGS["glm_t1"]
    say("case glm_t1 resid")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.batch_tokens(cfg, 5) * np.float32(12.0)
    g = _resid_layer(cfg, lay, x)
    np.testing.assert_array_equal(g["x_out"], x + g["y"])
    xn = orc.rmsnorm(x).astype(np.float32)
    check_all(cfg, g, xn, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), synth.expert_loader(cfg, 0))
    del lay
    gc.collect()
    torch.cuda.empty_cache()
