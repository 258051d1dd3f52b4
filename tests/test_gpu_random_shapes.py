"""GPU parity on a seeded sample of layer shapes drawn at random, against the
oracle, through the fused call and through the separate calls.

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
the router (group-limited top-k, shared experts, routed_scaling_factor), the
dequant-on-use codes (int8, packed int4, packed int2 with a scale per row)
and the batch union; the run options' --topp.  The shapes are drawn once
from a fixed seed: 1 to 64 tokens, hidden and inter sizes of whole 16-byte
code groups that are mostly not multiples of the kernels' tiles, 1 to 8
groups of 2 to 12 experts, top-k up to what the kept groups hold, 0 to 2
shared experts, every code width, plain top-k or top-p.  At 8 tokens and
more the separate calls use the expert-major down.  A second sample, of
whole activation blocks, runs the int8-activation call (the integer-dot
item: Q8_0-style activations) against the oracle's same quantisation, and
a third runs the pre-norm residual form (x_out = x + MoE(rmsnorm(x)), the
norm inside the launch) against the oracle on the normalised tokens.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc

from quantized_moe_decode_route_amd import ops, synth

from _parity import check_all, run_layer, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _shapes(n=40, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        bits = int(rng.choice([2, 4, 8]))
        q = 128 // bits                          # columns of one 16-byte code group
        H = int(rng.integers(2, 40)) * q
        I = int(rng.integers(1, 24)) * q
        G = int(rng.choice([1, 2, 3, 4, 8]))
        per = int(rng.integers(2, 13))
        E = G * per
        if E > 128:
            continue
        TG = int(rng.integers(1, G + 1))
        K = int(rng.integers(1, min(TG * per, 9) + 1))
        S = int(rng.integers(0, 3))
        T = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 24, 33, 64]))
        top_p = None if rng.random() < 0.6 else float(rng.choice([0.0, 0.5, 0.8]))
        out.append((T, H, I, E, G, TG, K, S, bits, top_p))
    return out


SHAPES = _shapes()
CASES = [(i, f) for i, s in enumerate(SHAPES) for f in (True, False) if not (f and s[0] > ops.FUSED_MAX_TOKENS)]


@pytest.mark.parametrize("i,fused", CASES, ids=[f"{i}-{'fused' if f else 'split'}" for i, f in CASES])
def test_random_shape_matches_oracle(i, fused):
    T, H, I, E, G, TG, K, S, bits, top_p = SHAPES[i]
    cfg = synth.MoEConfig(f"rand{i}", T, H, I, E, G, TG, K, S, bits, seed=100 + i)
    say(f"case rand{i} {'fused' if fused else 'split'}: T={T} H={H} I={I} E={E} G={G} TG={TG} K={K} S={S} "
        f"bits={bits} top_p={top_p}")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, T)
    g = run_layer(cfg, lay, x, fused=fused, top_p=top_p)
    check_all(cfg, g, x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), synth.expert_loader(cfg, 0))


def _act8_shapes(n=12, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        bits = int(rng.choice([2, 4, 8]))
        unit = max(32, 128 // bits)              # whole activation blocks and code groups
        H = int(rng.integers(1, 33)) * unit
        I = int(rng.integers(1, 25)) * unit
        G = int(rng.choice([1, 2, 4, 8]))
        per = int(rng.integers(2, 9))
        E = G * per
        TG = int(rng.integers(1, G + 1))
        K = int(rng.integers(1, min(TG * per, 8) + 1))
        S = int(rng.integers(0, 3))
        T = int(rng.choice([1, 2, 3, 6, 16]))
        top_p = None if rng.random() < 0.7 else float(rng.choice([0.0, 0.6]))
        out.append((T, H, I, E, G, TG, K, S, bits, top_p))
    return out


ACT8 = _act8_shapes()


@pytest.mark.parametrize("i", range(len(ACT8)))
def test_random_shape_act8_matches_oracle(i):
    T, H, I, E, G, TG, K, S, bits, top_p = ACT8[i]
    cfg = synth.MoEConfig(f"act8rand{i}", T, H, I, E, G, TG, K, S, bits, seed=200 + i)
    say(f"case act8rand{i}: T={T} H={H} I={I} E={E} G={G} TG={TG} K={K} S={S} bits={bits} top_p={top_p}")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, T)
    g = run_layer(cfg, lay, x, fused=True, top_p=top_p, act8=True)
    check_all(cfg, g, x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), synth.expert_loader(cfg, 0))


RESID = [s for s in _shapes(n=24, seed=2028) if s[0] <= ops.FUSED_MAX_TOKENS][:10]


@pytest.mark.parametrize("i", range(len(RESID)))
def test_random_shape_residual_form_matches_oracle(i):
    T, H, I, E, G, TG, K, S, bits, top_p = RESID[i]
    cfg = synth.MoEConfig(f"residrand{i}", T, H, I, E, G, TG, K, S, bits, seed=300 + i)
    say(f"case residrand{i}: T={T} H={H} I={I} E={E} G={G} TG={TG} K={K} S={S} bits={bits} top_p={top_p}")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, T) * np.float32(5.0)           # an un-normalised residual stream
    xt = torch.from_numpy(x).to(DEV)
    ex = ops.Experts.from_layer(lay, E, S, bits)
    buf = ops.LayerBuffers.allocate(T, H, I, E, K, S, DEV)
    xo = torch.empty_like(xt)
    try:
        ops.layer_fused(xt, lay["router_w"], lay["bias"], ex, buf=buf, top_p=top_p, x_out=xo, n_group=G,
                        topk_group=TG, top_k=K, rsf=cfg.rsf)
    except ops.MoedecError as err:
        if err.status == ops.MOEDEC_ERR_UNSUPPORTED:
            pytest.skip("the activations of this batch do not fit the fused call's LDS plan")
        raise
    torch.cuda.synchronize()
    assert not buf.fused_error()
    wl = buf.route.worklist
    n = int(wl.n_active.item())
    seg = wl.seg[:n + 1].cpu().numpy()
    g = dict(scores=buf.route.scores.cpu().numpy(), idx=buf.route.topk_idx.cpu().numpy(),
             w=buf.route.topk_w.cpu().numpy(), n_active=n, expert_id=wl.expert_id[:n].cpu().numpy(), seg=seg,
             assign=wl.assign[:int(seg[-1])].cpu().numpy(), h=buf.h.cpu().numpy(), y=buf.y.cpu().numpy(),
             top_p=top_p)
    np.testing.assert_array_equal(xo.cpu().numpy(), x + g["y"])          # x_out = x + y in fp32
    xn = orc.rmsnorm(x).astype(np.float32)
    check_all(cfg, g, xn, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), synth.expert_loader(cfg, 0))
