"""GPU parity at the full GLM-5.2 layer sizes, in the launch configuration the
benchmark times: every expert of the layer resident on the device, the path
run through the C ABI, and the oracle run on the host on the tokens it checks
(every output of those tokens)."""
import gc

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from quantized_moe_decode_route_amd import ops, synth

from _parity import MARGIN, TOL, check_all, oracle_layer_c, rel_err, run_layer, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _free():
    gc.collect()
    torch.cuda.empty_cache()


# fused: the single-launch call the benchmark times; split: the three separate calls
@pytest.mark.parametrize("name,steps,fused", [("glm_t1", (0, 1), True), ("glm_t1", (2,), False),
                                              ("glm_t3", (0,), True), ("glm_t3", (1,), False),
                                              ("glm_t1_q8", (0,), True), ("glm_t1_q2", (0,), True)])
def test_glm_layer(name, steps, fused):
    cfg = synth.CONFIGS[name]
    say(f"case {name} {'fused' if fused else 'split'}: T={cfg.tokens} bits={cfg.bits} steps={steps}")
    lay = synth.layer_device(cfg, 0, DEV)
    rw, b = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
    for step in steps:
        x = synth.batch_tokens(cfg, step)
        g = run_layer(cfg, lay, x, fused=fused)
        say(f"  step {step}: {g['n_active']} active experts")
        check_all(cfg, g, x, rw, b, synth.expert_loader(cfg, 0))
    del lay
    _free()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,layers,steps", [("glm_t1", (0, 1), range(8)), ("glm_t3", (0,), range(4))])
def test_glm_fused_many_batches(name, layers, steps):
    """The fused call as the benchmark runs it, over many pool batches: glm_t1
    on 16 tokens (8 steps on each of 2 resident layers), glm_t3 on 4 batches;
    every output of every batch against the plain-C oracle."""
    cfg = synth.CONFIGS[name]
    lays = {l: synth.layer_device(cfg, l, DEV) for l in layers}
    for l in layers:
        rw, b = synth.router_weight(cfg, l), synth.router_bias(cfg, l)
        for step in steps:
            say(f"case {name} fused: layer {l} step {step}")
            x = synth.batch_tokens(cfg, step + 8 * l)
            g = run_layer(cfg, lays[l], x, fused=True)
            check_all(cfg, g, x, rw, b, synth.expert_loader(cfg, l), c_oracle=True)
    del lays
    _free()


@pytest.mark.timeout(900)
def test_glm_stack16_sampled_tokens():
    """16 resident layers, 16 tokens, Zipf-skewed bias: the device runs the
    whole batch through x <- x + MoE(rmsnorm(x)); the plain-C oracle follows
    8 of the 16 tokens (they are independent in this step), at least 4 of
    them through 8 layers or more.  Each layer is checked on its own: the
    oracle takes the device's stream before the layer, normalises it in fp64,
    and its MoE output must match the device's y of that layer at 1e-3 (a
    token stops being followed at the first layer whose selection is not
    certified)."""
    cfg = synth.CONFIGS["glm_stack16"]
    T, H = cfg.tokens, cfg.hidden
    say(f"case glm_stack16: {cfg.layers} layers, T={T}")
    layers = [synth.layer_device(cfg, l, DEV) for l in range(cfg.layers)]
    x0 = synth.batch_tokens(cfg, 0)
    x = torch.from_numpy(x0).to(DEV)
    xn = torch.empty_like(x)
    ops.residual_rmsnorm(x, None, xn)
    xs_in, ys, idxs, active = [], [], [], []
    for l, lay in enumerate(layers):
        ex = ops.Experts.from_layer(lay, cfg.n_experts, cfg.n_shared, cfg.bits)
        xs_in.append(x.cpu().numpy().copy())
        buf = ops.moe_layer(xn, lay["router_w"], lay["bias"], ex, n_group=cfg.n_group,
                            topk_group=cfg.topk_group, top_k=cfg.top_k, rsf=cfg.rsf)
        ys.append(buf.y.cpu().numpy().copy())
        ops.residual_rmsnorm(x, buf.y, xn)
        idxs.append(buf.route.topk_idx.cpu().numpy())
        active.append(int(buf.route.worklist.n_active.item()))
    torch.cuda.synchronize()
    say(f"  unique experts per layer: {active}")
    del layers
    _free()
    follow = [5, 0, 9, 14, 2, 7, 11, 3]
    checked = {t: 0 for t in follow}
    for l in range(cfg.layers):
        if not follow:
            break
        rw, b = synth.router_weight(cfg, l), synth.router_bias(cfg, l)
        xin = orc.rmsnorm(xs_in[l][follow]).astype(np.float32)
        r = oracle_layer_c(cfg, xin, rw, b, synth.expert_loader(cfg, l))
        keep = []
        for i, t in enumerate(follow):
            if r.margin[i] < MARGIN:
                say(f"  layer {l}: token {t} selection margin {r.margin[i]:.1e} below {MARGIN}; stop following it")
                continue
            assert sorted(idxs[l][t]) == sorted(r.idx[i])
            e = rel_err(ys[l][t], r.y[i])
            assert e <= TOL, f"layer {l} token {t}: y err {e:.2e}"
            checked[t] += 1
            keep.append(t)
        say(f"  layer {l}: tokens {keep} within {TOL}")
        follow = keep
    say(f"  layers checked per token: {checked}")
    assert sum(v >= 8 for v in checked.values()) >= 4
