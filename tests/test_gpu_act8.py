"""GPU parity of the int8-activation layer (moe_layer_fused_act8_q*) against
the oracle run with the same Q8_0-style activation quantisation.

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
the integer-dot kernel item (Q8_0-style int8 activations).  The oracle
quantises x exactly as the launch does (same fp32 decisions on the same
inputs), so h matches to fp32 accumulation; the down input (h times its
routing weight) is quantised from the launch's own fp32 h and the oracle's
fp64 h rounded to fp32, so a code may differ by one step where a value sits
on a rounding boundary -- a change far inside the 1e-3 row tolerance.
"""
import gc

import numpy as np
import pytest
import torch

from quantized_moe_decode_route_amd import ops, synth

from _parity import check_all, run_layer, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name: (T, H, I, E, G, TG, K, S, bits); hidden and inter multiples of 512 / bits
SHAPES = {
    "tiny_q4": (1, 256, 128, 16, 4, 2, 4, 1, 4),
    "t3_q4_s2": (3, 2048, 512, 64, 8, 3, 6, 2, 4),
    "t5_q8_noshared": (5, 1536, 320, 16, 2, 1, 2, 0, 8),
    "t2_q2": (2, 512, 256, 32, 4, 2, 4, 1, 2),
    "t16_q4": (16, 1024, 256, 64, 8, 4, 8, 1, 4),
}


def _cfg(name, seed=31):
    T, H, I, E, G, TG, K, S, b = SHAPES[name]
    return synth.MoEConfig(name, T, H, I, E, G, TG, K, S, b, seed=seed)


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("top_p", [None, 0.75])
def test_act8_layer_matches_oracle(name, top_p):
    cfg = _cfg(name)
    say(f"case {name} act8 top_p={top_p}: {SHAPES[name]}")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens)
    g = run_layer(cfg, lay, x, fused=True, top_p=top_p, act8=True)
    rw, b = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
    check_all(cfg, g, x, rw, b, synth.expert_loader(cfg, 0))


def test_act8_blocks_of_very_different_scale():
    """A token whose blocks differ by twelve orders of magnitude and one zero
    block: every block keeps its own scale."""
    cfg = _cfg("t3_q4_s2", seed=37)
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens)
    blk = 512 // cfg.bits
    x[0, :blk] *= np.float32(1e-6)
    x[0, blk:2 * blk] *= np.float32(1e6)
    x[1, 3 * blk:4 * blk] = 0.0
    g = run_layer(cfg, lay, x, fused=True, act8=True)
    check_all(cfg, g, x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), synth.expert_loader(cfg, 0))


def test_act8_needs_whole_blocks():
    cfg = synth.MoEConfig("odd", 1, 256, 96, 16, 4, 2, 4, 1, 4, seed=3)     # inter 96: not whole 128-blocks
    lay = synth.layer_device(cfg, 0, DEV)
    xt = torch.from_numpy(synth.token_pool(cfg, 1)).to(DEV)
    ex = ops.Experts.from_layer(lay, cfg.n_experts, cfg.n_shared, cfg.bits)
    with pytest.raises(ops.MoedecError) as err:
        ops.moe_layer(xt, lay["router_w"], lay["bias"], ex, n_group=cfg.n_group, topk_group=cfg.topk_group,
                      top_k=cfg.top_k, rsf=cfg.rsf, act8=True)
    assert err.value.status == ops.MOEDEC_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["glm_t1", "glm_t1_q8", "glm_t1_q2"])
def test_glm_layer_act8(name):
    """The full GLM-5.2 layer (every expert resident) with int8 activations."""
    cfg = synth.CONFIGS[name]
    say(f"case {name} act8")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.batch_tokens(cfg, 1)
    g = run_layer(cfg, lay, x, fused=True, act8=True)
    check_all(cfg, g, x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), synth.expert_loader(cfg, 0))
    del lay
    gc.collect()
    torch.cuda.empty_cache()
