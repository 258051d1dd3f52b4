"""GPU parity of adaptive expert top-p (moe_route_topp, moe_layer_fused_topp_q*)
against the oracle, through the same checks as the plain top-k calls.

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "model download और run":
the --topp option keeps only as many routed experts per token as the mass p
needs, so fewer experts are read.  Shapes: small layers element by element
(both the one-wave and the workgroup batch-union paths, int8 / int4 / int2,
with and without a shared expert), p = 0 (one expert), mid values and p = 1
(bit-identical to plain top-k), and the full GLM-5.2 layer in the launch the
benchmark times.
"""
import gc

import numpy as np
import pytest
import torch

from quantized_moe_decode_route_amd import ops, synth

from _parity import check_all, run_layer, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name: (T, H, I, E, G, TG, K, S, bits)
SHAPES = {
    "tiny": (1, 256, 128, 16, 4, 2, 4, 1, 4),
    "t3_ragged_rows_s2": (3, 2048, 544, 64, 8, 3, 6, 2, 4),
    "t5_q8_noshared": (5, 1536, 320, 16, 2, 1, 2, 0, 8),
    "t16_q2": (16, 4096, 1024, 64, 8, 4, 8, 1, 2),
    "t64_max_tokens": (64, 512, 128, 64, 8, 4, 8, 1, 4),
    "t7_odd_groups_q4": (7, 2144, 96, 24, 3, 2, 5, 1, 4),
}


def _cfg(name, seed=13):
    T, H, I, E, G, TG, K, S, b = SHAPES[name]
    return synth.MoEConfig(name, T, H, I, E, G, TG, K, S, b, seed=seed)


CASES = [(n, p, f) for n in SHAPES for p in (0.0, 0.6, 0.85) for f in (False, True)
         if not (f and SHAPES[n][0] > ops.FUSED_MAX_TOKENS)]


@pytest.mark.parametrize("name,top_p,fused", CASES,
                         ids=[f"{n}-p{p}-{'fused' if f else 'split'}" for n, p, f in CASES])
def test_topp_layer_matches_oracle(name, top_p, fused):
    cfg = _cfg(name)
    say(f"case {name} top_p={top_p} {'fused' if fused else 'split'}: {SHAPES[name]}")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens)
    g = run_layer(cfg, lay, x, fused=fused, top_p=top_p)
    kept = (g["idx"] >= 0).sum(axis=1)
    say(f"  kept experts per token: {kept.tolist()}, unique experts {g['n_active']}")
    if top_p == 0.0:
        assert (kept == 1).all() and (g["w"][:, 0] == np.float32(cfg.rsf)).all()
    rw, b = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
    check_all(cfg, g, x, rw, b, synth.expert_loader(cfg, 0))


@pytest.mark.parametrize("fused", [False, True], ids=["split", "fused"])
def test_p_one_is_bit_identical_to_topk(fused):
    cfg = _cfg("t3_ragged_rows_s2", seed=17)
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens)
    a = run_layer(cfg, lay, x, fused=fused)
    b = run_layer(cfg, lay, x, fused=fused, top_p=1.0)
    for k in ("scores", "idx", "w", "expert_id", "seg", "assign", "h", "y"):
        np.testing.assert_array_equal(a[k], b[k])


def test_rejects_nan_p():
    cfg = _cfg("tiny")
    lay = synth.layer_device(cfg, 0, DEV)
    x = torch.from_numpy(synth.token_pool(cfg, 1)).to(DEV)
    ex = ops.Experts.from_layer(lay, cfg.n_experts, cfg.n_shared, cfg.bits)
    for fused in (False, True):
        with pytest.raises(ops.MoedecError):
            ops.moe_layer(x, lay["router_w"], lay["bias"], ex, n_group=cfg.n_group, topk_group=cfg.topk_group,
                          top_k=cfg.top_k, rsf=cfg.rsf, fused=fused, top_p=float("nan"))


@pytest.mark.parametrize("name,fused", [("glm_t1", True), ("glm_t1", False), ("glm_t3", True)])
def test_glm_layer_topp(name, fused):
    """The full GLM-5.2 layer (every expert resident) at p = 0.7, the value
    the pages run with; the oracle checks every output of the batch."""
    cfg = synth.CONFIGS[name]
    say(f"case {name} top_p=0.7 {'fused' if fused else 'split'}")
    lay = synth.layer_device(cfg, 0, DEV)
    rw, b = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
    x = synth.batch_tokens(cfg, 3)
    g = run_layer(cfg, lay, x, fused=fused, top_p=0.7)
    say(f"  kept experts per token: {(g['idx'] >= 0).sum(axis=1).tolist()}, unique experts {g['n_active']}")
    check_all(cfg, g, x, rw, b, synth.expert_loader(cfg, 0))
    del lay
    gc.collect()
    torch.cuda.empty_cache()
