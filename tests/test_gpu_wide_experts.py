"""Routing and layer parity at 512 and 1024 routed experts (8 and 16 experts
per lane in the selection's wave arg-max), through the fused call (at most
512 experts) and the separate calls, against the oracle.

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented
features", router item (sigmoid router, noaux_tc correction, group-limited
top-k); the pages' model has 256 experts, these cases cover the wider
instantiations the C ABI accepts.
"""
import pytest

from quantized_moe_decode_route_amd import synth

from _parity import check_all, run_layer, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name: (T, H, I, E, G, TG, K, S, bits), fused?
CASES = {
    "e512_fused": ((3, 512, 128, 512, 8, 4, 8, 1, 4), True),
    "e512_split": ((3, 512, 128, 512, 8, 4, 8, 1, 4), False),
    "e1024_split": ((2, 512, 128, 1024, 16, 4, 8, 1, 4), False),
    "e1024_split_t9": ((9, 256, 128, 1024, 8, 2, 6, 1, 8), False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_wide_expert_count(name):
    (T, H, I, E, G, TG, K, S, b), fused = CASES[name]
    cfg = synth.MoEConfig(name, T, H, I, E, G, TG, K, S, b, seed=63)
    say(f"case {name}: T={T} E={E} groups={G} fused={fused}")
    lay = synth.layer_device(cfg, 0, DEV)
    for step in (0, 1):
        x = synth.batch_tokens(cfg, step)
        g = run_layer(cfg, lay, x, fused=fused)
        say(f"  step {step}: {g['n_active']} active experts")
        check_all(cfg, g, x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), synth.expert_loader(cfg, 0))
