"""Non-finite routing inputs through the fused, the separate and the
int8-activation calls, against the oracle (reading R6: a NaN corrected score, or a NaN group score
from +inf and -inf in one group, ranks as -inf with ties to the lower index).

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented
features", router item: the group-limited top-k over corrected scores.  Cases:
  * NaN bias on three experts of different groups (never selected);
  * a group whose two largest corrected scores are +inf and -inf (its group
    score is NaN: the group is never kept, so its +inf expert is not chosen),
    and a group holding one +inf expert among finite ones (kept, that expert
    in slot 0);
  * a NaN element of one token's x: that token's scores are NaN, so it takes
    the lowest-index groups and experts (its h and y rows are unspecified);
    every other token is checked as usual.
"""
import numpy as np
import pytest
import torch

from quantized_moe_decode_route_amd import ops, synth

from _parity import check_all, run_layer, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CFG = synth.MoEConfig("nonfinite", 4, 512, 256, 64, 8, 4, 8, 1, 4, seed=61)


def _bias(case):
    b = synth.router_bias(CFG, 0).copy()
    if case == "nan_bias":
        b[[3, 17, 40]] = np.nan
    elif case == "inf_groups":
        b[16:24] = -np.inf                     # group 2: +inf and -inf on top -> NaN group score
        b[16] = np.inf
        b[41] = np.inf                         # group 5: one +inf among finite scores
    return b


@pytest.mark.parametrize("mode", ["fused", "split", "act8"])
@pytest.mark.parametrize("case", ["nan_bias", "inf_groups", "nan_x"])
def test_nonfinite_routing(case, mode):
    """(act8: the int8-activation call, whose NaN-x token has a NaN block
    scale -- reading R21 applied to activation blocks -- so its h and y are
    NaN; the other tokens as usual.)"""
    say(f"case {case} {mode}")
    lay = synth.layer_device(CFG, 0, DEV)
    b = _bias(case)
    lay["bias"] = torch.from_numpy(b).to(DEV)
    x = synth.batch_tokens(CFG, 0).copy()
    if case == "nan_x":
        x[1, 7] = np.nan
    g = run_layer(CFG, lay, x, fused=mode != "split", act8=mode == "act8")
    r = check_all(CFG, g, x, synth.router_weight(CFG, 0), b, synth.expert_loader(CFG, 0))
    if case == "nan_bias":
        assert not np.isin(g["idx"], [3, 17, 40]).any()
    elif case == "inf_groups":
        assert not np.isin(g["idx"], np.arange(16, 24)).any()
        assert (g["idx"][:, 0] == 41).all()
    else:
        # token 1: every corrected score ranks as -inf, so groups 0..3 and, within them, the lowest indices
        np.testing.assert_array_equal(g["idx"][1], np.arange(CFG.top_k))
        np.testing.assert_array_equal(r.idx[1], np.arange(CFG.top_k))
        others = [t for t in range(CFG.tokens) if t != 1]
        assert np.isfinite(g["y"][others]).all()
        if mode == "act8":
            assert np.isnan(g["y"][1]).all() and np.isnan(r.y[1]).all()
