"""The no-allocation down call (moe_expert_down_combine_em_noalloc_q4)
against the expert-major down call with a caller buffer: bit for bit on two
calls in a row, the second smaller than the first (the static array keeps the
first call's rows, which the second must not read), and the size limit.

The no-allocation call is for callers that cannot allocate device memory (HIP
graph capture, serving loops); it runs the same kernels as the buffered call
with its partial outputs in the library's static per-GPU array.
"""
import ctypes

import numpy as np
import pytest
import torch

from quantized_moe_decode_route_amd import ops, synth

from _parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(T, H, I, E, seed):
    cfg = synth.MoEConfig(f"noalloc_t{T}", T, H, I, E, 8, 4, 8, 1, 4, seed=seed)
    lay = synth.layer_device(cfg, 0, DEV)
    ex = ops.Experts.from_layer(lay, cfg.n_experts, cfg.n_shared, cfg.bits)
    x = torch.from_numpy(np.ascontiguousarray(synth.token_pool(cfg)[:T], np.float32)).to(DEV)
    kw = dict(n_group=cfg.n_group, topk_group=cfg.topk_group, top_k=cfg.top_k, rsf=cfg.rsf)
    r = ops.route_topk(x, lay["router_w"], lay["bias"], n_shared=cfg.n_shared, **kw)
    h = ops.gate_up_silu(x, ex, r.worklist, cfg.top_k)
    return cfg, ex, r, h


def _both(cfg, ex, r, h):
    part = torch.empty((cfg.tokens * cfg.slots, cfg.hidden), device=DEV)
    y_ref = ops.down_combine(h, ex, r.worklist, r.topk_w, cfg.top_k, part=part, topk_idx=r.topk_idx)
    y = torch.full((cfg.tokens, cfg.hidden), float("nan"), device=DEV)
    ops.down_combine_noalloc(h, ex, r.worklist, r.topk_w, cfg.top_k, out=y, topk_idx=r.topk_idx)
    torch.cuda.synchronize()
    return y, y_ref


def test_noalloc_matches_buffered_twice_then_smaller():
    # 16 tokens x 9 slots x 6144 = 884,736 floats of the 2^20 (the 16-token GLM-sized batch), then 3 tokens
    for T, H, I, E, seed in ((16, 6144, 512, 64, 71), (3, 2048, 256, 32, 72)):
        cfg, ex, r, h = _case(T, H, I, E, seed)
        y, y_ref = _both(cfg, ex, r, h)
        say(f"  T={T} H={H}: max |diff| {float((y - y_ref).abs().max()):.3g}")
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), f"T={T}: differs from the buffered call"


def test_noalloc_rejects_more_than_its_array():
    cfg, ex, r, h = _case(16, 8192, 256, 32, 73)          # 16 x 9 x 8192 = 1,179,648 floats > 2^20
    y = torch.empty((cfg.tokens, cfg.hidden), device=DEV)
    with pytest.raises(ops.MoedecError) as err:
        ops.down_combine_noalloc(h, ex, r.worklist, r.topk_w, cfg.top_k, out=y, topk_idx=r.topk_idx)
    assert err.value.status == ops.MOEDEC_ERR_UNSUPPORTED
