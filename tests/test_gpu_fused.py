"""The single-launch layer call beyond plain parity: every launch adds exactly
one arrival per workgroup to the scores exchange's counters of the
workspace, and launches back to back on one workspace and HIP-graph replays
give the eager results bit for bit (every reduction in the kernel has a fixed
order, so equal inputs give equal bits; rows of h no token is assigned to
hold a marker, compared as bits too)."""
import numpy as np
import pytest
import torch

from quantized_moe_decode_route_amd import ops, synth

from _parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CFG = synth.MoEConfig("fused_reuse", 3, 2048, 544, 64, 8, 3, 6, 2, 4, seed=21)
KW = dict(n_group=CFG.n_group, topk_group=CFG.topk_group, top_k=CFG.top_k, rsf=CFG.rsf)


def _setup(n_layers):
    layers = [synth.layer_device(CFG, l, DEV) for l in range(n_layers)]
    experts = [ops.Experts.from_layer(l, CFG.n_experts, CFG.n_shared, CFG.bits) for l in layers]
    pool = torch.from_numpy(synth.token_pool(CFG)).to(DEV)
    return layers, experts, pool


def _buffers(ws=None):
    b = ops.LayerBuffers.allocate(CFG.tokens, CFG.hidden, CFG.inter, CFG.n_experts, CFG.top_k, CFG.n_shared, DEV)
    if ws is not None:
        b.workspace = ws
    return b


def _tokens(pool, i):
    T = CFG.tokens
    b = i % (pool.shape[0] // T)
    return pool[b * T:(b + 1) * T]


def _bits(a):
    return a.view(torch.int32) if a.dtype == torch.float32 else a


def _eager(layers, experts, pool, i):
    l = i % len(layers)
    buf = ops.moe_layer(_tokens(pool, i), layers[l]["router_w"], layers[l]["bias"], experts[l], fused=True, **KW)
    torch.cuda.synchronize()
    assert not buf.fused_error()
    return buf


def test_back_to_back_launches_share_a_workspace():
    layers, experts, pool = _setup(3)
    n = 24
    ref = [_eager(layers, experts, pool, i) for i in range(n)]
    ws = torch.zeros(ops.FUSED_WORKSPACE_INTS, dtype=torch.int32, device=DEV)
    bufs = [_buffers(ws) for _ in range(n)]
    for i in range(n):                      # no synchronisation between the launches
        l = i % len(layers)
        ops.moe_layer(_tokens(pool, i), layers[l]["router_w"], layers[l]["bias"], experts[l], buf=bufs[i],
                      fused=True, **KW)
    torch.cuda.synchronize()
    nwg = torch.cuda.get_device_properties(DEV).multi_processor_count
    count = ops.pipe_arrivals(ws)
    err = int(ws[ops.FUSED_WS_ERROR].item())
    say(f"  workspace after {n} launches: arrivals {count} ({nwg} workgroups), error {err}")
    assert count == n * nwg and err == 0
    for i in range(n):
        for a, b in ((bufs[i].y, ref[i].y), (bufs[i].h, ref[i].h), (bufs[i].route.scores, ref[i].route.scores),
                     (bufs[i].route.topk_idx, ref[i].route.topk_idx), (bufs[i].route.topk_w, ref[i].route.topk_w),
                     (bufs[i].route.worklist.assign, ref[i].route.worklist.assign)):
            assert torch.equal(_bits(a), _bits(b)), f"launch {i} differs from its eager run"


def test_graph_replays_match_eager():
    layers, experts, pool = _setup(1)
    n = 6
    ref = [_eager(layers, experts, pool, i) for i in range(n)]
    x_static = _tokens(pool, 0).clone()
    buf = _buffers()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):          # warm-up outside the graph
        ops.moe_layer(x_static, layers[0]["router_w"], layers[0]["bias"], experts[0], buf=buf, fused=True, **KW)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        ops.moe_layer(x_static, layers[0]["router_w"], layers[0]["bias"], experts[0], buf=buf, fused=True, **KW)
    scratch = torch.randn(256, 256, device=DEV)
    for i in range(n):
        x_static.copy_(_tokens(pool, i))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        scratch = scratch @ scratch.T / 256.0        # the program's own work between replays
        torch.cuda.synchronize()
        assert not buf.fused_error()
        for a, b in ((buf.y, ref[i].y), (buf.h, ref[i].h), (buf.route.topk_idx, ref[i].route.topk_idx)):
            assert torch.equal(_bits(a), _bits(b)), f"replay {i} differs from the eager run"
    nwg = torch.cuda.get_device_properties(DEV).multi_processor_count
    # the warm-up launch and n replays (capture runs nothing)
    assert ops.pipe_arrivals(buf.workspace) == (n + 1) * nwg

