"""Every launch shape of the split router against the oracle.

The router GEMV runs in tiles of expert rows x tokens (1x1, 1x2, 1x4, 2x4,
4x4, and 2x4 for rows longer than 8192 at more than 8 tokens), each thread
taking one float4 column per sweep of 512 (1, 2, 3, 4 or 8 sweeps, the last
one ragged); expert counts of 72 leave the last tile of eight short and 1024
puts 16 experts on a lane.  Selection runs one workgroup per token, and the
workgroup that arrives last builds the batch union.  Scores, selections and
the worklist are checked as in every layer test (tests/_parity.py): scores
within 2e-6 of the oracle's fp64 sigmoid, sets and orders where the
oracle's margins certify them, the worklist bit-exact.  Each case runs the
same buffers twice, so the arrival count must start from zero each call.
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from quantized_moe_decode_route_amd import ops

from _parity import check_routing, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (T, H, E, n_group, topk_group, top_k, n_shared)
CASES = [
    (1, 6144, 256, 8, 4, 8, 1),      # 1x1 tile, 3 full sweeps
    (2, 4096, 256, 8, 4, 8, 1),      # 1x2, 2 full sweeps
    (3, 4100, 72, 8, 2, 6, 2),       # 1x4 with a clamped token, a 1-column third sweep, short last tile
    (4, 12, 64, 4, 2, 4, 0),         # 1x4, a tiny row
    (6, 8192, 256, 8, 4, 8, 1),      # 2x4, 4 full sweeps
    (8, 16384, 256, 8, 4, 8, 1),     # 2x4, 8 sweeps
    (9, 8196, 256, 8, 4, 8, 1),      # 2x4 at 8 sweeps for 5 (rows past 8192), ragged tokens
    (12, 7168, 256, 8, 4, 8, 1),     # 4x4 at 4 sweeps, the last one half full
    (16, 6144, 256, 8, 4, 8, 1),     # 4x4, 3 sweeps: the stack's shape
    (16, 16384, 1024, 8, 4, 8, 2),   # 2x4 at 8 sweeps, 16 experts per lane
    (33, 2048, 72, 4, 2, 5, 1),      # 4x4 with ragged token and expert tiles
    (64, 6144, 256, 8, 4, 8, 1),     # the most tokens: 16 token tiles, 64 selection workgroups
]


@pytest.mark.parametrize("T,H,E,G,TG,K,S", CASES)
def test_router_launch_shapes(T, H, E, G, TG, K, S):
    say(f"router T={T} H={H} E={E} G={G} TG={TG} K={K} S={S}")
    rng = np.random.default_rng(T * 100003 + H * 7 + E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32)
    cfg = SimpleNamespace(n_group=G, topk_group=TG, top_k=K, n_shared=S, rsf=2.5, n_experts=E)
    s64 = orc.router_scores(x, w)
    idx, wts = orc.select_experts(s64.astype(np.float32), bias, G, TG, K, cfg.rsf)
    r = orc.LayerResult(s64, idx, wts, orc.batch_union(idx, E, S), None, None,
                        orc.selection_margin(s64, bias, G, TG, K), orc.order_margin(s64, bias, idx),
                        np.full(T, np.inf))
    xt, wt, bt = (torch.from_numpy(a).to(DEV) for a in (x, w, bias))
    out = None
    for call in range(2):
        out = ops.route_topk(xt, wt, bt, n_group=G, topk_group=TG, top_k=K, n_shared=S, rsf=cfg.rsf, out=out)
        torch.cuda.synchronize()
        wl = out.worklist
        n = int(wl.n_active.item())
        seg = wl.seg[:n + 1].cpu().numpy()
        g = dict(scores=out.scores.cpu().numpy(), idx=out.topk_idx.cpu().numpy(), w=out.topk_w.cpu().numpy(),
                 n_active=n, expert_id=wl.expert_id[:n].cpu().numpy(), seg=seg,
                 assign=wl.assign[:int(seg[-1])].cpu().numpy(), top_p=None)
        set_ok, _ = check_routing(cfg, g, r, bias)
        assert set_ok.any()
