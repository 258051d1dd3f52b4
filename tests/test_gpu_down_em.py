"""GPU parity of the expert-major down + combine (moe_expert_down_combine_em_q*)
against the oracle and against the row-split down on the same h.

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
dequant-on-use kernels and the batch-union item (each selected expert's rows
are read once for every token routed to it).  The expert-major form stages
only the streamed expert's assignments and adds the per-assignment partial
outputs per token afterwards; shapes cover one to 64 tokens, all code
widths, a batch with and without a shared expert, and top-p's dropped slots.
"""
import numpy as np
import pytest
import torch

from quantized_moe_decode_route_amd import ops, synth

from oracle import moe_oracle as orc

from _parity import check_all, rel_err, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name: (T, H, I, E, G, TG, K, S, bits)
SHAPES = {
    "t1_q4": (1, 512, 256, 16, 4, 2, 4, 1, 4),
    "t3_ragged_rows_s2": (3, 2048, 544, 64, 8, 3, 6, 2, 4),
    "t5_q8_noshared": (5, 1536, 320, 16, 2, 1, 2, 0, 8),
    "t16_q2": (16, 4096, 1024, 64, 8, 4, 8, 1, 2),
    "t16_q4": (16, 2048, 512, 64, 8, 4, 8, 1, 4),
    "t64_max_tokens": (64, 512, 128, 64, 8, 4, 8, 1, 4),
}


def _cfg(name, seed=41):
    T, H, I, E, G, TG, K, S, b = SHAPES[name]
    return synth.MoEConfig(name, T, H, I, E, G, TG, K, S, b, seed=seed)


def _run(cfg, lay, x, top_p=None):
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    ex = ops.Experts.from_layer(lay, cfg.n_experts, cfg.n_shared, cfg.bits)
    kw = dict(n_group=cfg.n_group, topk_group=cfg.topk_group, top_k=cfg.top_k, rsf=cfg.rsf)
    r = ops.route_topk(xt, lay["router_w"], lay["bias"], n_shared=cfg.n_shared, top_p=top_p, **kw)
    h = ops.gate_up_silu(xt, ex, r.worklist, cfg.top_k)
    part = torch.empty((cfg.tokens * cfg.slots, cfg.hidden), device=DEV)
    y_em = ops.down_combine(h, ex, r.worklist, r.topk_w, cfg.top_k, part=part, topk_idx=r.topk_idx)
    y_rs = ops.down_combine(h, ex, r.worklist, r.topk_w, cfg.top_k)
    torch.cuda.synchronize()
    wl = r.worklist
    n = int(wl.n_active.item())
    seg = wl.seg[:n + 1].cpu().numpy()
    g = dict(scores=r.scores.cpu().numpy(), idx=r.topk_idx.cpu().numpy(), w=r.topk_w.cpu().numpy(), n_active=n,
             expert_id=wl.expert_id[:n].cpu().numpy(), seg=seg, assign=wl.assign[:int(seg[-1])].cpu().numpy(),
             h=h.cpu().numpy(), y=y_em.cpu().numpy(), top_p=top_p)
    return g, y_rs.cpu().numpy()


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("top_p", [None, 0.7])
def test_down_em_matches_oracle_and_row_split(name, top_p):
    cfg = _cfg(name)
    say(f"case {name} down expert-major top_p={top_p}: {SHAPES[name]}")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens)
    g, y_rs = _run(cfg, lay, x, top_p)
    e = rel_err(g["y"], y_rs)
    say(f"  expert-major vs row-split on the same h: {e:.2e}")
    assert e <= 2e-6                    # fp32 sums in another order on the same staged values
    check_all(cfg, g, x, synth.router_weight(cfg, 0), synth.router_bias(cfg, 0), synth.expert_loader(cfg, 0))


def test_down_em_repeat_is_bit_identical():
    cfg = _cfg("t16_q4", seed=43)
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens)
    a, _ = _run(cfg, lay, x)
    b, _ = _run(cfg, lay, x)
    np.testing.assert_array_equal(a["y"], b["y"])


def _tie_values(w: np.float32, n: int, rng) -> np.ndarray:
    """n fp32 values v whose fp32 product with w lands on an f16 tie (at its
    own binade) while the exact product lies on the side that rounding the
    exact product straight to f16 resolves the other way."""
    out = []
    while len(out) < n:
        v = rng.uniform(0.5, 4.0, 1 << 20).astype(np.float32) * rng.choice([-1, 1], 1 << 20).astype(np.float32)
        x32 = v * w                                          # fp32 product, RNE
        p = v.astype(np.float64) * np.float64(w)             # exact
        # scale every value into f16's normal range at the same binade offset
        e = np.frexp(x32)[1]
        xs = np.ldexp(x32.astype(np.float64), 14 - e)        # |xs| in [2^13, 2^14)
        ps = np.ldexp(p, 14 - e)
        two = xs.astype(np.float16).astype(np.float64) != ps.astype(np.float16).astype(np.float64)
        out.extend(v[two][: n - len(out)].tolist())
    return np.asarray(out, np.float32)


@pytest.mark.parametrize("em", [False, True], ids=["row_split", "expert_major"])
def test_f16_split_of_products_on_ties(em):
    """h times its routing weight is staged as an f16 hi + lo pair; a product
    whose fp32 rounding sits on an f16 tie must still give hi + lo = the fp32
    product (regression: the pair was built from two different roundings)."""
    T, H, I, E, G, TG, K, S, b = (4, 256, 128, 16, 4, 2, 4, 1, 4)
    cfg = synth.MoEConfig("ties", T, H, I, E, G, TG, K, S, b, seed=47)
    lay = synth.layer_device(cfg, 0, DEV)
    ex = ops.Experts.from_layer(lay, E, S, b)
    x = torch.from_numpy(synth.token_pool(cfg, T)).to(DEV)
    r = ops.route_topk(x, lay["router_w"], lay["bias"], n_shared=S, n_group=G, topk_group=TG, top_k=K, rsf=cfg.rsf)
    rng = np.random.default_rng(5)
    w = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    slots = K + S
    h = np.zeros((T * slots, I), np.float32)
    for t in range(T):
        for s in range(K):
            h[t * slots + s] = _tie_values(w[t, s], I, rng)
        h[t * slots + K] = rng.uniform(-2, 2, I).astype(np.float32)
    ht, wt = torch.from_numpy(h).to(DEV), torch.from_numpy(w).to(DEV)
    part = torch.empty((T * slots, H), device=DEV) if em else None
    y = ops.down_combine(ht, ex, r.worklist, wt, K, part=part, topk_idx=r.topk_idx if em else None).cpu().numpy()
    idx = r.topk_idx.cpu().numpy()
    ld = synth.expert_loader(cfg, 0)
    ref = np.zeros((T, H))
    for t in range(T):
        for s in range(slots):
            e = int(idx[t, s]) if s < K else E + (s - K)
            hv = (h[t * slots + s] * (w[t, s] if s < K else np.float32(1))).astype(np.float64)   # fp32 products
            a = ld(e)
            ref[t] += orc.dequantize(a["q_down"], a["s_down"], b) @ hv
    err = rel_err(y, ref)
    say(f"  {'expert-major' if em else 'row-split'} on tie products: err {err:.2e}")
    assert err <= 2e-6
