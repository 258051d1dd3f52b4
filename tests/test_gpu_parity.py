"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs (small shapes element by element, ragged tails, edge
cases; packing bit-exact)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from quantized_moe_decode_route_amd import ops, synth

from _parity import check_all, run_layer, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name: (T, H, I, E, G, TG, K, S, bits)
SHAPES = {
    "tiny": (1, 256, 128, 16, 4, 2, 4, 1, 4),
    "t1_h2048_q4": (1, 2048, 512, 32, 4, 2, 4, 1, 4),
    "t3_ragged_rows_s2": (3, 2048, 544, 64, 8, 3, 6, 2, 4),
    "t5_q8_noshared": (5, 1536, 320, 16, 2, 1, 2, 0, 8),
    "t16_q2": (16, 4096, 1024, 64, 8, 4, 8, 1, 2),
    "t2_glm_router_small_inter": (2, 6144, 256, 256, 8, 4, 8, 1, 4),
    "t4_top1_one_group": (4, 256, 128, 8, 1, 1, 1, 1, 4),
    "t64_max_tokens": (64, 512, 128, 64, 8, 4, 8, 1, 4),
    "t7_odd_groups_q4": (7, 2144, 96, 24, 3, 2, 5, 1, 4),
    "t1_q2_small": (1, 256, 128, 16, 4, 2, 4, 1, 2),
    "t2_q8_small": (2, 256, 128, 16, 4, 2, 4, 1, 8),
    # group sizes the selection's lane butterfly cannot take (LDS fallback)
    "t2_group_of_3": (2, 256, 128, 12, 4, 2, 3, 1, 4),
    "t1_e100": (1, 512, 128, 100, 4, 2, 6, 1, 4),
    # more tokens than LDS holds at H = 6144: tokens staged per segment
    "t8_h6144_segments": (8, 6144, 256, 64, 8, 4, 8, 1, 4),
    # one token (the fused call writes the batch union from the routing wave):
    # no shared expert; a single routed expert and two shared ones
    "t1_noshared": (1, 512, 256, 32, 4, 2, 6, 0, 4),
    "t1_top1_two_shared": (1, 768, 256, 24, 3, 1, 1, 2, 8),
}


def _cfg(name, seed=11):
    T, H, I, E, G, TG, K, S, b = SHAPES[name]
    return synth.MoEConfig(name, T, H, I, E, G, TG, K, S, b, seed=seed)


def _fits_fused(name):
    T, H, I, E, G, TG, K, S, b = SHAPES[name]
    return T <= ops.FUSED_MAX_TOKENS and E <= ops.FUSED_MAX_EXPERTS


# every shape through the separate calls; those within its limits also through the fused call
CASES = [(n, False) for n in SHAPES] + [(n, True) for n in SHAPES if _fits_fused(n)]


@pytest.mark.parametrize("name,fused", CASES, ids=[f"{n}-{'fused' if f else 'split'}" for n, f in CASES])
def test_layer_matches_oracle(name, fused):
    cfg = _cfg(name)
    say(f"case {name} {'fused' if fused else 'split'}: {SHAPES[name]}")
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens)
    g = run_layer(cfg, lay, x, fused=fused)
    rw, b = synth.router_weight(cfg, 0), synth.router_bias(cfg, 0)
    check_all(cfg, g, x, rw, b, synth.expert_loader(cfg, 0))


@pytest.mark.parametrize("fused", [False, True], ids=["split", "fused"])
def test_repeat_runs_are_bit_identical(fused):
    cfg = _cfg("t3_ragged_rows_s2", seed=5)
    lay = synth.layer_device(cfg, 0, DEV)
    x = synth.token_pool(cfg, cfg.tokens)
    a = run_layer(cfg, lay, x, fused=fused)
    b = run_layer(cfg, lay, x, fused=fused)
    for k in ("scores", "idx", "w", "h", "y"):
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("fused", [False, True], ids=["split", "fused"])
def test_all_tied_router(fused):
    """x = 0 and zero bias: every score is exactly 0.5; the lowest groups and
    indices are chosen and every weight is rsf / K exactly."""
    cfg = _cfg("tiny")
    lay = synth.layer_device(cfg, 0, DEV)
    lay["bias"].zero_()
    x = np.zeros((3, cfg.hidden), np.float32)
    g = run_layer(synth.scaled(cfg, tokens=3), lay, x, fused=fused)
    assert np.all(g["scores"] == 0.5)
    assert g["idx"].tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(g["w"] == np.float32(2.5 / 4))
    assert g["expert_id"].tolist() == [0, 1, 2, 3, 16]


@pytest.mark.parametrize("fused", [False, True], ids=["split", "fused"])
def test_one_hot_expert_closed_form(fused):
    """K = 1, one group, +10 bias on one expert, zero shared down-scales, a
    one-hot token: the output is the closed form of that single expert.

    The split calls carry activations as an f16 hi/lo pair (about 22 bits):
    within 1e-5 of the largest output.  The fused call carries them as 24-bit
    integers with a power-of-two scale per column, and its integer products
    are exact, so its error is what rounding the weighted h (2.5 h) to that
    grid allows: at most half a step, max|2.5 h| / 8323072, per element,
    times the row's sum of |code| * scale, plus fp32 rounding of the rest."""
    cfg = synth.MoEConfig("onehot", 1, 256, 128, 16, 1, 1, 1, 1, 4, seed=3)
    lay = synth.layer_device(cfg, 0, DEV)
    lay["bias"].zero_()
    lay["bias"][9] = 10.0
    lay["s_down"][16].zero_()
    x = np.zeros((1, 256), np.float32)
    x[0, 77] = 1.25
    g = run_layer(cfg, lay, x, fused=fused)
    assert g["idx"].tolist() == [[9]]
    d = synth.expert_arrays(cfg, 0, 9)
    qg = orc.unpack_rows(d["q_gate"], 4)[:, 77].astype(np.float64)
    qu = orc.unpack_rows(d["q_up"], 4)[:, 77].astype(np.float64)
    qd = orc.unpack_rows(d["q_down"], 4).astype(np.float64)
    gi = 1.25 * d["s_gate"].astype(np.float64) * qg
    ui = 1.25 * d["s_up"].astype(np.float64) * qu
    hv = gi / (1 + np.exp(-gi)) * ui
    sd = d["s_down"].astype(np.float64)
    want = 2.5 * sd * (qd @ hv)
    err = np.abs(g["y"][0] - want).max() / np.abs(want).max()
    say(f"  one-hot closed form err {err:.2e}")
    if not fused:
        assert err <= 1e-5
        return
    m = 2.5 * np.abs(hv).max()
    bound = sd * (np.abs(qd) @ np.ones_like(hv)) * m * (1.0 / 8323072 + 2e-6)
    worst = (np.abs(g["y"][0] - want) / bound).max()
    say(f"  fused: largest error / bound {worst:.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("rows,n", [(1, 64), (37, 1024), (5, 6144), (0, 32)])
def test_pack_unpack_bit_exact(bits, rows, n):
    rng = np.random.default_rng(bits * 1000 + rows)
    lo, hi = orc.code_range(bits)
    codes = rng.integers(lo, hi + 1, size=(rows, n)).astype(np.int8)
    ct = torch.from_numpy(codes).to(DEV)
    packed = ops.pack(ct, bits)
    want = orc.pack_rows(codes, bits) if rows else np.zeros((0, n * bits // 8), np.uint8)
    np.testing.assert_array_equal(packed.cpu().numpy(), want)
    back = ops.unpack(packed, bits)
    np.testing.assert_array_equal(back.cpu().numpy(), codes)


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_unpack_every_byte(bits):
    b = np.arange(256, dtype=np.uint8).reshape(4, 64)
    got = ops.unpack(torch.from_numpy(b).to(DEV), bits).cpu().numpy()
    np.testing.assert_array_equal(got, orc.unpack_rows(b, bits))


@pytest.mark.parametrize("T,H,offset", [(1, 4, 0), (3, 2048, 0), (16, 6144, 0), (2, 16384, 0), (4, 1000, 0),
                                         (2, 6143, 0), (3, 512, 1)])
def test_residual_rmsnorm_shapes(T, H, offset):
    """Every launch shape of the norm: float4 rows of 1-16 float4 per thread,
    odd row lengths and misaligned rows (the scalar kernel)."""
    rng = np.random.default_rng(H + T)
    x = rng.standard_normal((T, H)).astype(np.float32)
    y = (rng.standard_normal((T, H)) * 3).astype(np.float32)
    bx = torch.zeros(T * H + offset, device=DEV)
    by = torch.zeros(T * H + offset, device=DEV)
    xt, yt = bx[offset:].view(T, H), by[offset:].view(T, H)
    xt.copy_(torch.from_numpy(x))
    yt.copy_(torch.from_numpy(y))
    xn = torch.empty((T, H), device=DEV)
    ops.residual_rmsnorm(xt, yt, xn)
    np.testing.assert_array_equal(xt.cpu().numpy(), x + y)
    assert np.abs(xn.cpu().numpy() - orc.rmsnorm(x.astype(np.float64) + y)).max() <= 1e-5


def test_residual_rmsnorm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 6144)).astype(np.float32)
    y = rng.standard_normal((5, 6144)).astype(np.float32) * 40
    xt, yt = torch.from_numpy(x).to(DEV), torch.from_numpy(y).to(DEV)
    xn = torch.empty_like(xt)
    ops.residual_rmsnorm(xt, yt, xn)
    s = x.astype(np.float64) + y
    np.testing.assert_allclose(xt.cpu().numpy(), (x + y), rtol=0, atol=0)
    assert np.abs(xn.cpu().numpy() - orc.rmsnorm(s)).max() <= 1e-5
    ops.residual_rmsnorm(xt, None, xn)
    assert np.abs(xn.cpu().numpy() - orc.rmsnorm(s)).max() <= 1e-5


def test_generator_device_form_matches_host():
    """The code bytes the GPU tests and the benchmark generate on the device
    are the ones the oracle regenerates on the host."""
    cfg = synth.CONFIGS["glm_t1"]
    keys = [synth.stream_key(cfg.seed, 0, synth.K_GATE, e, cfg.bits) for e in (0, 255, 256)]
    dev = synth.splitmix_bytes_torch(keys, 4096, DEV).cpu().numpy()
    for i, k in enumerate(keys):
        np.testing.assert_array_equal(dev[i], synth.splitmix_bytes(k, 4096))
