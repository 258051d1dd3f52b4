"""Pins of the oracle's Q8_0-style int8 activations (a variant of the layer in
which the activations meeting the weights are quantised per block and the
dot products are integer sums).

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
the integer-dot kernel item (Q8_0-style int8 activations).  The block length
and the rounding rule are readings (Q8_0's block of 32 consecutive values;
the row quantiser's absmax / 127 rule): these tests pin the oracle to them
with lossless inputs, the per-block error bound, block independence, and
the layer's reduction to the exact layer when x is representable.
"""
import numpy as np
import pytest

from oracle import moe_oracle as orc


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_block_lengths(bits):
    assert orc.act8_block(bits) == 32


@pytest.mark.parametrize("block", [32, 64, 128])
def test_representable_values_are_kept(block):
    """Values q * 2^-5 with a block's largest |q| = 127 quantise losslessly."""
    rng = np.random.default_rng(block)
    q = rng.integers(-127, 128, size=(3, 4 * block))
    for b in range(4):
        q[:, b * block + rng.integers(0, block)] = rng.choice([-127, 127])
    v = (q * 2.0 ** -5).astype(np.float32)
    np.testing.assert_array_equal(orc.quantize_act8(v, block), v.astype(np.float64))


@pytest.mark.parametrize("block", [32, 64, 128])
def test_error_bound_and_block_independence(block):
    """Every element within half a step of its block's scale (absmax / 127),
    each block on its own scale: a block of tiny values next to a block of
    huge ones keeps its relative precision."""
    rng = np.random.default_rng(7 + block)
    v = rng.standard_normal((5, 6 * block)).astype(np.float32)
    v[:, :block] *= np.float32(1e-6)
    v[:, block:2 * block] *= np.float32(1e4)
    got = orc.quantize_act8(v, block)
    for b in range(6):
        blk = v[:, b * block:(b + 1) * block].astype(np.float64)
        step = np.abs(blk).max(axis=1, keepdims=True) / 127.0
        err = np.abs(got[:, b * block:(b + 1) * block] - blk)
        assert np.all(err <= 0.5 * step * (1 + 1e-6) + 1e-300)


def _layer(rng, H, I, E, bits):
    lo, hi = orc.code_range(bits)
    experts = {}
    for e in range(E + 1):
        experts[e] = {k: orc.pack_rows(rng.integers(lo, hi + 1, size=shp), bits)
                      for k, shp in (("q_gate", (I, H)), ("q_up", (I, H)), ("q_down", (H, I)))}
        experts[e].update({"s_gate": rng.uniform(0.005, 0.02, I), "s_up": rng.uniform(0.005, 0.02, I),
                           "s_down": rng.uniform(0.005, 0.02, H)})
    rw = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    return experts, rw, b


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_layer_with_representable_x_keeps_h(bits):
    """When every block of x is representable, the int8-activation layer's h is
    the exact layer's h bit for bit (only the down input is quantised then)."""
    rng = np.random.default_rng(11 + bits)
    blk = orc.act8_block(bits)
    H, I, E = 2 * blk, blk, 8
    experts, rw, b = _layer(rng, H, I, E, bits)
    q = rng.integers(-127, 128, size=(2, H))
    q[:, 0] = 127
    q[:, blk] = -127
    x = (q * 2.0 ** -6).astype(np.float32)
    kw = dict(n_group=2, topk_group=1, top_k=2, n_shared=1, rsf=2.5, bits=bits)
    r8 = orc.moe_layer(x, rw, b, experts.__getitem__, act8=True, **kw)
    r = orc.moe_layer(x, rw, b, experts.__getitem__, **kw)
    np.testing.assert_array_equal(r8.idx, r.idx)
    np.testing.assert_array_equal(r8.h, r.h)
    rel = np.abs(r8.y - r.y).max() / np.abs(r.y).max()
    assert 0 < rel < 2e-2                       # down input quantised: close, not equal


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_layer_error_is_bounded_by_the_blocks(bits):
    """The int8-activation layer against the exact one on random x: the
    difference of each output row is at most what the per-block steps allow,
    propagated through |W| (first order, with a margin)."""
    rng = np.random.default_rng(19 + bits)
    blk = orc.act8_block(bits)
    H, I, E = 2 * blk, blk, 8
    experts, rw, b = _layer(rng, H, I, E, bits)
    x = rng.standard_normal((3, H)).astype(np.float32)
    kw = dict(n_group=2, topk_group=1, top_k=2, n_shared=1, rsf=2.5, bits=bits)
    r8 = orc.moe_layer(x, rw, b, experts.__getitem__, act8=True, **kw)
    r = orc.moe_layer(x, rw, b, experts.__getitem__, **kw)
    np.testing.assert_array_equal(r8.idx, r.idx)
    dx = np.abs(orc.quantize_act8(x, blk) - x.astype(np.float64)).max()
    assert dx > 0
    # the relative change of y stays within a few block steps (1/254 each)
    rel = np.abs(r8.y - r.y).max() / np.abs(r.y).max()
    assert rel < 8 / 254
