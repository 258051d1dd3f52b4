"""Pins of the oracle's code packing (int8 / packed int4 / packed int2).

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features",
quantisation-kernel item, and the ideipro.ru article (packing verified bit for
bit): the checks here are exhaustive round trips plus hand-worked bytes.
"""
import itertools
import os

import numpy as np
import pytest

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_pack():
    rows = []
    with open(os.path.join(GOLDEN, "pack_bytes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            bits, codes, packed = (p.strip() for p in line.split("|"))
            rows.append((int(bits), [int(c) for c in codes.split(",")],
                         [int(b, 16) for b in packed.split()]))
    return rows


@pytest.mark.parametrize("bits,codes,packed", _golden_pack())
def test_pack_golden_bytes(bits, codes, packed):
    got = orc.pack_rows(np.array([codes]), bits)
    assert got.tolist() == [packed]
    back = orc.unpack_rows(np.array([packed], np.uint8), bits)
    assert back.tolist() == [codes]


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_every_byte_round_trips(bits):
    """unpack then pack gives back each of the 256 byte values."""
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes = orc.unpack_rows(b, bits)
    lo, hi = orc.code_range(bits)
    assert codes.min() >= lo and codes.max() <= hi
    assert np.array_equal(orc.pack_rows(codes, bits), b)


@pytest.mark.parametrize("bits", [4, 2])
def test_every_code_tuple_round_trips(bits):
    """pack then unpack gives back every tuple of codes that fills one byte."""
    per = 8 // bits
    lo, hi = orc.code_range(bits)
    tuples = np.array(list(itertools.product(range(lo, hi + 1), repeat=per)))
    assert len(tuples) == 256
    packed = orc.pack_rows(tuples, bits)           # one byte per tuple (row)
    assert packed.shape == (256, 1)
    assert sorted(packed[:, 0].tolist()) == list(range(256))   # a bijection
    assert np.array_equal(orc.unpack_rows(packed, bits), tuples)


def test_int8_is_plain_twos_complement():
    """int8 codes are the bytes themselves read as signed: numpy's own view."""
    b = np.arange(256, dtype=np.uint8).reshape(2, 128)
    assert np.array_equal(orc.unpack_rows(b, 8), b.view(np.int8))


def test_int4_byte_formula():
    """byte j = (q[2j] & 0xF) | ((q[2j+1] & 0xF) << 4), on random rows."""
    g = np.random.default_rng(7)
    q = g.integers(-8, 8, size=(5, 64))
    packed = orc.pack_rows(q, 4).astype(np.int64)
    want = (q[:, 0::2] & 0xF) | ((q[:, 1::2] & 0xF) << 4)
    assert np.array_equal(packed, want)


def test_pack_rejects_out_of_range():
    with pytest.raises(AssertionError):
        orc.pack_rows(np.array([[8, 0]]), 4)
    with pytest.raises(AssertionError):
        orc.pack_rows(np.array([[-3, 0, 0, 0]]), 2)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_dequantize_is_code_times_row_scale(bits):
    g = np.random.default_rng(bits)
    lo, hi = orc.code_range(bits)
    q = g.integers(lo, hi + 1, size=(6, 32))
    s = g.uniform(0.005, 0.02, size=6).astype(np.float32)
    w = orc.dequantize(orc.pack_rows(q, bits), s, bits)
    for r in range(6):
        for c in range(32):
            assert w[r, c] == float(q[r, c]) * float(s[r])
