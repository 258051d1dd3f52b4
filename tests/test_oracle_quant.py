"""Pins of the oracle's row quantiser (fp32 rows -> codes + one fp32 scale per row).

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
the offline converter requantises dequantised weights into the engine's
container, whose quantisation kernels keep one scale per row (int8, packed
int4, packed int2).  The rule itself is a reading (absmax / qmax, round half
to even): these tests pin the oracle to that reading with hand-worked rows, an
exact round trip, the nearest-code property over the whole code alphabet, and
symmetries that any slip in sign, rounding direction, axis or qmax breaks.
"""
import os

import numpy as np
import pytest

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
QMAX = {8: 127, 4: 7, 2: 1}


def _num(tok: str) -> float:
    tok = tok.strip()
    return float.fromhex(tok) if "0x" in tok else float(tok)


def _golden():
    rows = []
    with open(os.path.join(GOLDEN, "quantize_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            bits, vals, codes, scale = (p.strip() for p in line.split("|"))
            rows.append((int(bits), [_num(v) for v in vals.split(",")], [int(c) for c in codes.split(",")],
                         _num(scale)))
    return rows


def _same_f32(a, b) -> bool:
    a, b = np.float32(a), np.float32(b)
    if np.isnan(a) or np.isnan(b):
        return bool(np.isnan(a) and np.isnan(b))
    return a.tobytes() == b.tobytes() or (a == 0 and b == 0)


@pytest.mark.parametrize("bits,vals,codes,scale", _golden())
def test_golden_rows(bits, vals, codes, scale):
    q, s = orc.quantize_rows(np.array([vals], np.float32), bits)
    assert q.tolist() == [codes]
    assert _same_f32(s[0], scale), (s[0], scale)


def _exact_code_rows(rng, bits, rows, n):
    """Codes with +-qmax in every row and scales whose products with any code
    are exact in fp32 (16-bit mantissas), so w = q * s holds exactly."""
    qm = QMAX[bits]
    q = rng.integers(-qm, qm + 1, size=(rows, n))
    pos = rng.integers(0, n, size=rows)
    q[np.arange(rows), pos] = rng.choice([-qm, qm], size=rows)
    mant = rng.integers(1 << 15, 1 << 16, size=rows).astype(np.float64)
    expo = rng.integers(-40, 10, size=rows)
    s = (mant * np.exp2(expo - 16.0)).astype(np.float32)
    return q.astype(np.int8), s


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_exact_code_rows_round_trip(bits):
    rng = np.random.default_rng(20 + bits)
    q, s = _exact_code_rows(rng, bits, 64, 96)
    w = (q.astype(np.float64) * s.astype(np.float64)[:, None]).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), q.astype(np.float64) * s.astype(np.float64)[:, None])
    q2, s2 = orc.quantize_rows(w, bits)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, s)


def _rows(rng, rows, n):
    w = rng.standard_normal((rows, n)).astype(np.float32)
    w[::3] *= np.float32(0.01)                                   # small rows
    w[1::5] = rng.standard_cauchy((len(w[1::5]), n)).astype(np.float32)  # heavy tails
    return w


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_nearest_code_over_the_alphabet(bits):
    """Each code is the nearest one (ties to even) to the exact w / s among all
    codes of the field; only a ratio within one fp32 ulp of a half-way point
    may go to either neighbour (the fp32 division decides it)."""
    rng = np.random.default_rng(30 + bits)
    w = _rows(rng, 48, 64)
    q, s = orc.quantize_rows(w, bits)
    lo, hi = orc.code_range(bits)
    alphabet = np.arange(lo, hi + 1, dtype=np.float64)
    for r in range(w.shape[0]):
        sr = float(s[r])
        assert sr > 0
        ratio = w[r].astype(np.float64) / sr                         # exact ratio (to fp64)
        dist = np.abs(ratio[:, None] - alphabet[None, :])
        best = dist.min(axis=1)
        for j in range(w.shape[1]):
            cand = alphabet[dist[j] == best[j]]
            if len(cand) == 2:                                        # exact tie: the even code
                cand = cand[cand % 2 == 0]
            frac = abs(ratio[j] - np.floor(ratio[j]) - 0.5)
            near_half = frac <= 2.0 * np.spacing(np.float32(abs(ratio[j]) + 1.0))
            assert q[r, j] in cand or near_half, (r, j, ratio[j], q[r, j])


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_range_absmax_and_error_bound(bits):
    rng = np.random.default_rng(40 + bits)
    w = _rows(rng, 48, 80)
    q, s = orc.quantize_rows(w, bits)
    qm = QMAX[bits]
    assert np.all(np.abs(q.astype(np.int32)) <= qm)
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == qm)    # the absmax element maps to +-qmax
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= 0.5 * s.astype(np.float64)[:, None] * (1 + 1e-6))
    # the scale is absmax / qmax to within fp32 rounding
    am = np.abs(w.astype(np.float64)).max(axis=1)
    assert np.allclose(s.astype(np.float64), am / qm, rtol=2 ** -23, atol=0)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_sign_and_power_of_two_symmetry(bits):
    rng = np.random.default_rng(50 + bits)
    w = _rows(rng, 32, 64)
    q, s = orc.quantize_rows(w, bits)
    qn, sn = orc.quantize_rows(-w, bits)
    assert np.array_equal(qn.astype(np.int32), -q.astype(np.int32))
    assert np.array_equal(sn, s)
    for k in (-12, 5):
        qk, sk = orc.quantize_rows(w * np.float32(2.0 ** k), bits)
        assert np.array_equal(qk, q)
        assert np.array_equal(sk, s * np.float32(2.0 ** k))


def test_rows_are_independent_and_codes_pack():
    rng = np.random.default_rng(60)
    w = _rows(rng, 12, 32)
    w[4, 7] = np.nan
    w[9] = 0.0
    for bits in (8, 4, 2):
        q, s = orc.quantize_rows(w, bits)
        for r in range(w.shape[0]):
            qr, sr = orc.quantize_rows(w[r:r + 1], bits)
            assert np.array_equal(qr[0], q[r]) and _same_f32(sr[0], s[r])
        assert np.isnan(s[4]) and not q[4].any()
        assert s[9] == 0 and not q[9].any()
        back = orc.unpack_rows(orc.pack_rows(q, bits), bits)
        assert np.array_equal(back, q)
