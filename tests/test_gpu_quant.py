"""GPU parity of the row quantiser (moe_quantize_rows_q*, moe_quantize_pack_rows_q*)
against the oracle: codes, packed bytes and scales bit-exact.

Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented features":
the converter requantises dequantised weights into the container with one
scale per row.  Shapes cover every launch shape of the kernel (one, two or
four waves per row, 1 to 8 float4 per lane, and the two-pass path for rows
over 8192 columns), ragged row counts (spare waves in the last workgroup), the edge rows
(zeros, NaN, infinities, subnormals, scales that underflow, exact ties) and a
whole GLM-5.2-sized expert matrix.
"""
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc
from quantized_moe_decode_route_amd import ops, synth

from _parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
QMAX = {8: 127, 4: 7, 2: 1}
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(w: np.ndarray, bits: int, pack: bool):
    wd = torch.from_numpy(np.ascontiguousarray(w)).to(DEV)
    out, s = ops.quantize_rows(wd, bits, pack=pack)
    torch.cuda.synchronize()
    return out.cpu().numpy(), s.cpu().numpy()


def _check(w: np.ndarray, bits: int, pack: bool, tag: str):
    say(f"[quant] {tag} rows={w.shape[0]} n={w.shape[1]} bits={bits} pack={pack}")
    got, gs = _run(w, bits, pack)
    q, s = orc.quantize_rows(w, bits)
    want = orc.pack_rows(q, bits) if pack else q
    assert np.array_equal(got, want), f"{tag}: {int((got != want).sum())} codes differ"
    same = (gs.view(np.uint32) == s.view(np.uint32)) | (np.isnan(gs) & np.isnan(s))
    assert same.all(), f"{tag}: scales differ at rows {np.nonzero(~same)[0][:8]}"


def _edge_rows(bits: int, n: int, rng) -> np.ndarray:
    """Zero, negative-zero, NaN, +-inf, subnormal, underflowing-scale and exact-tie rows."""
    qm = QMAX[bits]
    rows = []
    rows.append(np.zeros(n, np.float32))
    rows.append(np.full(n, -0.0, np.float32))
    r = rng.standard_normal(n).astype(np.float32); r[n // 2] = np.nan; rows.append(r)
    r = rng.standard_normal(n).astype(np.float32); r[-1] = np.inf; rows.append(r)
    r = rng.standard_normal(n).astype(np.float32); r[0] = -np.inf; rows.append(r)
    sub = np.float32(2.0 ** -149)
    rows.append((rng.integers(-9, 10, n) * sub).astype(np.float32))           # subnormal values
    r = np.zeros(n, np.float32); r[3] = 3 * sub; rows.append(r)               # s underflows for qmax > 3
    # exact ties: (k + 1/2) * 2^-6 with an anchor at qmax * 2^-6, so w / s = k + 1/2 exactly
    k = rng.integers(-qm, qm, n).astype(np.float64)
    r = ((k + 0.5) * 2.0 ** -6).astype(np.float32); r[1] = qm * 2.0 ** -6; rows.append(r)
    # the largest finite magnitude
    r = rng.standard_normal(n).astype(np.float32); r[2] = np.float32(3.4028235e38); rows.append(r)
    return np.stack(rows)


def test_golden_rows_on_gpu():
    with open(os.path.join(GOLDEN, "quantize_rows.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    num = lambda t: float.fromhex(t) if "0x" in t else float(t)
    for line in lines:
        bits, vals, codes, scale = (p.strip() for p in line.split("|"))
        w = np.array([[num(v) for v in vals.split(",")]], np.float32)
        got, gs = _run(w, int(bits), False)
        assert got[0].tolist() == [int(c) for c in codes.split(",")], line
        want = np.float32(num(scale))
        assert (np.isnan(gs[0]) and np.isnan(want)) or gs[0].view(np.uint32) == want.view(np.uint32) or \
            (gs[0] == 0 and want == 0), line


# (rows, n): n spans every launch shape of the kernel: one wave per row with 1, 2, 4 or 8 float4 per
# lane (n <= 256, 512, 1024, 2048), two waves (n <= 3072, 4096), four waves (n <= 6144, 8192), and the
# two-pass path for longer rows; row counts that leave spare waves in the last workgroup
SHAPES = [(1, 4), (5, 12), (37, 512), (9, 516), (21, 2048), (6, 2052), (11, 4096), (5, 6000), (13, 6144),
          (3, 8192), (7, 8196), (2, 20000)]


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("pack", [False, True])
@pytest.mark.parametrize("rows,n", SHAPES)
def test_random_rows(rows, n, bits, pack):
    w = synth.float_weight_rows(100 + rows, rows, n)
    _check(w, bits, pack, f"random {rows}x{n}")


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("n", [8, 2048, 6144, 10000])
def test_edge_rows(bits, n):
    rng = np.random.default_rng(n + bits)
    w = _edge_rows(bits, n, rng)
    for pack in (False, True):
        _check(w, bits, pack, f"edge n={n}")


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_near_half_quotients(bits):
    """Rows whose w / s falls within a few ulps of k + 1/2 for a scale that is
    not a power of two: the codes hinge on the correctly rounded quotient, so
    any shortcut to it must give way there."""
    rng = np.random.default_rng(70 + bits)
    qm = QMAX[bits]
    rows = []
    for _ in range(64):
        anchor = np.float32(rng.uniform(0.01, 10.0))
        s = np.float32(anchor / np.float32(qm))
        k = rng.integers(-qm, qm, 2048).astype(np.float64)           # k + 1/2 in [-qm + 1/2, qm - 1/2]
        base = ((k + 0.5) * np.float64(s)).astype(np.float32)
        vals = (base.view(np.int32) + rng.integers(-3, 4, 2048).astype(np.int32)).view(np.float32)
        vals[rng.integers(0, 2048)] = anchor                         # the absmax, so s is as above
        rows.append(vals)
    for pack in (False, True):
        _check(np.stack(rows), bits, pack, "near-half")


def test_empty_and_zero_width():
    w = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    out, s = ops.quantize_rows(w, 4)
    assert out.shape == (0, 64) and s.shape == (0,)
    w = torch.empty((3, 0), dtype=torch.float32, device=DEV)
    s = torch.full((3,), 7.0, device=DEV)
    ops.quantize_rows(w, 4, scales=s)
    assert s.cpu().tolist() == [0.0, 0.0, 0.0]


def test_rejects_bad_arguments():
    w = torch.zeros((4, 10), dtype=torch.float32, device=DEV)           # row_len % 4 != 0
    with pytest.raises(ops.MoedecError):
        ops.quantize_rows(w, 4)
    flat = torch.zeros(4 * 64 + 1, dtype=torch.float32, device=DEV)
    w = flat[1:].view(4, 64)                                             # 4-byte, not 16-byte, aligned
    with pytest.raises(ops.MoedecError):
        ops.quantize_rows(w, 4)


@pytest.mark.parametrize("which", ["gate", "down"])
def test_full_size_expert_matrix(which):
    """One GLM-5.2 expert matrix (gate [2048, 6144] or down [6144, 2048]) as int4,
    packed, in the launch the quantiser's measurement times."""
    rows, n = (2048, 6144) if which == "gate" else (6144, 2048)
    w = synth.float_weight_rows(7, rows, n)
    _check(w, 4, True, f"glm expert {which}")
