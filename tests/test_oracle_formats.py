"""Pins of the oracle's element formats and MXFP8 quantiser.

The element formats are those of the OCP Microscaling (MX) v1.0 family; the
pages require the OCP FP8 dialect on MI355X (aijianwen.com MI300X log, FP8
section: fnuz and OCP share a bit layout but differ by one in exponent bias,
so a misread byte comes out twice or half as large) and an MXFP4 expert path
(same log, profiling section).  The pins below do not restate the oracle's
formulas: they use the spec's value tables, PyTorch's own float8_e4m3fn
conversion (a library routine), exact rational brute force, and invariants.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle

# OCP MX v1.0 FP4 E2M1 value table (magnitudes of codes 0..7).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_all_codes():
    for c in range(16):
        want = E2M1_TABLE[c & 7]
        got = oracle.e2m1(c)
        assert got == want * (-1 if c & 8 else 1)
        assert math.copysign(1.0, got) == (-1.0 if c & 8 else 1.0)  # -0 for code 8


def test_e8m0_key_codes_and_doubling():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(119) == 1.0 / 256
    assert oracle.e8m0(121) == 1.0 / 64 and oracle.e8m0(125) == 0.25  # the weight-scale range
    assert oracle.e8m0(0) == float.fromhex("0x1p-127")
    assert oracle.e8m0(254) == float.fromhex("0x1p127")
    assert math.isnan(oracle.e8m0(255))
    for c in range(254):
        assert oracle.e8m0(c + 1) == 2.0 * oracle.e8m0(c)


def test_e4m3_all_bytes_match_torch():
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double()
    for b in range(256):
        got = oracle.e4m3(b)
        want = float(lib[b])
        if b in (0x7F, 0xFF):
            assert math.isnan(got) and math.isnan(want)
        else:
            assert got == want, hex(b)
            assert math.copysign(1, got) == math.copysign(1, want)


def test_e4m3_key_codes():
    assert oracle.e4m3(0x38) == 1.0
    assert oracle.e4m3(0x78) == 256.0
    assert oracle.e4m3(0x7C) == 384.0
    assert oracle.e4m3(0x7E) == 448.0
    assert oracle.e4m3(0x08) == 2.0 ** -6
    assert oracle.e4m3(0x01) == 2.0 ** -9
    vals = [oracle.e4m3(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:])), "finite codes must increase"


def _grid():
    return [Fraction(oracle.e4m3(c)) for c in range(0x7F)]


def exact_rne_sat(a: Fraction) -> int:
    """Nearest e4m3 code by exhaustive rational search; ties -> even code; saturating."""
    sign = 0x80 if a < 0 else 0
    m = abs(a)
    grid = _GRID
    if m >= grid[-1]:
        return sign | 0x7E
    best = min(range(0x7F), key=lambda c: (abs(grid[c] - m), c & 1))
    return sign | best


_GRID = _grid()


def test_rne_sat_matches_torch_below_overflow():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.uniform(-463.9, 463.9, 20000),
        rng.normal(0, 1, 20000) * np.exp2(rng.integers(-12, 8, 20000)),
        # every midpoint between consecutive codes, and just either side of it
        *[(np.array(_GRID[1:], dtype=np.float64) + np.array(_GRID[:-1], dtype=np.float64)) / 2 + d
          for d in (0.0, 1e-9, -1e-9)],
    ]).astype(np.float32)
    vals = vals[np.abs(vals) < 464.0]
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_rne_sat(float(v)) for v in vals], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (vals[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_rne_sat_saturates_and_keeps_sign():
    for v in (448.0, 449.0, 464.0, 480.0, 511.9, 1e6):
        assert oracle.e4m3_rne_sat(v) == 0x7E
        assert oracle.e4m3_rne_sat(-v) == 0xFE
    assert oracle.e4m3_rne_sat(-0.0) == 0x80
    assert oracle.e4m3_rne_sat(-2.0 ** -12) == 0x80  # underflow keeps the sign
    assert oracle.e4m3_rne_sat(2.0 ** -11) == 0x00   # exactly 1/4 of the smallest step -> 0
    assert oracle.e4m3_rne_sat(2.0 ** -10) == 0x00   # tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_rne_sat(3 * 2.0 ** -10) == 0x02  # tie between codes 1 and 2 -> 2


def test_rne_sat_exact_rational_brute_force():
    rng = np.random.default_rng(1)
    cases = [Fraction(int(n), 1 << 20) for n in rng.integers(-(448 << 20), 448 << 20, 3000)]
    cases += [(_GRID[c] + _GRID[c + 1]) / 2 for c in range(0x7E)]  # all ties
    for a in cases:
        assert oracle.e4m3_rne_sat(float(a)) == exact_rne_sat(a), a


# Hand-worked MXFP8 blocks (32 elements, the unlisted ones 0).  Each row:
# (nonzero leading values, scale code, leading bytes).
#   {1.0}: floor(log2 1) - 8 = -8 -> code 119; 1.0 * 2^8 = 256 -> 0x78
#   {3.0}: floor(log2 3) = 1 -> X = -7 (code 120); 3 * 128 = 384 -> 0x7C
#   {-0.3, 3.0}: X = -7; -0.3 * 128 = -38.4, grid step 4 in [32,64) -> -40 = 0xE2
#   {1.0625}: X = -8; 272 lies half way between 256 and 288 -> even code 0x78
#   {1.0, 0.53125, 0.5703125}: X = -8; 136 ties 128/144 -> 128 (0x70); 146 -> 144 (0x71)
#   {1.99}: X = -8; 509.44 >= 448 -> saturates to 0x7E
#   {2^-140}: X clamped to -127 (code 0); 2^-140 * 2^127 = 2^-13 -> 0
HAND_BLOCKS = [
    ([1.0], 119, [0x78]),
    ([3.0], 120, [0x7C]),
    ([-0.3, 3.0], 120, [0xE2, 0x7C]),
    ([1.0625], 119, [0x78]),
    ([1.0, 0.53125, 0.5703125], 119, [0x78, 0x70, 0x71]),
    ([1.99], 119, [0x7E]),
    ([2.0 ** -140], 0, [0x00]),
    ([], 0, []),
]


@pytest.mark.parametrize("lead,scale,lead_bytes", HAND_BLOCKS)
def test_quant_block_hand_worked(lead, scale, lead_bytes):
    v = np.zeros(32)
    v[: len(lead)] = lead
    q, s = oracle.quant_block32(v)
    assert s == scale
    assert list(q[: len(lead_bytes)]) == lead_bytes
    assert not q[len(lead_bytes):].any()


def test_quant_scale_invariant_random_blocks():
    """OCP MX floor rule: the block maximum lands in [256, 512) after scaling."""
    rng = np.random.default_rng(2)
    for _ in range(2000):
        v = rng.normal(0, 1, 32) * 2.0 ** rng.integers(-30, 30)
        q, s = oracle.quant_block32(v)
        X = s - 127
        r = np.max(np.abs(v)) * 2.0 ** (-X)
        assert 256 <= r < 512
        deq = np.array([oracle.e4m3(b) for b in q])
        # below the saturation bound every element is within half a grid step:
        # steps are 2^(E-3) in the binade [2^E, 2^(E+1)) and 2^-9 under 2^-6
        for vi, di in zip(v * 2.0 ** (-X), deq):
            if abs(vi) < 448:
                assert abs(vi - di) <= max(abs(vi) * 2.0 ** -4, 2.0 ** -10)
            else:
                assert di == math.copysign(448.0, vi)


def test_quant_rows_match_blocks():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, (3, 128)).astype(np.float32)
    q, s = oracle.quant_mxfp8_f32(x)
    for r in range(3):
        for b in range(4):
            qb, sb = oracle.quant_block32(x[r, 32 * b: 32 * b + 32].astype(np.float64))
            assert (q[r, 32 * b: 32 * b + 32] == qb).all() and s[r, b] == sb


def test_bf16_decode_is_exact():
    assert oracle.bf16(0x3F80) == 1.0
    assert oracle.bf16(0xC000) == -2.0
    assert oracle.bf16(0x0001) == float.fromhex("0x1p-133")
