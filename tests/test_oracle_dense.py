"""Pins of the oracle's FP8 dense projection (CPU only).

* exact rational brute force on a tiny case (pure Python fractions over the
  e4m3 / E8M0 definitions, no library matmul);
* a one-hot weight (code 0x38 = 1.0, scale 2^0) returns decoded activations;
* one more E8M0 step on every weight scale doubles y exactly;
* weights whose e4m3 codes are the e2m1 values give, with the same scales,
  exactly what the already pinned FP4 down projection gives for the nibbles.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

# unit roundoff of each oracle build (round to nearest)
UNIT = {"fp32": Fraction(1, 2 ** 24), "fp64": Fraction(1, 2 ** 53)}


def gamma(n: int, u: Fraction) -> Fraction:
    """The classic bound of recursive summation: |fl(sum a_i) - sum a_i| <=
    gamma_(n-1) * sum |a_i|, gamma_n = n u / (1 - n u) (Higham, Accuracy and
    Stability of Numerical Algorithms, section 4.2)."""
    return n * u / (1 - n * u)


def _e4m3_frac(b: int) -> Fraction:
    sign = -1 if b & 0x80 else 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _e8m0_frac(c: int) -> Fraction:
    return Fraction(2) ** (c - 127)


@pytest.mark.parametrize("prec", ["fp32", "fp64"])
def test_dense_exact_brute_force(prec):
    """Each product of two scaled e4m3 values is exact, so the only error is the
    summation's: within gamma_(K-1) * sum |products| of the exact rational sum."""
    inp = synth.make_dense_inputs("d0", T=3, K=64, N=5)
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    with oracle.using(prec):
        y = oracle.dense_fp8(xq, xs, inp.wq, inp.ws)
    assert y.shape == (3, 5)
    for t in range(3):
        for n in range(5):
            prods = [_e4m3_frac(int(xq[t, k])) * _e8m0_frac(int(xs[t, k // 32]))
                     * _e4m3_frac(int(inp.wq[n, k])) * _e8m0_frac(int(inp.ws[n, k // 32]))
                     for k in range(64)]
            exact = sum(prods)
            bound = gamma(63, UNIT[prec]) * sum(abs(v) for v in prods)
            assert abs(Fraction(y[t, n]) - exact) <= bound, (t, n)


def test_dense_one_hot_weights_give_the_activations():
    inp = synth.make_dense_inputs("d0")
    T, K, N = inp.x.shape[0], inp.x.shape[1], inp.wq.shape[0]
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    wq = np.zeros((N, K), dtype=np.uint8)
    cols = (11 * np.arange(N) + 5) % K
    wq[np.arange(N), cols] = 0x38                     # +1.0 in e4m3
    ws = np.full((N, K // 32), 127, dtype=np.uint8)   # 2^0
    y = oracle.dense_fp8(xq, xs, wq, ws)
    xd = oracle.decode_mxfp8(xq, xs)
    assert np.array_equal(y, xd[:, cols].astype(np.float64))


def test_dense_scale_step_doubles_exactly():
    inp = synth.make_dense_inputs("d0")
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    y = oracle.dense_fp8(xq, xs, inp.wq, inp.ws)
    y2 = oracle.dense_fp8(xq, xs, inp.wq, (inp.ws + 1).astype(np.uint8))
    assert np.array_equal(y2, 2 * y)
    assert np.abs(y).max() > 0


# e2m1 code -> the e4m3 code of the same value
_E2M1_AS_E4M3 = [0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C]


def test_dense_equals_fp4_down_projection_on_e2m1_values():
    rng = np.random.default_rng(9)
    N, K = 48, 256
    nib = rng.integers(0, 16, size=(N, K))
    w2 = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)    # even K in the low nibble
    wq = np.array([_E2M1_AS_E4M3[v & 7] | ((v & 8) << 4) for v in nib.ravel()],
                  dtype=np.uint8).reshape(N, K)
    ws = rng.integers(118, 126, size=(N, K // 32)).astype(np.uint8)
    inp = synth.make_dense_inputs("d0", T=4, K=K, N=N)
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    y = oracle.dense_fp8(xq, xs, wq, ws)
    for t in range(4):
        O = oracle.expert_down(xq[t], xs[t], w2, ws)
        np.testing.assert_allclose(y[t], O, rtol=1e-13, atol=1e-13 * np.abs(O).max())
    # a transposed weight must not pass
    y_bad = oracle.dense_fp8(xq, xs, wq[::-1].copy(), ws[::-1].copy())
    assert not np.allclose(y_bad, y)
