"""Pins of the oracle's router logits and shared-expert layer (CPU only).

The router is pinned by an exact rational brute force on a tiny case (pure
Python fractions, no numpy matmul) and by a one-hot Wg whose logits are the
activations themselves; the shared-expert layer by invariants against the
already pinned routed layer: no shared expert changes nothing, an all-zero
shared expert changes nothing, and with one routed expert (k = 1, gate 1)
whose weights are also the shared ones the output doubles exactly."""
from fractions import Fraction

import numpy as np

import oracle
import synth


def _bf16_frac(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(m, 1 << 7)) * (Fraction(2) ** (e - 127))


def test_router_logits_exact_brute_force():
    rng = np.random.default_rng(3)
    T, H, E = 3, 8, 5
    x = synth.f32_to_bf16_bits(rng.normal(size=(T, H)).astype(np.float32))
    wg = synth.f32_to_bf16_bits((rng.normal(size=(E, H)) * 0.3).astype(np.float32))
    logit, absum = oracle.router_logits(x, wg)
    for t in range(T):
        for e in range(E):
            exact = sum(_bf16_frac(int(x[t, h])) * _bf16_frac(int(wg[e, h])) for h in range(H))
            a = sum(abs(_bf16_frac(int(x[t, h])) * _bf16_frac(int(wg[e, h]))) for h in range(H))
            assert logit[t, e] == float(exact), (t, e)   # 8 exact products: exact in fp64
            assert absum[t, e] == float(a), (t, e)
    assert logit.shape == (T, E)


def test_router_logits_one_hot_rows_give_the_activations():
    rng = np.random.default_rng(4)
    T, H, E = 6, 64, 16
    xf = rng.normal(size=(T, H)).astype(np.float32)
    x = synth.f32_to_bf16_bits(xf)
    wg = np.zeros((E, H), dtype=np.uint16)
    for e in range(E):
        wg[e, (5 * e + 3) % H] = 0x3F80                     # +1.0 in bf16
    logit, absum = oracle.router_logits(x, wg)
    xv = synth.bf16_bits_to_f32(x).astype(np.float64)
    cols = (5 * np.arange(E) + 3) % H
    assert np.array_equal(logit, xv[:, cols])
    assert np.array_equal(absum, np.abs(xv[:, cols]))


def _small(T=5, H=256, I=128, E=4, k=2, seed=61):
    sh = synth.Shape(T=T, H=H, I=I, E=E, k=k, seed=seed)
    return sh, synth.make_inputs(sh)


def test_shared_layer_without_shared_expert_is_the_routed_layer():
    sh, inp = _small()
    y0 = oracle.layer_tokens(inp)
    y1 = oracle.layer_tokens_shared(inp, inp.logits, None)
    assert np.array_equal(y0, y1)


def test_zero_shared_expert_adds_nothing():
    sh, inp = _small(seed=62)
    zero = [np.zeros_like(a) for a in synth.make_shared_weights(sh)]
    y0 = oracle.layer_tokens(inp)
    y1 = oracle.layer_tokens_shared(inp, inp.logits, zero)
    assert np.array_equal(y0, y1)


def test_shared_copy_of_the_only_routed_expert_doubles_the_output():
    sh, inp = _small(T=6, E=1, k=1, seed=63)
    y0 = oracle.layer_tokens(inp)
    shared = (inp.w1, inp.s1, inp.w3, inp.s3, inp.w2, inp.s2)
    y1 = oracle.layer_tokens_shared(inp, inp.logits, shared)
    assert np.array_equal(y1, 2 * y0)                     # g = 1; y = O + O exactly
    # a shared expert with other weights does not double it
    other = synth.make_shared_weights(sh)
    y2 = oracle.layer_tokens_shared(inp, inp.logits, other)
    assert not np.array_equal(y2, 2 * y0)


def test_shared_expert_with_its_own_intermediate_size():
    sh, inp = _small(seed=64)
    sw = synth.make_shared_weights(sh, I_shared=256)
    y = oracle.layer_tokens_shared(inp, inp.logits, sw, tokens=np.array([0, 3], dtype=np.int32))
    y_r = oracle.layer_tokens(inp, np.array([0, 3], dtype=np.int32))
    # the shared part, rebuilt from the pinned single-expert steps
    xq, xs = oracle.quant_mxfp8_bf16(inp.x[[0, 3]])
    for n in range(2):
        G, U = oracle.expert_gate_up(xq[n], xs[n], sw[0][0], sw[1][0], sw[2][0], sw[3][0])
        _, hq, hs = oracle.swiglu_requant(G, U)
        Os = oracle.expert_down(hq, hs, sw[4][0], sw[5][0])
        assert np.allclose(y[n], y_r[n].astype(np.float64) + Os, rtol=1e-6, atol=1e-6 * np.abs(y[n]).max())
