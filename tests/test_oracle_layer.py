"""Pins of the oracle's expert FFN and whole layer.

The layer is the FP4 routed-expert computation whose down-projection (W2)
layout had to be repaired at load time after the fast path produced an output
permutation ("DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and
Inference Performance Engineering", abstract).  Pins:

* a hand-worked two-token layer whose outputs are exact closed forms;
* an identity-structured W2 probe whose output is a closed form of h, with
  negative controls (a permuted W2 must fail the probe);
* the projections against a library float64 matmul of the decoded operands
  (the decoders are pinned by the format tests);
* a permutation-structured W1 (one non-zero per row) with a closed form;
* the dense formulation (all experts, zero gates off the top-k).
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _inputs(x_f32, logits, k, w1, s1, w3, s3, w2, s2):
    T, H = x_f32.shape
    E = logits.shape[1]
    I = w1.shape[1]
    sh = synth.Shape(T=T, H=H, I=I, E=E, k=k)
    return synth.LayerInputs(shape=sh, x=synth.f32_to_bf16_bits(x_f32), logits=logits.astype(np.float32),
                             w1=w1, s1=s1, w3=w3, s3=s3, w2=w2, s2=s2)


def _const_weights(E, rows, K, codes, scales):
    w = np.empty((E, rows, K // 2), dtype=np.uint8)
    s = np.empty((E, rows, K // 32), dtype=np.uint8)
    for e in range(E):
        w[e] = codes[e] | (codes[e] << 4)
        s[e] = scales[e]
    return w, s


@pytest.mark.parametrize("prec", ["fp32", "fp64"])
def test_hand_worked_layer(prec):
    """T=2, E=3, k=2, H=I=32 (exact in both oracle builds).

    x0 = 1.0 x32 -> MXFP8 scale 2^-8, bytes 0x78 (1.0 exactly).
    x1 = 2.0 x16, -1.0 x16 -> scale 2^-7, bytes 0x78 / 0xF0 (exact).
    e0: W1 = 1.0*2^-5, W3 = 3.0*2^-5; e1: W1 = -0.5*2^-4, W3 = 2.0*2^-4;
    e2: W1 = 1.5*2^-6, W3 = -4.0*2^-6; W2 = the identity probe.
    (t0,e0): G=1, U=3, h=3/(1+e^-1)=2.19318 -> scale 2^-7, 280.7 -> 288 (0x79) = 2.25
    (t0,e1): G=-1, U=4, h=-4/(1+e)=-1.07577 -> scale 2^-8, 275.4 -> 288 (0xF9) = -1.125
    (t1,e2): G=0.375, U=-1, h=-0.22225 -> scale 2^-11, 455.2 saturates (0xFE) = -0.21875
    (t1,e1): G=-0.5, U=2, h=-0.37754 -> scale 2^-10, 386.6 -> 384 (0xFC) = -0.375
    y0 = 0.5*2.25 + 0.5*(-1.125) = 0.5625;  y1 = 0.75*(-0.21875) + 0.25*(-0.375) = -0.2578125
    """
    H = I = 32
    x = np.zeros((2, H), dtype=np.float32)
    x[0] = 1.0
    x[1, :16] = 2.0
    x[1, 16:] = -1.0
    logits = np.array([[0.5, 0.5, -1.0], [-1.0, 0.0, math.log(3.0)]])
    w1, s1 = _const_weights(3, I, H, [0x2, 0x9, 0x3], [122, 123, 121])
    w3, s3 = _const_weights(3, I, H, [0x5, 0x4, 0xE], [122, 123, 121])
    w2, s2 = synth.w2_probe(3, H, I)
    inp = _inputs(x, logits, 2, w1, s1, w3, s3, w2, s2)
    with oracle.using(prec):
        assert oracle.precision() == prec
        y, h, hq, hs = oracle.layer_tokens(inp, want_pairs=True)
    # pair order (t, j): (0,e0) (0,e1) (1,e2) (1,e1)
    assert np.allclose(h[:, 0], [3 / (1 + math.exp(-1)), -4 / (1 + math.e),
                                 -0.375 / (1 + math.exp(-0.375)), -1 / (1 + math.exp(0.5))], rtol=1e-6)
    assert (h == h[:, :1]).all()
    assert hq[:, 0].tolist() == [0x79, 0xF9, 0xFE, 0xFC] and (hq == hq[:, :1]).all()
    assert hs[:, 0].tolist() == [120, 119, 116, 117]
    assert (y[0] == 0.5625).all()
    assert np.allclose(y[1], -0.2578125, rtol=0, atol=2e-7)


def _rand_expert(rng, H, I):
    w1 = rng.integers(0, 256, (I, H // 2), dtype=np.uint8)
    w3 = rng.integers(0, 256, (I, H // 2), dtype=np.uint8)
    w2 = rng.integers(0, 256, (H, I // 2), dtype=np.uint8)
    s1 = rng.integers(121, 126, (I, H // 32), dtype=np.uint8)
    s3 = rng.integers(121, 126, (I, H // 32), dtype=np.uint8)
    s2 = rng.integers(121, 126, (H, I // 32), dtype=np.uint8)
    return w1, s1, w3, s3, w2, s2


# unit roundoff of each oracle build (round to nearest)
UNIT = {"fp32": 2.0 ** -24, "fp64": 2.0 ** -53}


def _sum_bound(n, abs_sum, prec):
    """gamma_(n-1) * sum |a_i|: the error bound of recursive summation of n
    exactly representable terms (Higham, Accuracy and Stability of Numerical
    Algorithms, section 4.2), with a margin for the float64 evaluation of the
    library reference itself."""
    u = UNIT[prec]
    return (n - 1) * u / (1 - (n - 1) * u) * abs_sum + 2 * n * 2.0 ** -53 * abs_sum


@pytest.mark.parametrize("prec", ["fp32", "fp64"])
@pytest.mark.parametrize("H,I", [(256, 128), (128, 384)])
def test_projections_match_library_matmul(H, I, prec):
    """Every product of a decoded e4m3 and e2m1 value is exact, so each
    projection is within the summation bound of a library float64 matmul of
    the decoded operands; SwiGLU matches its closed form in the build's
    precision; h's bytes are the pinned quantiser's."""
    rng = np.random.default_rng(H + I)
    w1, s1, w3, s3, w2, s2 = _rand_expert(rng, H, I)
    xq, xs = oracle.quant_mxfp8_f32(rng.normal(0, 1, (1, H)).astype(np.float32))
    with oracle.using(prec):
        G, U = oracle.expert_gate_up(xq[0], xs[0], w1, s1, w3, s3)
        xd = oracle.decode_mxfp8(xq, xs)[0]
        for got, (w, s) in ((G, (w1, s1)), (U, (w3, s3))):
            W = oracle.decode_fp4_matrix(w, s)
            assert (np.abs(got - W @ xd) <= _sum_bound(H, np.abs(W) @ np.abs(xd), prec)).all()
        h, hq, hs = oracle.swiglu_requant(G, U)
        if prec == "fp64":
            assert np.array_equal(h, (G / (1 + np.exp(-G)) * U).astype(np.float32))
        else:
            g32, u32 = G.astype(np.float32), U.astype(np.float32)
            want = (g32 / (np.float32(1) + np.exp(-g32)) * u32).astype(np.float32)
            # numpy's float32 exp and the C library's expf may differ in the last place
            assert np.allclose(h, want, rtol=4 * 2.0 ** -24, atol=0)
        q2, s2q = oracle.quant_mxfp8_f32(h[None, :])
        assert (q2[0] == hq).all() and (s2q[0] == hs).all()
        O = oracle.expert_down(hq, hs, w2, s2)
        hd = oracle.decode_mxfp8(hq[None, :], hs[None, :])[0]
        W2 = oracle.decode_fp4_matrix(w2, s2)
        assert (np.abs(O - W2 @ hd) <= _sum_bound(I, np.abs(W2) @ np.abs(hd), prec)).all()


def test_permutation_structured_w1_closed_form():
    """W1 with a single +1.0 per row at column pi(i): G[i] = x[pi(i)] exactly."""
    H, I = 256, 128
    rng = np.random.default_rng(11)
    pi = rng.permutation(H)[:I]
    w1 = np.zeros((I, H // 2), dtype=np.uint8)
    for i, c in enumerate(pi):
        w1[i, c // 2] |= 0x2 << (4 * (c & 1))
    s1 = np.full((I, H // 32), 127, dtype=np.uint8)
    w3 = w1.copy()
    s3 = np.full((I, H // 32), 128, dtype=np.uint8)  # W3 = 2 * W1
    xq, xs = oracle.quant_mxfp8_f32(rng.normal(0, 1, (1, H)).astype(np.float32))
    G, U = oracle.expert_gate_up(xq[0], xs[0], w1, s1, w3, s3)
    xd = [oracle.e4m3(int(xq[0, c])) * 2.0 ** (int(xs[0, c // 32]) - 127) for c in pi]
    assert G.tolist() == xd
    assert U.tolist() == [2 * v for v in xd]


def _probe_closed_form(inp, hq, hs):
    """y[t, r] = sum_j g_j * deq(hq_{t,j})[(r + e_j) mod I] for the identity W2."""
    sh = inp.shape
    ids, gates = oracle.route(inp.logits, sh.k)
    hd = oracle.decode_mxfp8(hq, hs)
    y = np.zeros((sh.T, sh.H))
    r = np.arange(sh.H)
    for t in range(sh.T):
        for j in range(sh.k):
            e = ids[t, j]
            y[t] += float(gates[t, j]) * hd[t * sh.k + j, (r + e) % sh.I]
    return y


def test_w2_probe_closed_form_c0():
    inp = synth.make_inputs("c0", probe_w2=True)
    y, h, hq, hs = oracle.layer_tokens(inp, want_pairs=True)
    assert np.allclose(y, _probe_closed_form(inp, hq, hs), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("mistake", ["swap_rows", "swap_k_in_block", "swap_nibbles", "transpose_expert"])
def test_w2_probe_negative_controls(mistake):
    """A W2 laid out wrongly must fail the probe (the bug class of the paper)."""
    inp = synth.make_inputs("c0", probe_w2=True)
    w2 = inp.w2.copy()
    if mistake == "swap_rows":
        w2[:, [3, 4]] = w2[:, [4, 3]]
    elif mistake == "swap_k_in_block":  # columns 2..3 <-> 4..5 of every row
        w2[:, :, [1, 2]] = w2[:, :, [2, 1]]
    elif mistake == "swap_nibbles":
        w2 = ((w2 >> 4) | (w2 << 4)).astype(np.uint8)
    elif mistake == "transpose_expert":
        w2 = w2[::-1].copy()
    inp.w2 = np.ascontiguousarray(w2)
    y, h, hq, hs = oracle.layer_tokens(inp, want_pairs=True)
    assert not np.allclose(y, _probe_closed_form(inp, hq, hs), rtol=1e-6, atol=1e-7)


def test_dense_formulation_c0():
    """y equals a sum over ALL experts with gate 0 off the top-k (numpy matmuls)."""
    inp = synth.make_inputs("c0")
    sh = inp.shape
    y = oracle.layer_tokens(inp)
    ids, gates = oracle.route(inp.logits, sh.k)
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    xd = oracle.decode_mxfp8(xq, xs)
    dense = np.zeros((sh.T, sh.H))
    for e in range(sh.E):
        G = xd @ oracle.decode_fp4_matrix(inp.w1[e], inp.s1[e]).T
        U = xd @ oracle.decode_fp4_matrix(inp.w3[e], inp.s3[e]).T
        h = (G / (1 + np.exp(-G)) * U).astype(np.float32)
        hq, hs = oracle.quant_mxfp8_f32(h)
        O = oracle.decode_mxfp8(hq, hs) @ oracle.decode_fp4_matrix(inp.w2[e], inp.s2[e]).T
        g = np.zeros(sh.T)
        for t in range(sh.T):
            for j in range(sh.k):
                if ids[t, j] == e:
                    g[t] = gates[t, j]
        dense += g[:, None] * O
    assert np.allclose(y, dense, rtol=1e-5, atol=1e-5 * np.abs(dense).max())


def test_single_expert_k1_is_one_ffn():
    inp = synth.make_inputs(synth.Shape(T=5, H=128, I=64, E=1, k=1, seed=9))
    y = oracle.layer_tokens(inp)
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    for t in range(5):
        G, U = oracle.expert_gate_up(xq[t], xs[t], inp.w1[0], inp.s1[0], inp.w3[0], inp.s3[0])
        _, hq, hs = oracle.swiglu_requant(G, U)
        O = oracle.expert_down(hq, hs, inp.w2[0], inp.s2[0])
        assert np.array_equal(y[t], O.astype(np.float32))


def test_token_rows_are_independent():
    """Computing a subset of tokens gives the same rows as the full layer."""
    inp = synth.make_inputs("c0")
    y = oracle.layer_tokens(inp)
    sub = np.array([13, 2, 7], dtype=np.int32)
    assert np.array_equal(oracle.layer_tokens(inp, sub), y[sub])


@pytest.mark.parametrize("name", ["c0", "c1"])
def test_fp32_build_within_its_rounding_of_fp64(name):
    """The fp32 oracle (the method's precision) against the fp64 diagnostic
    build on whole workloads: integer outputs identical, y within 1e-5 of
    max|y| -- a thousandth of the GPU tolerance (1e-2), so the choice of
    build cannot decide a parity test -- and h's bytes equal but for rare
    rounding flips of the requantisation."""
    inp = synth.make_inputs(name)
    y32, _, hq32, hs32 = oracle.layer_tokens(inp, want_pairs=True)
    with oracle.using("fp64"):
        y64, _, hq64, hs64 = oracle.layer_tokens(inp, want_pairs=True)
        ids64, gates64 = oracle.route(inp.logits, inp.shape.k)
    ids32, gates32 = oracle.route(inp.logits, inp.shape.k)
    assert np.array_equal(ids32, ids64)
    assert np.allclose(gates32, gates64, rtol=4 * 2.0 ** -24, atol=0)
    ratio = np.abs(y32.astype(np.float64) - y64).max() / np.abs(y64).max()
    assert ratio <= 1e-5, ratio
    assert (hq32 == hq64).mean() >= 0.9999 and (hs32 == hs64).mean() >= 0.999


def test_layer_pairs_equal_the_token_layer_c0():
    """The per-pair entry gives the token entry's h, hq, hs pair by pair (same
    steps), and the slot-order gate-weighted sum of its O rows is y."""
    inp = synth.make_inputs("c0")
    sh = inp.shape
    y, h, hq, hs = oracle.layer_tokens(inp, want_pairs=True)
    order = np.random.default_rng(5).permutation(sh.T * sh.k).astype(np.int32)
    ex, h2, hq2, hs2, O = oracle.layer_pairs(inp, order)
    ids, gates = oracle.route(inp.logits, sh.k)
    assert np.array_equal(ex, ids.reshape(-1)[order])
    assert np.array_equal(h2, h[order]) and np.array_equal(hq2, hq[order]) and np.array_equal(hs2, hs[order])
    Op = np.empty_like(O)
    Op[order] = O
    acc = np.zeros((sh.T, sh.H), dtype=np.float32)
    for j in range(sh.k):
        acc += gates[:, j:j + 1] * Op.reshape(sh.T, sh.k, sh.H)[:, j].astype(np.float32)
    assert np.array_equal(acc, y)


def test_layer_pairs_w2_probe_closed_form_and_negative_control():
    """Identity-structured W2: O[n, r] = deq(hq_n)[(r + e_n) mod I] exactly, a
    single non-zero product per output; a W2 with two rows swapped fails."""
    inp = synth.make_inputs("c0", probe_w2=True)
    sh = inp.shape
    pairs = np.arange(sh.T * sh.k, dtype=np.int32)
    ex, _, hq, hs, O = oracle.layer_pairs(inp, pairs)
    hd = oracle.decode_mxfp8(hq, hs)
    r = np.arange(sh.H)
    closed = np.stack([hd[n, (r + ex[n]) % sh.I] for n in range(pairs.size)])
    assert np.array_equal(O, closed)
    w2 = inp.w2.copy()
    w2[:, [3, 4]] = w2[:, [4, 3]]
    inp.w2 = np.ascontiguousarray(w2)
    _, _, hq2, hs2, O2 = oracle.layer_pairs(inp, pairs)
    hd2 = oracle.decode_mxfp8(hq2, hs2)
    closed2 = np.stack([hd2[n, (r + ex[n]) % sh.I] for n in range(pairs.size)])
    assert not np.array_equal(O2, closed2)
