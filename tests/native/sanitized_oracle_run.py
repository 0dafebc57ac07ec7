"""Run by tests/test_sanitizers.py in a child process whose environment
preloads the gcc AddressSanitizer and UBSan runtimes: the oracle and the input
generator, built with -fsanitize=address,undefined, on small workloads that
reach every entry point.  Exits non-zero on the first sanitizer report."""
import os
import sys

ROOT = sys.argv[1]
BUILD = sys.argv[2]
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

oracle._SOS["fp32"] = os.path.join(BUILD, "liboracle_san.so")
oracle._SOS["fp64"] = os.path.join(BUILD, "liboracle_f64_san.so")
synth._SO = os.path.join(BUILD, "libsynth_san.so")

for prec in ("fp32", "fp64"):
    with oracle.using(prec):
        assert oracle.precision() == prec
        for shape, probe in ((synth.CONFIGS["c0"], False), (synth.Shape(T=5, H=384, I=640, E=5, k=3, seed=7), True)):
            inp = synth.make_inputs(shape, probe_w2=probe)
            sh = inp.shape
            y, h, hq, hs = oracle.layer_tokens(inp, want_pairs=True)
            ex, h2, hq2, hs2, O = oracle.layer_pairs(inp, np.arange(sh.T * sh.k, dtype=np.int32)[::-1].copy())
            ids, gates = oracle.route(inp.logits, sh.k)
            counts, offsets, sp, pp = oracle.sort(ids, sh.E)
            xq, xs = oracle.quant_mxfp8_bf16(inp.x)
            oracle.decode_mxfp8(xq, xs)
            oracle.decode_fp4_matrix(inp.w1[0], inp.s1[0])
            G, U = oracle.expert_gate_up(xq[0], xs[0], inp.w1[0], inp.s1[0], inp.w3[0], inp.s3[0])
            oracle.swiglu_requant(G, U)
            sw = synth.make_shared_weights(sh)
            wg = synth.make_router_weights(sh)
            lg, ab = oracle.router_logits(inp.x, wg)
            oracle.layer_tokens_shared(inp, lg.astype(np.float32), sw)
            oracle.layer_tokens_shared(inp, inp.logits, None)
        dn = synth.make_dense_inputs("d0")
        dq, ds = oracle.quant_mxfp8_bf16(dn.x)
        oracle.dense_fp8(dq, ds, dn.wq, dn.ws)
        oracle.quant_mxfp8_f32(np.array([[0.0] * 32 + [1e-40] * 32], dtype=np.float32))
        for b in range(256):
            oracle.e4m3(b)
        for v in (0.0, -0.0, 1e-30, 447.9, 448.0, 1e9, -3.0):
            oracle.e4m3_rne_sat(v)
        synth.zipf_bias(4, 256, 1.2)
        synth.f32_to_bf16_bits(np.array([1.0, -2.5, 3e38], dtype=np.float32))
print("sanitized oracle run ok")
