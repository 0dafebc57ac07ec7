"""Seeded sweeps of shapes through both expert paths, against the oracle.

Layer: thirty shapes drawn once from a fixed seed (token counts 1..700, 1..300
experts, k up to 12, H and I of one to five 128-blocks, with and without a
Zipf popularity bias that leaves hot and empty experts): routing ids, the sort
and the quantised x bit-exact, y within the output tolerance on sampled
tokens, each through the weight-streaming and the MFMA path; the one-call
layer entry gives bitwise the chain's y.  Full layer (router GEMM + shared
experts): ten drawn shapes with 0-2 shared experts, the one-call entry
bitwise equal to the chain of stage calls and y against the oracle.  FP8
dense projection: ten drawn (T, K, N) through both of its paths, the
quantised x bit-exact and y against the oracle on every token."""
import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import oracle
import synth
from gpu_cases import check_y, get_case, log, sample_tokens
from test_gpu_dense import get_dense
from test_gpu_parity import PATHS, _run_layer
from test_gpu_router_shared import test_layer_full as _full_case

pytestmark = pytest.mark.gpu


def _shapes(n=30, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 7, 16, 33, 64, 100, 257, 300]))
        k = int(rng.integers(1, min(E, 12) + 1))
        T = int(rng.choice([1, 3, 17, 64, 129, 250, 411, 700]))
        H = 128 * int(rng.integers(1, 6))
        I = 128 * int(rng.integers(1, 4))
        zipf = float(rng.choice([0.0, 0.0, 1.1]))
        sigma = float(rng.choice([0.5, 1.0, 3.0]))
        out.append(synth.Shape(T=T, H=H, I=I, E=E, k=k, x_sigma=sigma, zipf_s=zipf, seed=500 + i))
    return out


SWEEP = _shapes()


@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("shape", SWEEP, ids=lambda s: f"T{s.T}H{s.H}I{s.I}E{s.E}k{s.k}z{s.zipf_s:g}")
def test_sweep(shape, path, dev):
    c = get_case(shape, dev)
    log(f"[sweep] {shape} {path}")
    y, it = _run_layer(c, PATHS[path])
    assert np.array_equal(it["topk_ids"].cpu().numpy(), c.ids)
    assert np.array_equal(it["expert_counts"].cpu().numpy(), c.counts)
    assert np.array_equal(it["sorted_pair"].cpu().numpy(), c.sorted_pair)
    assert np.array_equal(it["pair_pos"].cpu().numpy(), c.pair_pos)
    assert np.array_equal(it["xq"].cpu().numpy(), c.xq)
    assert np.array_equal(it["xs"].cpu().numpy(), c.xs)
    y_entry = moe.layer_forward(c.pw, c.x, c.logits, c.sh.k, PATHS[path])
    torch.cuda.synchronize()
    assert torch.equal(y_entry, y)
    toks = sample_tokens(c.sh.T, 32, seed=7)
    check_y(y.cpu().numpy()[toks], oracle.layer_tokens(c.inp, toks), f"sweep/{path}")


def _full_shapes(n=10, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([2, 8, 16, 64, 130]))
        k = int(rng.integers(1, min(E, 8) + 1))
        ns = int(rng.integers(0, 3))
        T = int(rng.choice([1, 5, 32, 33, 100, 300]))
        H = 128 * int(rng.integers(1, 5))
        I = 128 * int(rng.integers(1, 3))
        flags = int(rng.choice([0, moe.MOE_FLAG_FORCE_DECODE, moe.MOE_FLAG_FORCE_PREFILL]))
        out.append((synth.Shape(T=T, H=H, I=I, E=E, k=k, seed=700 + i), ns, flags))
    return out


FULL_SWEEP = _full_shapes()


@pytest.mark.parametrize("shape,ns,flags", FULL_SWEEP,
                         ids=[f"T{s.T}H{s.H}I{s.I}E{s.E}k{s.k}-ns{n}-f{f}" for s, n, f in FULL_SWEEP])
def test_sweep_full(shape, ns, flags, dev):
    _full_case(shape, ns, flags, 16, dev)


def _dense_shapes(n=10, seed=99):
    rng = np.random.default_rng(seed)
    return [dict(T=int(rng.choice([1, 7, 32, 33, 150, 257, 300])), K=128 * int(rng.integers(1, 9)),
                 N=32 * int(rng.integers(1, 33))) for _ in range(n)]


DENSE_SWEEP = _dense_shapes()


@pytest.mark.parametrize("flags", [moe.MOE_FLAG_FORCE_DECODE, moe.MOE_FLAG_FORCE_PREFILL], ids=["decode", "prefill"])
@pytest.mark.parametrize("over", DENSE_SWEEP, ids=[f"T{o['T']}K{o['K']}N{o['N']}" for o in DENSE_SWEEP])
def test_sweep_dense(over, flags, dev):
    c = get_dense("d0", dev, **over)
    log(f"[sweep dense] {over} flags={flags}")
    xq, xs = moe.quant_act_mxfp8(c.x)
    assert np.array_equal(xq.cpu().numpy(), c.xq) and np.array_equal(xs.cpu().numpy(), c.xs)
    y = moe.dense_forward(c.dw, xq, xs, flags)
    torch.cuda.synchronize()
    check_y(y.float().cpu().numpy(), c.ref(np.arange(c.sh.T, dtype=np.int32)), f"sweep/dense/{over}/f{flags}")
