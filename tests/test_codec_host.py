"""The library's MXFP8 codec helpers (csrc/common.h: the e4m3 rounding and the
E8M0 scale rule every quantising kernel uses) compiled for the host and run on
the CPU against the oracle's quantiser, which is pinned by the format tests:

* every e4m3 grid value and every midpoint between neighbouring codes, each
  +-16 fp32 ulps, both signs (ties to even, the subnormal range, the
  saturation band 448..512);
* 200k random fp32 values below 512;
* the scale of every positive bf16 block maximum, and of fp32 maxima across
  the subnormal range, 2^n - ulp, 2^n and 1.75 * 2^n;
* whole adversarial blocks (all zero, subnormal, with elements that scale to
  448 / 464 / 480 and to midpoints).

The OCP MX v1.0 rules the two sides follow are restated in the oracle."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "codec_host.cpp")
HDR = os.path.join(os.path.dirname(HERE), "fp4_routed_expert_amd", "csrc", "common.h")
SO = os.path.join(HERE, "native", "_build", "libcodec_host.so")


@pytest.fixture(scope="module")
def codec():
    newest = max(os.path.getmtime(SRC), os.path.getmtime(HDR))
    if not os.path.exists(SO) or os.path.getmtime(SO) < newest:
        os.makedirs(os.path.dirname(SO), exist_ok=True)
        subprocess.check_call(["/opt/rocm/bin/hipcc", "-O2", "-fPIC", "-shared", "-x", "hip",
                               "--offload-host-only", SRC, "-o", SO + ".tmp"])
        os.replace(SO + ".tmp", SO)
    lib = ctypes.CDLL(SO)
    p, i64 = ctypes.c_void_p, ctypes.c_long
    lib.host_f32_to_e4m3.argtypes = [p, i64, p]
    lib.host_mx_scale.argtypes = [p, i64, p, p]
    lib.host_quant_block32.argtypes = [p, p, p]
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _e4m3(lib, a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.size, dtype=np.uint8)
    lib.host_f32_to_e4m3(_ptr(a), a.size, _ptr(out))
    return out


def _oracle_codes(a):
    return np.array([oracle.e4m3_rne_sat(float(v)) for v in a], dtype=np.uint8)


def _around(values, ulps=16):
    v = np.asarray(values, dtype=np.float32)
    out = [v]
    up, dn = v.copy(), v.copy()
    for _ in range(ulps):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        out += [up.copy(), dn.copy()]
    return np.concatenate(out)


def test_e4m3_rounding_at_every_grid_value_and_midpoint(codec):
    grid = np.array([oracle.e4m3(c) for c in range(0x7F)], dtype=np.float64)  # 0 .. 448
    mids = (grid[:-1] + grid[1:]) / 2
    assert np.array_equal(mids.astype(np.float32).astype(np.float64), mids)  # exact in fp32
    sat = np.array([448.0, 456.0, 464.0, 472.0, 480.0, 496.0, 511.0], dtype=np.float32)
    a = _around(np.concatenate([grid, mids, sat]).astype(np.float32))
    a = a[(a >= 0) & (a < 512)]
    a = np.concatenate([a, -a])
    got = _e4m3(codec, a)
    want = _oracle_codes(a)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(a[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]
    # the ties themselves go to the even code
    tie = _e4m3(codec, mids.astype(np.float32))
    assert ((tie & 1) == 0).all()


def test_e4m3_rounding_random(codec):
    rng = np.random.default_rng(7)
    a = np.concatenate([rng.uniform(0, 512, 100_000), 2.0 ** rng.uniform(-12, 9, 100_000)])
    a = a.astype(np.float32)
    a = np.where(rng.random(a.size) < 0.5, -a, a).astype(np.float32)
    got = _e4m3(codec, a)
    want = _oracle_codes(a)
    assert np.array_equal(got, want)


def _oracle_scale(amax: float) -> int:
    v = np.zeros(32)
    v[0] = amax
    return oracle.quant_block32(v)[1]


def test_scale_rule_every_bf16_maximum_and_fp32_edges(codec):
    bf = (np.arange(0x0000, 0x7F80, dtype=np.uint32) << 16).view(np.float32)   # 0 .. bf16 max
    edges = []
    for n in range(-149, 128):
        p = np.float32(2.0 ** n)
        edges += [p, np.nextafter(p, np.float32(0)), np.float32(1.75) * p if n < 127 else p]
    f32 = np.array(edges, dtype=np.float32)
    amax = np.concatenate([bf, f32[np.isfinite(f32)]])
    code = np.empty(amax.size, dtype=np.uint8)
    mul = np.empty(amax.size, dtype=np.float32)
    codec.host_mx_scale(_ptr(amax), amax.size, _ptr(code), _ptr(mul))
    want = np.array([_oracle_scale(float(v)) for v in amax], dtype=np.uint8)
    assert np.array_equal(code, want)
    assert np.array_equal(mul.astype(np.float64), 2.0 ** (127 - code.astype(np.float64)))


def _adversarial_blocks(rng):
    blocks = [np.zeros(32), -np.zeros(32)]
    blocks.append(np.array([2.0 ** -149 * (i + 1) * (-1) ** i for i in range(32)]))   # fp32 subnormals
    blocks.append(np.array([2.0 ** -133 * (i % 7) for i in range(32)]))               # bf16 subnormals
    for n in (-20, -1, 0, 3, 15):
        base = 2.0 ** n
        for lead in (base * (1 - 2.0 ** -24), base, 1.75 * base, 1.875 * base, 1.9375 * base):
            b = rng.normal(0, base / 4, 32)
            b[rng.integers(32)] = lead
            blocks.append(b)
        # elements that land on 448, 464, 480 and on midpoints after scaling (scale 2^(n-8))
        unit = 2.0 ** (n - 8)
        b = np.array([448, 464, 480, 500, 511, 1.0625, 0.5 * 2.0 ** -6, 2.0 ** -10, 3 * 2.0 ** -10,
                      17, 18, 19, 36, 38, 272, 288, 304, 320, 240, 248, 0, -448, -464, -480, -17,
                      -19, -2.0 ** -10, -2.0 ** -11, 100, 104, 108, 1.0], dtype=np.float64) * unit
        b[0] = 1.5 * 2.0 ** n   # the maximum sets the scale 2^(n - 8)
        blocks.append(b)
    return [np.asarray(b, dtype=np.float32) for b in blocks]


def test_whole_blocks(codec):
    rng = np.random.default_rng(3)
    for b in _adversarial_blocks(rng) + [rng.normal(0, s, 32).astype(np.float32) for s in (1e-30, 1.0, 1e30)]:
        q = np.empty(32, dtype=np.uint8)
        s = np.empty(1, dtype=np.uint8)
        codec.host_quant_block32(_ptr(b), _ptr(q), _ptr(s))
        wq, ws = oracle.quant_block32(b.astype(np.float64))
        assert int(s[0]) == ws and np.array_equal(q, wq), b
