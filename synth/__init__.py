"""Seeded synthetic inputs for the FP4 routed-expert MoE layer.

Shared by the CPU oracle's tests and by the GPU path's tests and benchmark.
Holds no arithmetic of the layer itself: it draws random numbers (see
``synth.c``) and returns numpy arrays in the layer's input storage formats:

* ``x``       bf16 bit patterns, uint16 ``[T, H]``
* ``logits``  float32 ``[T, E]``
* ``w1, w3``  packed e2m1 nibbles, uint8 ``[E, I, H/2]`` (even K in the low nibble)
* ``s1, s3``  E8M0 scale codes, uint8 ``[E, I, H/32]``
* ``w2``      uint8 ``[E, H, I/2]``;  ``s2`` uint8 ``[E, H, I/32]``

Workload shapes follow the five layer shapes the method is exercised on:
a tiny layer, two decode-shaped layers, the 4,604-token prefill of the
paper's abstract ("DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and
Inference Performance Engineering", abstract) and a Zipf-skewed stress layer.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

# tensor ids of the counter-based generator
TID_X, TID_LOGITS, TID_ZIPF, TID_W1, TID_S1, TID_W3, TID_S3, TID_W2, TID_S2 = range(9)
# the router weights and the shared expert's weights (one more expert in the
# same format as the routed ones)
TID_WG, TID_SW1, TID_SS1, TID_SW3, TID_SS3, TID_SW2, TID_SS2 = range(9, 16)
# the FP8 dense projection: activations, weight codes, weight scales
TID_DX, TID_DW, TID_DS = range(16, 19)


@dataclasses.dataclass(frozen=True)
class Shape:
    T: int
    H: int
    I: int
    E: int
    k: int
    x_sigma: float = 1.0
    zipf_s: float = 0.0          # 0 = no popularity bias on the logits
    seed: int = 0


CONFIGS = {
    "c0": Shape(T=16, H=256, I=128, E=8, k=2, seed=0),
    "c1": Shape(T=8, H=4096, I=1536, E=64, k=6, seed=1),
    "c2": Shape(T=64, H=7168, I=2048, E=256, k=8, seed=2),
    "c3": Shape(T=4604, H=7168, I=2048, E=256, k=8, x_sigma=1.5, seed=3),
    "c4": Shape(T=16384, H=7168, I=2048, E=256, k=8, zipf_s=1.2, seed=4),
}

CONFIG_NAMES = {
    "c0": "tiny T16 H256 I128 E8 top2",
    "c1": "decode T8 H4096 I1536 E64 top6",
    "c2": "decode-batch T64 H7168 I2048 E256 top8",
    "c3": "prefill T4604 H7168 I2048 E256 top8",
    "c4": "zipf-skew T16384 H7168 I2048 E256 top8",
}


def build() -> str:
    src = os.path.join(_HERE, "synth.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           src, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        lib.synth_mix64.restype = u64
        lib.synth_mix64.argtypes = [u64]
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_draw.restype = u64
        lib.synth_draw.argtypes = [u64, u64]
        lib.synth_bytes.argtypes = [u64, u64, p, ctypes.c_size_t]
        lib.synth_uniform_codes.argtypes = [u64, u64, p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int]
        lib.synth_normal_f32.argtypes = [u64, u64, p, ctypes.c_size_t, ctypes.c_double]
        lib.synth_f32_to_bf16.argtypes = [p, p, ctypes.c_size_t]
        lib.synth_zipf_bias.argtypes = [u64, u64, ctypes.c_int, ctypes.c_double, p]
        lib.synth_add_col_bias.argtypes = [p, p, ctypes.c_size_t, ctypes.c_int]
        lib.synth_w2_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, p, p]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def mix64(x: int) -> int:
    return int(_load().synth_mix64(x))


def draw(seed: int, tensor_id: int, n: int) -> int:
    lib = _load()
    return int(lib.synth_draw(lib.synth_key(seed, tensor_id), n))


def random_bytes(seed: int, tensor_id: int, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint8)
    _load().synth_bytes(seed, tensor_id, _ptr(out), out.size)
    return out


def uniform_codes(seed: int, tensor_id: int, shape, lo: int, hi: int) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint8)
    _load().synth_uniform_codes(seed, tensor_id, _ptr(out), out.size, lo, hi)
    return out


def normal_f32(seed: int, tensor_id: int, shape, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(seed, tensor_id, _ptr(out), out.size, float(sigma))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(_ptr(a), _ptr(out), a.size)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def zipf_bias(seed: int, E: int, s: float) -> np.ndarray:
    out = np.empty(E, dtype=np.float32)
    _load().synth_zipf_bias(seed, TID_ZIPF, E, float(s), _ptr(out))
    return out


def w2_probe(E: int, H: int, I: int):
    w2 = np.empty((E, H, I // 2), dtype=np.uint8)
    s2 = np.empty((E, H, I // 32), dtype=np.uint8)
    _load().synth_w2_probe(E, H, I, _ptr(w2), _ptr(s2))
    return w2, s2


@dataclasses.dataclass
class LayerInputs:
    shape: Shape
    x: np.ndarray
    logits: np.ndarray
    w1: np.ndarray | None = None
    s1: np.ndarray | None = None
    w3: np.ndarray | None = None
    s3: np.ndarray | None = None
    w2: np.ndarray | None = None
    s2: np.ndarray | None = None


def make_activations(sh: Shape):
    """x (bf16 bits [T,H]) and router logits (f32 [T,E])."""
    x = f32_to_bf16_bits(normal_f32(sh.seed, TID_X, (sh.T, sh.H), sh.x_sigma))
    logits = normal_f32(sh.seed, TID_LOGITS, (sh.T, sh.E), 1.0)
    if sh.zipf_s > 0:
        bias = zipf_bias(sh.seed, sh.E, sh.zipf_s)
        _load().synth_add_col_bias(_ptr(logits), _ptr(bias), sh.T, sh.E)
    return x, logits


def make_weights(sh: Shape, probe_w2: bool = False):
    """Packed e2m1 weights with E8M0 block scales; scale exponents uniform in [-6, -2]."""
    E, H, I = sh.E, sh.H, sh.I
    w1 = random_bytes(sh.seed, TID_W1, (E, I, H // 2))
    s1 = uniform_codes(sh.seed, TID_S1, (E, I, H // 32), 121, 125)
    w3 = random_bytes(sh.seed, TID_W3, (E, I, H // 2))
    s3 = uniform_codes(sh.seed, TID_S3, (E, I, H // 32), 121, 125)
    if probe_w2:
        w2, s2 = w2_probe(E, H, I)
    else:
        w2 = random_bytes(sh.seed, TID_W2, (E, H, I // 2))
        s2 = uniform_codes(sh.seed, TID_S2, (E, H, I // 32), 121, 125)
    return w1, s1, w3, s3, w2, s2


def make_inputs(cfg, probe_w2: bool = False, with_weights: bool = True, **overrides) -> LayerInputs:
    sh = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    if overrides:
        sh = dataclasses.replace(sh, **overrides)
    x, logits = make_activations(sh)
    li = LayerInputs(shape=sh, x=x, logits=logits)
    if with_weights:
        li.w1, li.s1, li.w3, li.s3, li.w2, li.s2 = make_weights(sh, probe_w2)
    return li


def make_router_weights(sh: Shape) -> np.ndarray:
    """Router weights Wg as bf16 bits [E, H]: N(0, 1/H), so that with N(0, sigma)
    activations the logits x . Wg[e] are about N(0, sigma^2)."""
    return f32_to_bf16_bits(normal_f32(sh.seed, TID_WG, (sh.E, sh.H), 1.0 / np.sqrt(sh.H)))


def make_shared_weights(sh: Shape, I_shared: int | None = None):
    """One shared expert (E = 1) in the routed experts' format, intermediate size
    I_shared (default I): w1, s1, w3, s3 [1, Is, H/2 | H/32], w2, s2 [1, H, Is/2 | Is/32]."""
    H, Is = sh.H, (sh.I if I_shared is None else I_shared)
    w1 = random_bytes(sh.seed, TID_SW1, (1, Is, H // 2))
    s1 = uniform_codes(sh.seed, TID_SS1, (1, Is, H // 32), 121, 125)
    w3 = random_bytes(sh.seed, TID_SW3, (1, Is, H // 2))
    s3 = uniform_codes(sh.seed, TID_SS3, (1, Is, H // 32), 121, 125)
    w2 = random_bytes(sh.seed, TID_SW2, (1, H, Is // 2))
    s2 = uniform_codes(sh.seed, TID_SS2, (1, H, Is // 32), 121, 125)
    return w1, s1, w3, s3, w2, s2


# ------------------------------------------------------ FP8 dense projection
@dataclasses.dataclass(frozen=True)
class DenseShape:
    T: int
    K: int
    N: int
    seed: int = 0


DENSE_CONFIGS = {
    "d0": DenseShape(T=5, K=256, N=96, seed=20),
    "d1": DenseShape(T=8, K=16384, N=7168, seed=21),
    "d3": DenseShape(T=4604, K=16384, N=7168, seed=23),
}

DENSE_NAMES = {
    "d0": "dense tiny T5 K256 N96",
    "d1": "dense-decode T8 K16384 N7168",
    "d3": "dense-prefill T4604 K16384 N7168",
}


@dataclasses.dataclass
class DenseInputs:
    shape: DenseShape
    x: np.ndarray    # [T, K] bf16 bits
    wq: np.ndarray   # [N, K] e4m3 codes (no NaN codes)
    ws: np.ndarray   # [N, K/32] E8M0 codes


def make_dense_inputs(cfg, **overrides) -> DenseInputs:
    """x bf16 N(0, 1); weight codes uniform over the 254 non-NaN e4m3 bytes;
    weight scale codes uniform over {118..122} (2^-9 .. 2^-5)."""
    sh = DENSE_CONFIGS[cfg] if isinstance(cfg, str) else cfg
    if overrides:
        sh = dataclasses.replace(sh, **overrides)
    x = f32_to_bf16_bits(normal_f32(sh.seed, TID_DX, (sh.T, sh.K), 1.0))
    c = uniform_codes(sh.seed, TID_DW, (sh.N, sh.K), 0, 253)
    wq = (c + (c >= 0x7F)).astype(np.uint8)          # skip 0x7F; 253 + 1 = 0xFE tops out below 0xFF
    ws = uniform_codes(sh.seed, TID_DS, (sh.N, sh.K // 32), 118, 122)
    return DenseInputs(shape=sh, x=x, wq=wq, ws=ws)
