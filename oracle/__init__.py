"""CPU oracle for the FP4 routed-expert MoE layer (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the GPU library or its
Python binding.  Every function here is the plain definition of one step of
the layer (see the header of ``oracle.c`` for the passages of the pages each
step follows).

``oracle.c`` is built twice: ``liboracle.so`` accumulates in fp32 (the
precision the method fixes; the default, ``PRECISION``), ``liboracle_f64.so``
in fp64 (a diagnostic of the fp32 build's own rounding).  ``using("fp64")``
switches the functions below to the diagnostic build inside a ``with`` block.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SOS = {"fp32": os.path.join(_HERE, "liboracle.so"), "fp64": os.path.join(_HERE, "liboracle_f64.so")}
_DEFS = {"fp32": [], "fp64": ["-DORC_ACC_FP64"]}
PRECISION = "fp32"


def build() -> str:
    src = os.path.join(_HERE, "oracle.c")
    for prec, so in _SOS.items():
        tmp = so + ".tmp"
        # -ffp-contract=off: no fused multiply-adds, every product is rounded as written
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-ffp-contract=off", *_DEFS[prec], src, "-o", tmp, "-lm"])
        os.replace(tmp, so)
    return _SOS["fp32"]


_libs: dict = {}
_current = [PRECISION]


@contextlib.contextmanager
def using(precision: str):
    """Run the oracle calls inside the block on the build of `precision`."""
    assert precision in _SOS, precision
    old = _current[0]
    _current[0] = precision
    try:
        yield
    finally:
        _current[0] = old


def precision() -> str:
    """The accumulation precision the calls run in now (as reported by the build)."""
    return _load().orc_precision().decode()


def _load():
    prec = _current[0]
    if prec not in _libs:
        so = _SOS[prec]
        if not os.path.exists(so):
            build()
        lib = ctypes.CDLL(so)
        p, i32, i64, u = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_uint
        d = ctypes.c_double
        lib.orc_e2m1.restype = d
        lib.orc_e2m1.argtypes = [u]
        lib.orc_e8m0.restype = d
        lib.orc_e8m0.argtypes = [u]
        lib.orc_e4m3.restype = d
        lib.orc_e4m3.argtypes = [u]
        lib.orc_bf16.restype = d
        lib.orc_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_e4m3_rne_sat.restype = u
        lib.orc_e4m3_rne_sat.argtypes = [d]
        lib.orc_decode_fp4_matrix.argtypes = [p, p, i64, i32, p]
        lib.orc_decode_mxfp8.argtypes = [p, p, i64, i32, p]
        lib.orc_quant_block32.argtypes = [p, p, p]
        lib.orc_quant_mxfp8_bf16.argtypes = [p, i64, i32, p, p]
        lib.orc_quant_mxfp8_f32.argtypes = [p, i64, i32, p, p]
        lib.orc_route_token.argtypes = [p, i32, i32, p, p]
        lib.orc_route.argtypes = [p, i64, i32, i32, p, p]
        lib.orc_sort.argtypes = [p, i64, i32, p, p, p, p]
        lib.orc_expert_gate_up.argtypes = [p, p, i32, i32, p, p, p, p, p, p]
        lib.orc_router_logits.argtypes = [p, p, i64, i32, i32, p, p]
        lib.orc_layer_tokens_shared.argtypes = [p, p, i32, i32, i32, i32, p, p, p, p, p, p, i32,
                                                p, p, p, p, p, p, p, i64, p]
        lib.orc_swiglu_requant.argtypes = [p, p, i32, p, p, p]
        lib.orc_expert_down.argtypes = [p, p, i32, i32, p, p, p]
        lib.orc_dense_fp8.argtypes = [p, p, p, p, i32, i32, p, i64, p]
        lib.orc_layer_tokens.argtypes = [p, p, i32, i32, i32, i32, p, p, p, p, p, p,
                                         p, i64, p, p, p, p]
        lib.orc_layer_pairs.argtypes = [p, p, i32, i32, i32, i32, p, p, p, p, p, p,
                                        p, i64, p, p, p, p, p]
        lib.orc_precision.restype = ctypes.c_char_p
        lib.orc_precision.argtypes = []
        _libs[prec] = lib
    return _libs[prec]


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "contiguous numpy array required"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ decoders
def e2m1(code: int) -> float:
    return _load().orc_e2m1(code)


def e8m0(code: int) -> float:
    return _load().orc_e8m0(code)


def e4m3(byte: int) -> float:
    return _load().orc_e4m3(byte)


def bf16(bits: int) -> float:
    return _load().orc_bf16(bits)


def e4m3_rne_sat(a: float) -> int:
    return int(_load().orc_e4m3_rne_sat(float(a)))


def decode_fp4_matrix(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Packed e2m1 [rows, K/2] + scales [rows, K/32] -> float64 [rows, K]."""
    w = _c(w, np.uint8)
    s = _c(s, np.uint8)
    K = w.shape[-1] * 2
    rows = w.size // w.shape[-1]
    out = np.empty(w.shape[:-1] + (K,), dtype=np.float64)
    _load().orc_decode_fp4_matrix(_p(w), _p(s), rows, K, _p(out))
    return out


def decode_mxfp8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    K = q.shape[-1]
    rows = q.size // K
    out = np.empty(q.shape, dtype=np.float64)
    _load().orc_decode_mxfp8(_p(q), _p(s), rows, K, _p(out))
    return out


# -------------------------------------------------------------- quantisation
def quant_block32(v) -> tuple[np.ndarray, int]:
    v = _c(v, np.float64)
    assert v.shape == (32,)
    q = np.empty(32, dtype=np.uint8)
    s = np.empty(1, dtype=np.uint8)
    _load().orc_quant_block32(_p(v), _p(q), _p(s))
    return q, int(s[0])


def quant_mxfp8_bf16(x_bits: np.ndarray):
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 32), dtype=np.uint8)
    _load().orc_quant_mxfp8_bf16(_p(x), M, K, _p(q), _p(s))
    return q, s


def quant_mxfp8_f32(x: np.ndarray):
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 32), dtype=np.uint8)
    _load().orc_quant_mxfp8_f32(_p(x), M, K, _p(q), _p(s))
    return q, s


# -------------------------------------------------------------- route / sort
def route(logits: np.ndarray, k: int):
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float32)
    _load().orc_route(_p(lg), T, E, k, _p(ids), _p(gates))
    return ids, gates


def sort(ids: np.ndarray, E: int):
    ids = _c(ids, np.int32).reshape(-1)
    P = ids.size
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_pair = np.empty(P, dtype=np.int32)
    pair_pos = np.empty(P, dtype=np.int32)
    _load().orc_sort(_p(ids), P, E, _p(counts), _p(offsets), _p(sorted_pair), _p(pair_pos))
    return counts, offsets, sorted_pair, pair_pos


# ------------------------------------------------------------------- experts
def expert_gate_up(xq_row, xs_row, w1e, s1e, w3e, s3e):
    xq_row = _c(xq_row, np.uint8)
    xs_row = _c(xs_row, np.uint8)
    I, Hh = w1e.shape
    H = Hh * 2
    G = np.empty(I, dtype=np.float64)
    U = np.empty(I, dtype=np.float64)
    _load().orc_expert_gate_up(_p(xq_row), _p(xs_row), H, I, _p(_c(w1e, np.uint8)),
                               _p(_c(s1e, np.uint8)), _p(_c(w3e, np.uint8)),
                               _p(_c(s3e, np.uint8)), _p(G), _p(U))
    return G, U


def swiglu_requant(G, U):
    G = _c(G, np.float64)
    U = _c(U, np.float64)
    I = G.size
    h = np.empty(I, dtype=np.float32)
    hq = np.empty(I, dtype=np.uint8)
    hs = np.empty(I // 32, dtype=np.uint8)
    _load().orc_swiglu_requant(_p(G), _p(U), I, _p(h), _p(hq), _p(hs))
    return h, hq, hs


def expert_down(hq, hs, w2e, s2e):
    hq = _c(hq, np.uint8)
    hs = _c(hs, np.uint8)
    H, Ih = w2e.shape
    I = Ih * 2
    O = np.empty(H, dtype=np.float64)
    _load().orc_expert_down(_p(hq), _p(hs), H, I, _p(_c(w2e, np.uint8)), _p(_c(s2e, np.uint8)), _p(O))
    return O


def layer_tokens(inp, tokens=None, want_pairs: bool = False):
    """The layer's output rows y[t] (float32 [len(tokens), H]) for the given tokens.

    ``inp`` is a ``synth.LayerInputs``.  With ``want_pairs`` also returns the
    per-(token, slot) h (fp32), hq and hs.
    """
    sh = inp.shape
    T, H, I, E, k = sh.T, sh.H, sh.I, sh.E, sh.k
    toks = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    n = toks.size
    y = np.empty((n, H), dtype=np.float32)
    h = hq = hs = None
    if want_pairs:
        h = np.empty((n * k, I), dtype=np.float32)
        hq = np.empty((n * k, I), dtype=np.uint8)
        hs = np.empty((n * k, I // 32), dtype=np.uint8)
    _load().orc_layer_tokens(_p(_c(inp.x, np.uint16)), _p(_c(inp.logits, np.float32)), H, I, E, k,
                             _p(inp.w1), _p(inp.s1), _p(inp.w3), _p(inp.s3), _p(inp.w2), _p(inp.s2),
                             _p(toks), n, _p(y), _p(h), _p(hq), _p(hs))
    if want_pairs:
        return y, h, hq, hs
    return y


def layer_pairs(inp, pairs):
    """Per-pair intermediates of the layer for (token, slot) pairs p = t*k + j:
    (expert [n] int32, h [n, I] fp32, hq [n, I], hs [n, I/32], O [n, H] float64
    holding the build's accumulation-precision values), by the same steps as
    ``layer_tokens``."""
    sh = inp.shape
    H, I, E, k = sh.H, sh.I, sh.E, sh.k
    pr = _c(pairs, np.int32)
    n = pr.size
    ex = np.empty(n, dtype=np.int32)
    h = np.empty((n, I), dtype=np.float32)
    hq = np.empty((n, I), dtype=np.uint8)
    hs = np.empty((n, I // 32), dtype=np.uint8)
    O = np.empty((n, H), dtype=np.float64)
    _load().orc_layer_pairs(_p(_c(inp.x, np.uint16)), _p(_c(inp.logits, np.float32)), H, I, E, k,
                            _p(inp.w1), _p(inp.s1), _p(inp.w3), _p(inp.s3), _p(inp.w2), _p(inp.s2),
                            _p(pr), n, _p(ex), _p(h), _p(hq), _p(hs), _p(O))
    return ex, h, hq, hs, O


# ------------------------------------------------- router and shared expert
def router_logits(x_bits: np.ndarray, wg_bits: np.ndarray):
    """Exact router logits x . Wg[e] (fp64) of bf16 operands and the absolute
    sums that bound any fp32 evaluation's rounding error: ([T, E], [T, E])."""
    x = _c(x_bits, np.uint16)
    wg = _c(wg_bits, np.uint16)
    T, H = x.shape
    E = wg.shape[0]
    assert wg.shape[1] == H
    logit = np.empty((T, E), dtype=np.float64)
    absum = np.empty((T, E), dtype=np.float64)
    _load().orc_router_logits(_p(x), _p(wg), T, H, E, _p(logit), _p(absum))
    return logit, absum


def layer_tokens_shared(inp, logits, shared, tokens=None):
    """y rows of the layer with routing on the given fp32 logits [T, E] and, if
    ``shared`` = (w1, s1, w3, s3, w2, s2) of one expert is not None, that
    expert's output added after the k routed slots."""
    sh = inp.shape
    T, H, I, E, k = sh.T, sh.H, sh.I, sh.E, sh.k
    toks = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    y = np.empty((toks.size, H), dtype=np.float32)
    if shared is None:
        sp = [None] * 6
        Is = 0
    else:
        sp = [_c(a, np.uint8) for a in shared]
        Is = sp[0].shape[-2]
    _load().orc_layer_tokens_shared(
        _p(_c(inp.x, np.uint16)), _p(_c(logits, np.float32)), H, I, E, k,
        _p(inp.w1), _p(inp.s1), _p(inp.w3), _p(inp.s3), _p(inp.w2), _p(inp.s2), Is,
        *[(None if a is None else _p(a)) for a in sp], _p(toks), toks.size, _p(y))
    return y


# ------------------------------------------------------ FP8 dense projection
def dense_fp8(xq, xs, wq, ws, tokens=None):
    """y [ntok, N] fp64 = MXFP8 rows of x (xq [T, K], xs [T, K/32]) times the
    FP8 weights (wq [N, K] e4m3, ws [N, K/32] E8M0), rows ``tokens``."""
    xq = _c(xq, np.uint8)
    xs = _c(xs, np.uint8)
    wq = _c(wq, np.uint8)
    ws = _c(ws, np.uint8)
    T, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and xs.shape == (T, K // 32) and ws.shape == (N, K // 32)
    toks = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    y = np.empty((toks.size, N), dtype=np.float64)
    _load().orc_dense_fp8(_p(xq), _p(xs), _p(wq), _p(ws), N, K, _p(toks), toks.size, _p(y))
    return y
