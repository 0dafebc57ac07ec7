"""MI355X-native FP4 routed-expert MoE layer: thin Python binding.

Every function marshals torch tensors (device memory) and the current HIP
stream into one call of the C ABI in ``include/moe_fp4.h``; every step of the
layer runs in the gfx950 kernels of ``libmoe_fp4.so``.  PyTorch provides
device memory and streams only.

    pw = prepack_weights(w1, s1, w3, s3, w2, s2)          # once, at load time
    y  = moe_layer(pw, x_bf16, logits, k)                  # route/sort/quant/experts/combine
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib
from ._lib import (MOE_FLAG_FORCE_DECODE, MOE_FLAG_FORCE_PREFILL, MoeError,  # noqa: F401
                   MoeFp4Weights)

__all__ = [
    "route_topk", "sort_permute", "quant_act_mxfp8", "prepack_weights", "PackedWeights",
    "expert_up", "expert_down", "combine", "grouped_forward", "moe_layer",
    "forward_workspace_size", "layer_forward", "layer_workspace_size", "layer_forward_noalloc",
    "router_logits",
    "router_workspace_size",
    "shared_workspace_size", "shared_expert", "combine_shared", "layer_full_workspace_size",
    "layer_forward_full", "DenseWeights", "dense_prepack", "dense_forward", "dense_layer",
    "MOE_FLAG_FORCE_DECODE", "MOE_FLAG_FORCE_PREFILL", "MoeError",
]


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise ValueError("device tensor required")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor required")
    return ctypes.c_void_p(t.data_ptr())


def _check_dtype(t: torch.Tensor, dtypes, name: str):
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")


def route_topk(logits: torch.Tensor, k: int, ids: torch.Tensor | None = None,
               gates: torch.Tensor | None = None):
    """logits [T, E] fp32 -> (topk_ids [T, k] int32, topk_gates [T, k] fp32)."""
    _check_dtype(logits, (torch.float32,), "logits")
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if gates is None:
        gates = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _lib.check(_lib.lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(gates),
                                         _stream(logits)), "moe_route_topk")
    return ids, gates


def sort_permute(ids: torch.Tensor, E: int, out=None, workspace: torch.Tensor | None = None):
    """topk_ids [T, k] -> (counts [E], offsets [E+1], sorted_pair [T*k], pair_pos [T*k])."""
    _check_dtype(ids, (torch.int32,), "topk_ids")
    T, k = ids.shape
    dev = ids.device
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev))
    counts, offsets, sp, pp = out
    L = _lib.lib()
    need = L.moe_sort_permute_workspace_size(T, E, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel()
    _lib.check(L.moe_sort_permute(_ptr(ids), T, E, k, _ptr(counts), _ptr(offsets), _ptr(sp),
                                  _ptr(pp), _ptr(workspace), wsb, _stream(ids)),
               "moe_sort_permute")
    return counts, offsets, sp, pp


def quant_act_mxfp8(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """x [M, K] bf16 -> (q [M, K] e4m3fn bytes as uint8, s [M, K/32] E8M0 codes as uint8)."""
    _check_dtype(x, (torch.bfloat16, torch.int16, torch.uint16), "x")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _lib.check(_lib.lib().moe_quant_act_mxfp8(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(x)),
               "moe_quant_act_mxfp8")
    return q, s


@dataclasses.dataclass
class PackedWeights:
    """Prepacked expert weights: the device buffer plus the plain-C descriptor."""
    buffer: torch.Tensor
    desc: MoeFp4Weights

    @property
    def E(self):
        return self.desc.E

    @property
    def H(self):
        return self.desc.H

    @property
    def I(self):
        return self.desc.I


def packed_weight_bytes(E: int, H: int, I: int) -> int:
    return int(_lib.lib().moe_fp4_packed_weight_bytes(E, H, I))


def prepack_weights(w1, s1, w3, s3, w2, s2) -> PackedWeights:
    """Canonical packed-e2m1 weights + E8M0 scales (uint8 device tensors):
    w1, w3 [E, I, H/2], s1, s3 [E, I, H/32], w2 [E, H, I/2], s2 [E, H, I/32]."""
    for name, t in (("w1", w1), ("s1", s1), ("w3", w3), ("s3", s3), ("w2", w2), ("s2", s2)):
        _check_dtype(t, (torch.uint8,), name)
    E, I, Hh = w1.shape
    H = Hh * 2
    nbytes = packed_weight_bytes(E, H, I)
    if nbytes == 0:
        raise MoeError(_lib.MOE_ERR_UNSUPPORTED, "moe_fp4_packed_weight_bytes")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=w1.device)
    desc = MoeFp4Weights()
    _lib.check(_lib.lib().moe_fp4_prepack_weights(
        _ptr(w1), _ptr(s1), _ptr(w3), _ptr(s3), _ptr(w2), _ptr(s2), E, H, I, _ptr(buf), nbytes,
        ctypes.byref(desc), _stream(w1)), "moe_fp4_prepack_weights")
    return PackedWeights(buffer=buf, desc=desc)


def stage_workspace_size(T: int, E: int, k: int, H: int, I: int) -> int:
    return int(_lib.lib().moe_fp4_stage_workspace_size(T, E, k, H, I))


def _stage_ws(T, k, pw, dev, workspace):
    need = stage_workspace_size(T, pw.E, k, pw.H, pw.I)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    return workspace


def expert_up(pw: PackedWeights, xq, xs, offsets, sorted_pair, T: int, k: int, flags: int = 0,
              hq=None, hs=None, workspace=None):
    """Gate/up GEMM + SwiGLU + MXFP8 of h -> (hq [T*k, I], hs [T*k, I/32]), sorted order."""
    dev = xq.device
    P = T * k
    if hq is None:
        hq = torch.empty((P, pw.I), dtype=torch.uint8, device=dev)
    if hs is None:
        hs = torch.empty((P, pw.I // 32), dtype=torch.uint8, device=dev)
    workspace = _stage_ws(T, k, pw, dev, workspace)
    _lib.check(_lib.lib().moe_fp4_expert_up(
        ctypes.byref(pw.desc), _ptr(xq), _ptr(xs), _ptr(offsets), _ptr(sorted_pair), T, k, _ptr(hq),
        _ptr(hs), _ptr(workspace), workspace.numel(), flags, _stream(xq)), "moe_fp4_expert_up")
    return hq, hs


def expert_down(pw: PackedWeights, hq, hs, offsets, T: int, k: int, flags: int = 0, O=None,
                workspace=None):
    """Down GEMM -> O [T*k, H] bf16 (fp32 accumulation, rounded once), sorted order."""
    dev = hq.device
    if O is None:
        O = torch.empty((T * k, pw.H), dtype=torch.bfloat16, device=dev)
    _check_dtype(O, (torch.bfloat16,), "O")
    workspace = _stage_ws(T, k, pw, dev, workspace)
    _lib.check(_lib.lib().moe_fp4_expert_down(
        ctypes.byref(pw.desc), _ptr(hq), _ptr(hs), _ptr(offsets), T, k, _ptr(O), _ptr(workspace),
        workspace.numel(), flags, _stream(hq)), "moe_fp4_expert_down")
    return O


def combine(O, gates, pair_pos, T: int, k: int, H: int, y=None):
    """y [T, H] fp32 = gate-weighted sum of the bf16 expert outputs O, in slot order."""
    _check_dtype(O, (torch.bfloat16,), "O")
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=O.device)
    _lib.check(_lib.lib().moe_combine(_ptr(O), _ptr(gates), _ptr(pair_pos), T, k, H, _ptr(y),
                                      _stream(O)), "moe_combine")
    return y


def forward_workspace_size(T: int, E: int, k: int, H: int, I: int, flags: int = 0) -> int:
    return int(_lib.lib().moe_fp4_forward_workspace_size(T, E, k, H, I, flags))


def grouped_forward(pw: PackedWeights, xq, xs, gates, offsets, sorted_pair, pair_pos, flags: int = 0,
                    y=None, workspace=None):
    """Expert GEMMs + combine -> y [T, H] fp32."""
    T, k = gates.shape
    dev = xq.device
    if y is None:
        y = torch.empty((T, pw.H), dtype=torch.float32, device=dev)
    if workspace is None:
        need = forward_workspace_size(T, pw.E, k, pw.H, pw.I, flags)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _lib.check(_lib.lib().moe_fp4_grouped_forward(
        ctypes.byref(pw.desc), _ptr(xq), _ptr(xs), _ptr(gates), _ptr(offsets), _ptr(sorted_pair),
        _ptr(pair_pos), T, k, _ptr(y), _ptr(workspace), workspace.numel(), flags, _stream(xq)),
        "moe_fp4_grouped_forward")
    return y


def layer_workspace_size(T: int, E: int, k: int, H: int, I: int, flags: int = 0) -> int:
    return int(_lib.lib().moe_fp4_layer_workspace_size(T, E, k, H, I, flags))


def layer_forward(pw: PackedWeights, x: torch.Tensor, logits: torch.Tensor, k: int, flags: int = 0,
                  y=None, workspace=None):
    """The whole layer in one library call (moe_fp4_layer_forward) -> y [T, H] fp32."""
    _check_dtype(x, (torch.bfloat16, torch.int16, torch.uint16), "x")
    _check_dtype(logits, (torch.float32,), "logits")
    T, H = x.shape
    if logits.shape[0] != T or H != pw.H or logits.shape[1] != pw.E:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, logits {tuple(logits.shape)}, "
                         f"weights E={pw.E} H={pw.H}")
    dev = x.device
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
    if workspace is None:
        need = layer_workspace_size(T, pw.E, k, pw.H, pw.I, flags)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _lib.check(_lib.lib().moe_fp4_layer_forward(
        ctypes.byref(pw.desc), _ptr(x), _ptr(logits), T, k, _ptr(y), _ptr(workspace),
        workspace.numel(), flags, _stream(x)), "moe_fp4_layer_forward")
    return y


def layer_forward_noalloc(pw: PackedWeights, x: torch.Tensor, logits: torch.Tensor, k: int,
                          flags: int = 0, y=None):
    """The whole layer with the library's fixed per-GPU scratch as workspace
    (moe_fp4_layer_forward_noalloc): the call allocates nothing itself."""
    _check_dtype(x, (torch.bfloat16, torch.int16, torch.uint16), "x")
    _check_dtype(logits, (torch.float32,), "logits")
    T, H = x.shape
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _lib.check(_lib.lib().moe_fp4_layer_forward_noalloc(
        ctypes.byref(pw.desc), _ptr(x), _ptr(logits), T, k, _ptr(y), flags, _stream(x)),
        "moe_fp4_layer_forward_noalloc")
    return y


def moe_layer(pw: PackedWeights, x: torch.Tensor, logits: torch.Tensor, k: int, flags: int = 0,
              return_intermediates: bool = False):
    """The whole layer: route -> sort/permute -> MXFP8(x) -> experts -> combine."""
    ids, gates = route_topk(logits, k)
    counts, offsets, sp, pp = sort_permute(ids, pw.E)
    xq, xs = quant_act_mxfp8(x)
    y = grouped_forward(pw, xq, xs, gates, offsets, sp, pp, flags)
    if return_intermediates:
        return y, dict(topk_ids=ids, topk_gates=gates, expert_counts=counts, expert_offsets=offsets,
                       sorted_pair=sp, pair_pos=pp, xq=xq, xs=xs)
    return y


# ----------------------------------------------------- router and shared expert
def router_workspace_size(T: int, H: int, E: int) -> int:
    return int(_lib.lib().moe_router_workspace_size(T, H, E))


def router_logits(x: torch.Tensor, router_w: torch.Tensor, logits=None, workspace=None):
    """logits [T, E] fp32 = x [T, H] bf16 . router_w [E, H] bf16^T (fp32 accumulation)."""
    _check_dtype(x, (torch.bfloat16, torch.int16, torch.uint16), "x")
    _check_dtype(router_w, (torch.bfloat16, torch.int16, torch.uint16), "router_w")
    T, H = x.shape
    E, H2 = router_w.shape
    if H2 != H:
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, router_w {tuple(router_w.shape)}")
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check_dtype(logits, (torch.float32,), "logits")
    if workspace is None:
        need = router_workspace_size(T, H, E)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _lib.check(_lib.lib().moe_router_logits(_ptr(x), _ptr(router_w), T, H, E, _ptr(logits),
                                            _ptr(workspace), workspace.numel(), _stream(x)),
               "moe_router_logits")
    return logits


def shared_workspace_size(T: int, H: int, I_shared: int, flags: int = 0) -> int:
    return int(_lib.lib().moe_fp4_shared_workspace_size(T, H, I_shared, flags))


def shared_expert(pws: PackedWeights, xq, xs, flags: int = 0, O_shared=None, workspace=None):
    """The always-active expert (E == 1) on every token's MXFP8 row -> O_shared [T, H] bf16."""
    T = xq.shape[0]
    dev = xq.device
    if O_shared is None:
        O_shared = torch.empty((T, pws.H), dtype=torch.bfloat16, device=dev)
    _check_dtype(O_shared, (torch.bfloat16,), "O_shared")
    if workspace is None:
        need = shared_workspace_size(T, pws.H, pws.I, flags)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _lib.check(_lib.lib().moe_fp4_shared_expert(
        ctypes.byref(pws.desc), _ptr(xq), _ptr(xs), T, _ptr(O_shared), _ptr(workspace),
        workspace.numel(), flags, _stream(xq)), "moe_fp4_shared_expert")
    return O_shared


def combine_shared(O, gates, pair_pos, O_shared, T: int, k: int, H: int, y=None):
    """combine() plus the shared expert's row, added after the k routed slots."""
    _check_dtype(O, (torch.bfloat16,), "O")
    _check_dtype(O_shared, (torch.bfloat16,), "O_shared")
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=O.device)
    _lib.check(_lib.lib().moe_combine_shared(_ptr(O), _ptr(gates), _ptr(pair_pos), _ptr(O_shared),
                                             T, k, H, _ptr(y), _stream(O)), "moe_combine_shared")
    return y


def layer_full_workspace_size(T: int, E: int, k: int, H: int, I: int, n_shared: int = 0,
                              flags: int = 0) -> int:
    return int(_lib.lib().moe_fp4_layer_full_workspace_size(T, E, k, H, I, n_shared, flags))


def layer_forward_full(pw: PackedWeights, n_shared: int, router_w: torch.Tensor, x: torch.Tensor,
                       k: int, flags: int = 0, y=None, workspace=None):
    """Router GEMM + the layer in one library call; the last ``n_shared`` experts of ``pw``
    are shared (every token, weight 1), the router covers the others."""
    _check_dtype(x, (torch.bfloat16, torch.int16, torch.uint16), "x")
    _check_dtype(router_w, (torch.bfloat16, torch.int16, torch.uint16), "router_w")
    T, H = x.shape
    if H != pw.H or tuple(router_w.shape) != (pw.E - n_shared, pw.H):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, router_w {tuple(router_w.shape)}, "
                         f"weights E={pw.E} (n_shared={n_shared}) H={pw.H}")
    dev = x.device
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
    if workspace is None:
        need = layer_full_workspace_size(T, pw.E, k, pw.H, pw.I, n_shared, flags)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _lib.check(_lib.lib().moe_fp4_layer_forward_full(
        ctypes.byref(pw.desc), n_shared, _ptr(router_w), _ptr(x), T, k, _ptr(y), _ptr(workspace),
        workspace.numel(), flags, _stream(x)), "moe_fp4_layer_forward_full")
    return y


# ------------------------------------------------------ FP8 dense projection
@dataclasses.dataclass
class DenseWeights:
    """Prepacked FP8 dense weights: the device buffer plus the plain-C descriptor."""
    buffer: torch.Tensor
    desc: _lib.MoeFp8DenseWeights

    @property
    def N(self):
        return self.desc.N

    @property
    def K(self):
        return self.desc.K


def dense_prepack(wq, ws) -> DenseWeights:
    """wq [N, K] e4m3 codes, ws [N, K/32] E8M0 codes (uint8 device tensors)."""
    _check_dtype(wq, (torch.uint8,), "wq")
    _check_dtype(ws, (torch.uint8,), "ws")
    N, K = wq.shape
    nbytes = int(_lib.lib().moe_fp8_dense_packed_bytes(N, K))
    if nbytes == 0:
        raise MoeError(_lib.MOE_ERR_UNSUPPORTED, "moe_fp8_dense_packed_bytes")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=wq.device)
    desc = _lib.MoeFp8DenseWeights()
    _lib.check(_lib.lib().moe_fp8_dense_prepack(_ptr(wq), _ptr(ws), N, K, _ptr(buf), nbytes,
                                                ctypes.byref(desc), _stream(wq)),
               "moe_fp8_dense_prepack")
    return DenseWeights(buffer=buf, desc=desc)


def dense_forward(dw: DenseWeights, xq, xs, flags: int = 0, y=None):
    """y [T, N] bf16 = MXFP8 rows (xq [T, K], xs [T, K/32]) times the FP8 dense weights."""
    T = xq.shape[0]
    if y is None:
        y = torch.empty((T, dw.N), dtype=torch.bfloat16, device=xq.device)
    _check_dtype(y, (torch.bfloat16,), "y")
    _lib.check(_lib.lib().moe_fp8_dense_forward(ctypes.byref(dw.desc), _ptr(xq), _ptr(xs), T, _ptr(y),
                                                flags, _stream(xq)), "moe_fp8_dense_forward")
    return y


def dense_layer(dw: DenseWeights, x: torch.Tensor, flags: int = 0):
    """bf16 x [T, K] -> MXFP8 (moe_quant_act_mxfp8) -> y [T, N] bf16."""
    xq, xs = quant_act_mxfp8(x)
    return dense_forward(dw, xq, xs, flags)
