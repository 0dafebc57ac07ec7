"""ctypes declarations of libmoe_fp4.so (the C ABI in include/moe_fp4.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "libmoe_fp4.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe_fp4.h")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_FLAG_FORCE_DECODE = 1
MOE_FLAG_FORCE_PREFILL = 2
MOE_FP4_LAYOUT_VERSION = 1
MOE_FP8_DENSE_LAYOUT_VERSION = 1
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeFp4Weights(ctypes.Structure):
    _fields_ = [
        ("E", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("layout_version", ctypes.c_uint32),
        ("packed", ctypes.c_void_p),
        ("packed_bytes", ctypes.c_size_t),
    ]


class MoeFp8DenseWeights(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("layout_version", ctypes.c_uint32),
        ("packed", ctypes.c_void_p),
        ("packed_bytes", ctypes.c_size_t),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (hip error {last_hip_error()})")


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
_WP = ctypes.POINTER(MoeFp4Weights)
_DP = ctypes.POINTER(MoeFp8DenseWeights)

SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_hip_error": (ctypes.c_int, []),
    "moe_route_topk": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_sort_permute_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "moe_sort_permute": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_quant_act_mxfp8": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P]),
    "moe_fp4_packed_weight_bytes": (_SZ, [_I32, _I32, _I32]),
    "moe_fp4_prepack_weights": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _SZ,
                                               _WP, _P]),
    "moe_fp4_stage_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "moe_fp4_expert_up": (ctypes.c_int, [_WP, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _SZ, _U32, _P]),
    "moe_fp4_expert_down": (ctypes.c_int, [_WP, _P, _P, _P, _I32, _I32, _P, _P, _SZ, _U32, _P]),
    "moe_combine": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "moe_fp4_forward_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _U32]),
    "moe_fp4_grouped_forward": (ctypes.c_int, [_WP, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _SZ,
                                               _U32, _P]),
    "moe_fp4_layer_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _U32]),
    "moe_fp4_layer_forward": (ctypes.c_int, [_WP, _P, _P, _I32, _I32, _P, _P, _SZ, _U32, _P]),
    "moe_fp4_layer_forward_noalloc": (ctypes.c_int, [_WP, _P, _P, _I32, _I32, _P, _U32, _P]),
    "moe_router_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "moe_router_logits": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "moe_fp4_shared_workspace_size": (_SZ, [_I32, _I32, _I32, _U32]),
    "moe_fp4_shared_expert": (ctypes.c_int, [_WP, _P, _P, _I32, _P, _P, _SZ, _U32, _P]),
    "moe_combine_shared": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "moe_fp4_layer_full_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _U32]),
    "moe_fp4_layer_forward_full": (ctypes.c_int, [_WP, _I32, _P, _P, _I32, _I32, _P, _P, _SZ, _U32,
                                                  _P]),
    "moe_fp8_dense_packed_bytes": (_SZ, [_I32, _I32]),
    "moe_fp8_dense_prepack": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _SZ, _DP, _P]),
    "moe_fp8_dense_forward": (ctypes.c_int, [_DP, _P, _P, _I32, _P, _U32, _P]),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise RuntimeError(
                f"{SO_PATH} is not built; run `python -m fp4_routed_expert_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(SO_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def last_hip_error() -> int:
    return int(lib().moe_last_hip_error())


def check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, what)
