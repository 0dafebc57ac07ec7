"""The no-allocation entry point (moe_fp4_layer_forward_noalloc), through the
C ABI: its output equals moe_fp4_layer_forward's bit for bit on two calls in a
row, the second smaller than the first, on both expert paths; a shape whose
workspace exceeds the fixed scratch is rejected before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
from fp4_routed_expert_amd import _lib
from gpu_cases import get_case, log

pytestmark = pytest.mark.gpu


def _noalloc(pw, x, logits, k, flags, y):
    return _lib.lib().moe_fp4_layer_forward_noalloc(
        ctypes.byref(pw.desc), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(logits.data_ptr()),
        x.shape[0], k, ctypes.c_void_p(y.data_ptr()), flags,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("name,T2", [("c1", 3), ("c2", 17)])
@pytest.mark.parametrize("flags", [0, moe.MOE_FLAG_FORCE_DECODE, moe.MOE_FLAG_FORCE_PREFILL],
                         ids=["auto", "decode", "prefill"])
def test_noalloc_equals_layer_forward_two_calls(name, T2, flags, dev):
    c = get_case(name, dev)
    k, H = c.sh.k, c.sh.H
    for T in (c.sh.T, T2):                      # the second call is smaller
        x = c.x[:T].contiguous()
        lg = c.logits[:T].contiguous()
        y_ref = moe.layer_forward(c.pw, x, lg, k, flags)
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
        rc = _noalloc(c.pw, x, lg, k, flags, y)
        torch.cuda.synchronize()
        log(f"[noalloc/{name}/T{T}/f{flags}] rc={rc}")
        assert rc == _lib.MOE_OK, _lib.status_string(rc)
        assert torch.equal(y, y_ref), f"{name} T={T}: differs from moe_fp4_layer_forward"


def test_noalloc_rejects_shapes_beyond_the_scratch(dev):
    c = get_case("c2", dev)
    k, H, E, I = c.sh.k, c.sh.H, c.sh.E, c.sh.I
    T = 4096                                  # its layer workspace is far beyond 64 MiB
    assert moe.layer_workspace_size(T, E, k, H, I) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    lg = torch.zeros((T, E), dtype=torch.float32, device=dev)
    y = torch.full((T, H), 7.0, dtype=torch.float32, device=dev)
    rc = _noalloc(c.pw, x, lg, k, 0, y)
    torch.cuda.synchronize()
    assert rc == _lib.MOE_ERR_WORKSPACE
    assert bool((y == 7.0).all()), "a rejected call wrote its output"
