"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments before it touches the GPU (no device
here: every case below must return its error code without a HIP call)."""
import ctypes
import os
import re

import pytest

from fp4_routed_expert_amd import _lib

L = None


def setup_module():
    global L
    if not os.path.exists(_lib.SO_PATH):
        from fp4_routed_expert_amd import build
        build.build()
    L = _lib.lib()


def declared_functions():
    text = open(_lib.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) == 27, names
    so = ctypes.CDLL(_lib.SO_PATH)
    for n in names:
        assert hasattr(so, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings():
    assert _lib.status_string(0) == "MOE_OK"
    assert _lib.status_string(3) == "MOE_ERR_WORKSPACE"
    assert L.moe_last_hip_error() == 0


A = ctypes.c_void_p(1 << 20)        # 256-aligned stand-ins: never dereferenced on error paths
MIS = ctypes.c_void_p((1 << 20) + 4)
NUL = ctypes.c_void_p(0)
INV, UNS, WSE = _lib.MOE_ERR_INVALID_ARGUMENT, _lib.MOE_ERR_UNSUPPORTED, _lib.MOE_ERR_WORKSPACE


def test_route_argument_errors():
    assert L.moe_route_topk(A, -1, 8, 2, A, A, NUL) == INV
    assert L.moe_route_topk(A, 4, 0, 1, A, A, NUL) == INV
    assert L.moe_route_topk(A, 4, 8, 0, A, A, NUL) == INV
    assert L.moe_route_topk(A, 4, 8, 9, A, A, NUL) == UNS        # k > E
    assert L.moe_route_topk(A, 4, 1025, 2, A, A, NUL) == UNS     # E > 1024
    assert L.moe_route_topk(A, 4, 64, 33, A, A, NUL) == UNS      # k > 32
    assert L.moe_route_topk(NUL, 4, 8, 2, A, A, NUL) == INV
    assert L.moe_route_topk(A, 0, 8, 2, NUL, NUL, NUL) == 0       # T = 0: no-op
    assert L.moe_route_topk(A, 1 << 27, 64, 16, A, A, NUL) == UNS  # T*k >= 2^31


def test_sort_argument_errors():
    assert L.moe_sort_permute_workspace_size(16, 8, 2) == 0       # one workgroup: no workspace
    need = L.moe_sort_permute_workspace_size(16384, 256, 8)
    assert need == 64 * 256 * 4                                  # 64 chunks of 2048 pairs
    assert L.moe_sort_permute(A, 16384, 256, 8, A, A, A, A, A, need - 1, NUL) == WSE
    assert L.moe_sort_permute(A, 16384, 256, 8, A, A, A, A, NUL, need, NUL) == WSE
    assert L.moe_sort_permute(A, 16384, 256, 8, A, A, A, A, MIS, need, NUL) == INV
    assert L.moe_sort_permute(A, 4, 8, 2, NUL, A, A, A, NUL, 0, NUL) == INV


def test_quant_argument_errors():
    assert L.moe_quant_act_mxfp8(A, 4, 48, A, A, NUL) == UNS       # K % 32
    assert L.moe_quant_act_mxfp8(A, -1, 64, A, A, NUL) == INV
    assert L.moe_quant_act_mxfp8(MIS, 4, 64, A, A, NUL) == INV
    assert L.moe_quant_act_mxfp8(A, 0, 64, NUL, NUL, NUL) == 0


def test_packed_bytes_and_prepack_errors():
    nb = L.moe_fp4_packed_weight_bytes(256, 7168, 2048)
    nibbles = 256 * 3 * 7168 * 2048 // 2
    scales = 256 * 3 * 7168 * 2048 // 32
    assert nibbles + scales <= nb <= nibbles + scales + (1 << 20)
    assert L.moe_fp4_packed_weight_bytes(8, 200, 128) == 0        # H % 128
    desc = _lib.MoeFp4Weights()
    nb0 = L.moe_fp4_packed_weight_bytes(8, 256, 128)
    assert L.moe_fp4_prepack_weights(A, A, A, A, A, A, 8, 256, 96, A, nb0, ctypes.byref(desc), NUL) == UNS
    assert L.moe_fp4_prepack_weights(A, A, A, A, A, A, 8, 256, 128, A, nb0 - 1, ctypes.byref(desc), NUL) == INV
    assert L.moe_fp4_prepack_weights(A, A, A, A, A, A, 8, 256, 128, MIS, nb0, ctypes.byref(desc), NUL) == INV
    assert L.moe_fp4_prepack_weights(A, A, A, A, A, A, 0, 256, 128, A, nb0, ctypes.byref(desc), NUL) == INV


def _desc(E=8, H=256, I=128, version=1):
    d = _lib.MoeFp4Weights()
    d.E, d.H, d.I, d.layout_version = E, H, I, version
    d.packed = 1 << 20
    d.packed_bytes = L.moe_fp4_packed_weight_bytes(E, H, I)
    return d


def test_forward_argument_errors():
    d = _desc()
    ws = L.moe_fp4_forward_workspace_size(16, 8, 2, 256, 128, 0)
    assert ws >= 32 * 128 + 32 * 4 + 32 * 256 * 2   # hq, hs and the bf16 expert outputs O
    fwd = L.moe_fp4_grouped_forward
    assert fwd(ctypes.byref(_desc(version=7)), A, A, A, A, A, A, 16, 2, A, A, ws, 0, NUL) == INV
    assert fwd(ctypes.byref(d), A, A, A, A, A, A, 16, 2, A, A, ws, 3, NUL) == INV  # both paths forced
    assert fwd(ctypes.byref(d), A, A, A, A, A, A, 16, 2, A, A, ws - 1, 0, NUL) == WSE
    assert fwd(ctypes.byref(d), A, A, A, A, A, A, 16, 9, A, A, ws, 0, NUL) == UNS  # k > E
    assert fwd(ctypes.byref(d), NUL, A, A, A, A, A, 16, 2, A, A, ws, 0, NUL) == INV
    assert fwd(ctypes.byref(d), A, A, A, A, A, A, 0, 2, A, A, 0, 0, NUL) == 0      # T = 0
    small = _desc()
    small.packed_bytes -= 1
    assert fwd(ctypes.byref(small), A, A, A, A, A, A, 16, 2, A, A, ws, 0, NUL) == INV
    up = L.moe_fp4_expert_up
    sws = L.moe_fp4_stage_workspace_size(16, 8, 2, 256, 128)
    assert sws >= 32 * (256 // 128) * 4          # the activation scales by K-step
    assert L.moe_fp4_stage_workspace_size(16, 8, 2, 200, 128) == 0
    assert up(ctypes.byref(d), A, A, A, A, 16, 2, A, A, A, sws - 1, 0, NUL) == WSE
    big = _desc(E=8, H=1 << 20, I=128)
    bws = L.moe_fp4_stage_workspace_size(4096, 8, 2, 1 << 20, 128)
    assert up(ctypes.byref(big), A, A, A, A, 4096, 2, A, A, A, bws, 2, NUL) == UNS  # T*H >= 2^32, prefill
    assert L.moe_combine(A, A, A, 4, 2, 250, A, NUL) == UNS       # H % 4
    assert L.moe_combine(A, A, A, 4, 0, 256, A, NUL) == INV


def test_layer_forward_argument_errors():
    d = _desc()
    need = L.moe_fp4_layer_workspace_size(16, 8, 2, 256, 128, 0)
    # holds at least the forward workspace plus ids, gates, sort arrays and MXFP8 x
    assert need >= L.moe_fp4_forward_workspace_size(16, 8, 2, 256, 128, 0) + 16 * 256
    assert L.moe_fp4_layer_workspace_size(16, 8, 9, 256, 128, 0) == 0   # k > E
    lf = L.moe_fp4_layer_forward
    assert lf(ctypes.byref(d), A, A, 16, 2, A, A, need - 1, 0, NUL) == WSE
    assert lf(ctypes.byref(d), A, A, 16, 2, A, NUL, need, 0, NUL) == WSE
    assert lf(ctypes.byref(d), A, A, 16, 2, A, MIS, need, 0, NUL) == INV
    assert lf(ctypes.byref(d), MIS, A, 16, 2, A, A, need, 0, NUL) == INV   # x not 16-aligned
    assert lf(ctypes.byref(d), A, NUL, 16, 2, A, A, need, 0, NUL) == INV
    assert lf(ctypes.byref(d), A, A, 16, 2, A, A, need, 3, NUL) == INV     # both paths forced
    assert lf(ctypes.byref(d), A, A, 16, 40, A, A, need, 0, NUL) == UNS    # k > 32
    assert lf(ctypes.byref(_desc(version=2)), A, A, 16, 2, A, A, need, 0, NUL) == INV
    assert lf(ctypes.byref(d), NUL, NUL, 0, 2, NUL, NUL, 0, 0, NUL) == 0  # T = 0


def test_router_and_shared_argument_errors():
    rl = L.moe_router_logits
    rws = L.moe_router_workspace_size(8, 4096, 64)
    # decode: the K range is split into slices whose fp32 partial sums live in the workspace
    assert rws >= 2 * 8 * 64 * 4 and rws % (8 * 64 * 4) == 0
    # 128 output tiles of 128 x 256 fill half the chip: two K slices
    assert L.moe_router_workspace_size(16384, 7168, 256) == 2 * 16384 * 256 * 4
    assert L.moe_router_workspace_size(4096, 256, 1024) == 0     # K too short to split
    assert L.moe_router_workspace_size(8, 200, 64) == 0         # unsupported H
    assert rl(A, A, 4, 200, 8, A, A, 1 << 20, NUL) == UNS          # H % 128
    assert rl(A, A, 4, 256, 1025, A, A, 1 << 20, NUL) == UNS       # E > 1024
    assert rl(A, A, -1, 256, 8, A, A, 1 << 20, NUL) == INV
    assert rl(A, A, 4, 256, 0, A, A, 1 << 20, NUL) == INV
    assert rl(MIS, A, 4, 256, 8, A, A, 1 << 20, NUL) == INV        # x not 16-aligned
    assert rl(A, NUL, 4, 256, 8, A, A, 1 << 20, NUL) == INV
    assert rl(A, A, 8, 4096, 64, A, A, rws - 1, NUL) == WSE
    assert rl(A, A, 8, 4096, 64, A, NUL, rws, NUL) == WSE
    assert rl(A, A, 8, 4096, 64, A, MIS, rws, NUL) == INV
    assert rl(NUL, NUL, 0, 256, 8, NUL, NUL, 0, NUL) == 0          # T = 0
    d1 = _desc(E=1, I=256)
    sws = L.moe_fp4_shared_workspace_size(16, 256, 256, 0)
    # identity routing, h (MXFP8) of the shared intermediate size and the stage workspace
    assert sws >= 16 * 256 + 16 * 8 + L.moe_fp4_stage_workspace_size(16, 1, 1, 256, 256)
    se = L.moe_fp4_shared_expert
    assert se(ctypes.byref(_desc(E=2)), A, A, 16, A, A, sws, 0, NUL) == INV   # E != 1
    assert se(ctypes.byref(d1), A, A, 16, A, A, sws - 1, 0, NUL) == WSE
    assert se(ctypes.byref(d1), A, A, 16, A, MIS, sws, 0, NUL) == INV
    assert se(ctypes.byref(d1), A, A, 16, NUL, A, sws, 0, NUL) == INV
    assert se(ctypes.byref(d1), A, A, 16, A, A, sws, 3, NUL) == INV           # both paths forced
    assert se(ctypes.byref(d1), NUL, NUL, 0, NUL, NUL, 0, 0, NUL) == 0      # T = 0: no-op
    cs = L.moe_combine_shared
    assert cs(A, A, A, NUL, 4, 2, 256, A, NUL) == INV                        # no shared output
    assert cs(A, A, A, A, 4, 2, 250, A, NUL) == UNS                          # H % 4
    assert cs(A, A, A, MIS, 4, 2, 256, A, NUL) == INV                        # not 8-aligned
    assert cs(A, A, A, A, 4, 2, 256, MIS, NUL) == INV                        # y not 16-aligned
    d = _desc()                    # 8 experts
    full = L.moe_fp4_layer_full_workspace_size
    n0 = full(16, 8, 2, 256, 128, 0, 0)
    n1 = full(16, 8, 2, 256, 128, 1, 0)   # 7 routed + 1 shared: 3 slots per token
    assert n0 >= (L.moe_fp4_layer_workspace_size(16, 8, 2, 256, 128, 0)
                  + L.moe_router_workspace_size(16, 256, 8))                  # + router planes
    assert n1 >= L.moe_fp4_layer_workspace_size(16, 8, 3, 256, 128, 0)
    assert full(16, 8, 2, 256, 128, 8, 0) == 0          # no routed expert left
    assert full(16, 8, 2, 256, 128, -1, 0) == 0
    assert full(16, 8, 8, 256, 128, 1, 0) == 0          # k > routed experts
    assert full(16, 64, 30, 256, 128, 3, 0) == 0        # k + n_shared > 32
    lf = L.moe_fp4_layer_forward_full
    assert lf(ctypes.byref(d), 0, A, A, 16, 2, A, A, n0 - 1, 0, NUL) == WSE
    assert n1 > n0
    assert lf(ctypes.byref(d), 1, A, A, 16, 2, A, A, n1 - 1, 0, NUL) == WSE   # the shared slot's rows
    assert lf(ctypes.byref(d), 8, A, A, 16, 2, A, A, n1, 0, NUL) == INV       # n_shared >= E
    assert lf(ctypes.byref(d), -1, A, A, 16, 2, A, A, n1, 0, NUL) == INV
    assert lf(ctypes.byref(d), 1, A, A, 16, 8, A, A, n1, 0, NUL) == UNS       # k > E - n_shared
    assert lf(ctypes.byref(d), 0, NUL, A, 16, 2, A, A, n0, 0, NUL) == INV     # no router weights
    assert lf(ctypes.byref(d), 0, MIS, A, 16, 2, A, A, n0, 0, NUL) == INV
    assert lf(ctypes.byref(d), 0, A, A, 16, 2, A, A, n0, 3, NUL) == INV       # both paths forced
    assert lf(ctypes.byref(d), 0, NUL, NUL, 0, 2, NUL, NUL, 0, 0, NUL) == 0   # T = 0


def test_dense_argument_errors():
    nb = L.moe_fp8_dense_packed_bytes(7168, 16384)
    assert 7168 * 16384 * (1 + 1 / 32) <= nb <= 7168 * 16384 * (1 + 1 / 32) + 512
    assert L.moe_fp8_dense_packed_bytes(112, 256) == 0         # N % 32
    assert L.moe_fp8_dense_packed_bytes(96, 200) == 0          # K % 128
    d = _lib.MoeFp8DenseWeights()
    pre = L.moe_fp8_dense_prepack
    nb0 = L.moe_fp8_dense_packed_bytes(96, 256)
    assert pre(A, A, 96, 200, A, nb0, ctypes.byref(d), NUL) == UNS
    assert pre(A, A, 96, 256, A, nb0 - 1, ctypes.byref(d), NUL) == INV
    assert pre(A, A, 96, 256, MIS, nb0, ctypes.byref(d), NUL) == INV
    assert pre(MIS, A, 96, 256, A, nb0, ctypes.byref(d), NUL) == INV
    assert pre(A, A, 0, 256, A, nb0, ctypes.byref(d), NUL) == INV
    d.N, d.K, d.layout_version, d.packed, d.packed_bytes = 96, 256, 1, 1 << 20, nb0
    fw = L.moe_fp8_dense_forward
    assert fw(ctypes.byref(d), A, A, 0, NUL, 0, NUL) == 0            # T = 0
    assert fw(ctypes.byref(d), A, A, -1, A, 0, NUL) == INV
    assert fw(ctypes.byref(d), A, A, 4, A, 3, NUL) == INV            # both paths forced
    assert fw(ctypes.byref(d), MIS, A, 4, A, 0, NUL) == INV          # xq not 16-aligned
    assert fw(ctypes.byref(d), A, NUL, 4, A, 0, NUL) == INV
    big = _lib.MoeFp8DenseWeights()
    big.N, big.K, big.layout_version, big.packed = 96, 1 << 20, 1, 1 << 20
    big.packed_bytes = L.moe_fp8_dense_packed_bytes(96, 1 << 20)
    assert fw(ctypes.byref(big), A, A, 4096, A, 0, NUL) == UNS        # T * K >= 2^32
    d.layout_version = 2
    assert fw(ctypes.byref(d), A, A, 4, A, 0, NUL) == INV
    d.layout_version = 1
    d.packed_bytes = nb0 - 1
    assert fw(ctypes.byref(d), A, A, 4, A, 0, NUL) == INV


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "SO_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_noalloc_argument_errors():
    """The no-allocation layer rejects bad arguments and shapes beyond its fixed
    scratch before any HIP call (no device here)."""
    w = _lib.MoeFp4Weights(E=256, H=7168, I=2048, layout_version=_lib.MOE_FP4_LAYOUT_VERSION,
                           packed=A.value, packed_bytes=1 << 40)
    f = L.moe_fp4_layer_forward_noalloc
    wp = ctypes.byref(w)
    assert f(None, A, A, 8, 8, A, 0, NUL) == INV
    assert f(wp, NUL, A, 8, 8, A, 0, NUL) == INV
    assert f(wp, A, A, 8, 8, MIS, 0, NUL) == INV
    assert f(wp, A, A, 8, 8, A, 3, NUL) == INV                  # both paths forced
    assert f(wp, A, A, 8, 300, A, 0, NUL) == UNS                # k > 32
    assert f(wp, A, A, 0, 8, NUL, 0, NUL) == 0                  # T = 0: no-op
    assert L.moe_fp4_layer_workspace_size(477, 256, 8, 7168, 2048, 0) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    assert f(wp, A, A, 477, 8, A, 0, NUL) == WSE                # beyond the fixed scratch


def test_size_queries_take_t_e_k_order():
    """Every size query takes (T, E, k, ...), like moe_sort_permute_workspace_size:
    swapping E and k changes the answer (or makes the shape invalid)."""
    T, E, k, H, I = 64, 32, 4, 256, 128
    for f, extra in ((L.moe_fp4_stage_workspace_size, ()), (L.moe_fp4_forward_workspace_size, (0,)),
                     (L.moe_fp4_layer_workspace_size, (0,))):
        assert f(T, E, k, H, I, *extra) > 0
        assert f(T, k, E, H, I, *extra) == 0           # k = 32 > E = 4
    full = L.moe_fp4_layer_full_workspace_size
    assert full(T, E, k, H, I, 1, 0) > 0 and full(T, k, E, H, I, 1, 0) == 0
    assert L.moe_fp4_layer_workspace_size(T, E, k, H, I, 0) > L.moe_fp4_layer_workspace_size(T, E, 2, H, I, 0)
