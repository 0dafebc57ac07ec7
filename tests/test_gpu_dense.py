"""GPU parity of the FP8 dense projection, through the C ABI.

y (bf16) against the oracle's sums on the same MXFP8 rows, on both
paths (weight streaming and the LDS-tiled GEMM, in each of its tile
geometries: 128 x 128, 192 x 256, and 256 x 256 by LDS-DMA for even K-step
counts, taken by the fewest rounds of workgroups weighted by their round
times, and the smaller one's K range split over two wave groups when its
tiles are fewer than the CUs): the tiny workload, ragged
token counts, an odd K-step count (the tiled kernel's zero padding step),
weight-row counts that leave a partial 128-row tile, the decode-shaped and
prefill-shaped projections at full size (sampled tokens), plus the prepacked
layout read back bit for bit and a one-hot weight whose outputs are exact."""
import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import oracle
import synth
from gpu_cases import check_y, log, sample_tokens, to_dev

pytestmark = pytest.mark.gpu

DEC, PRE = moe.MOE_FLAG_FORCE_DECODE, moe.MOE_FLAG_FORCE_PREFILL


class DenseCase:
    def __init__(self, cfg, dev, **over):
        self.inp = synth.make_dense_inputs(cfg, **over)
        self.sh = self.inp.shape
        self.x = to_dev(self.inp.x.view(np.int16), dev).view(torch.bfloat16)
        self.dw = moe.dense_prepack(to_dev(self.inp.wq, dev), to_dev(self.inp.ws, dev))
        self.xq, self.xs = oracle.quant_mxfp8_bf16(self.inp.x)
        torch.cuda.synchronize()

    def ref(self, toks):
        return oracle.dense_fp8(self.xq, self.xs, self.inp.wq, self.inp.ws, toks)


_cache = {}


def get_dense(key, dev, **over):
    k = (key, tuple(sorted(over.items())))
    if k not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        log(f"[dense case] {k}")
        _cache[k] = DenseCase(key, dev, **over)
    return _cache[k]


SMALL = [
    ("d0", {}),                                   # T5 K256 N96
    ("d0", dict(T=37, K=384, N=160)),             # odd K-step count, partial row tile
    ("d0", dict(T=130, K=256, N=288)),            # two token tiles (ragged), three row tiles
    ("d0", dict(T=1, K=128, N=32)),               # smallest
    ("d0", dict(T=300, K=384, N=288)),            # ragged tokens and rows, odd K-steps (two K groups)
]


@pytest.mark.parametrize("cfg,over", SMALL, ids=["d0", "T37K384N160", "T130K256N288", "T1K128N32", "T300K384N288"])
@pytest.mark.parametrize("flags", [0, DEC, PRE], ids=["auto", "decode", "prefill"])
def test_dense_small(cfg, over, flags, dev):
    c = get_dense(cfg, dev, **over)
    log(f"[dense] {cfg} {over} flags={flags}")
    xq, xs = moe.quant_act_mxfp8(c.x)
    assert np.array_equal(xq.cpu().numpy(), c.xq) and np.array_equal(xs.cpu().numpy(), c.xs)
    y = moe.dense_forward(c.dw, xq, xs, flags)
    torch.cuda.synchronize()
    toks = np.arange(c.sh.T, dtype=np.int32)
    check_y(y.float().cpu().numpy(), c.ref(toks), f"dense/{over or cfg}/f{flags}")


@pytest.mark.parametrize("cfg,ntok", [("d1", 8), ("d3", 16)])
def test_dense_full_size(cfg, ntok, dev):
    c = get_dense(cfg, dev)
    log(f"[dense] {cfg} full size")
    y = moe.dense_layer(c.dw, c.x)
    y_other = moe.dense_layer(c.dw, c.x, PRE) if c.sh.T <= 96 else None   # the other path
    torch.cuda.synchronize()
    toks = sample_tokens(c.sh.T, ntok, seed=13)
    ref = c.ref(toks)
    check_y(y.float().cpu().numpy()[toks], ref, f"dense/{cfg}")
    if y_other is not None:
        check_y(y_other.float().cpu().numpy()[toks], ref, f"dense/{cfg}/other-path")
    y2 = moe.dense_layer(c.dw, c.x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_dense_prefill_full_size_every_token_against_streaming(dev):
    """d3 (T4604 K16384 N7168, the 256 x 256 LDS-DMA kernel): every token of
    the tiled GEMM against the weight-streaming kernel forced on the same rows
    (an independent kernel, fp32 sums in another order), plus sampled tokens
    of both against the oracle."""
    c = get_dense("d3", dev)
    log("[dense] d3 every token: LDS-DMA tiles against forced streaming")
    xq, xs = moe.quant_act_mxfp8(c.x)
    y = moe.dense_forward(c.dw, xq, xs)
    y_dec = moe.dense_forward(c.dw, xq, xs, DEC)
    torch.cuda.synchronize()
    check_y(y.float().cpu().numpy(), y_dec.float().cpu().numpy(), "dense/d3/tiled-vs-streaming")
    toks = np.unique(np.concatenate([sample_tokens(c.sh.T, 8, seed=17), np.arange(4600, 4604)])).astype(np.int32)
    ref = c.ref(toks)
    check_y(y_dec.float().cpu().numpy()[toks], ref, "dense/d3/streaming")


def test_dense_large_tile_geometry(dev):
    """1300 tokens x 7136 rows: the 128 x 128 tiles would need two rounds of
    workgroups on 256 CUs and the 192 x 256 tiles one, so the larger geometry
    runs -- ragged in tokens (1300 = 6 x 192 + 148) and rows (7136 = 27 x 256 +
    224), with an odd K-step count; sampled tokens plus the ragged tail."""
    c = get_dense("d0", dev, T=1300, K=384, N=7136)
    log("[dense] large-tile geometry T1300 K384 N7136")
    xq, xs = moe.quant_act_mxfp8(c.x)
    y = moe.dense_forward(c.dw, xq, xs, PRE)
    y_auto = moe.dense_forward(c.dw, xq, xs)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_auto.view(torch.int16))
    toks = np.unique(np.concatenate([sample_tokens(c.sh.T, 40, seed=5), np.arange(1290, 1300)])).astype(np.int32)
    check_y(y.float().cpu().numpy()[toks], c.ref(toks), "dense/large-geometry")


@pytest.mark.parametrize("K", [256, 1024, 2304])
def test_dense_lds_dma_geometry(K, dev):
    """2100 tokens x 4064 rows: 9 x 16 tiles of 256 x 256 fit one round on 256
    CUs, where the 128 x 128 tiles would need two, so the LDS-DMA kernel runs
    (K-step counts 2, 8 and 18: one, four and nine pairs of steps) -- ragged in
    tokens (2100 = 8 x 256 + 52) and rows (4064 = 15 x 256 + 224, the last
    tile's top weight pair re-reading the last one); every token against the
    oracle, and the same bits run to run."""
    c = get_dense("d0", dev, T=2100, K=K, N=4064)
    log(f"[dense] LDS-DMA geometry T2100 K{K} N4064")
    xq, xs = moe.quant_act_mxfp8(c.x)
    y = moe.dense_forward(c.dw, xq, xs)
    y2 = moe.dense_forward(c.dw, xq, xs, PRE)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    toks = np.arange(c.sh.T, dtype=np.int32)
    check_y(y.float().cpu().numpy(), c.ref(toks), f"dense/lds-dma/K{K}")


def test_dense_small_tile_unsplit(dev):
    """1100 tokens x 4096 rows: 288 small tiles, more than the CUs, so each
    runs its whole K range (two share a CU) -- the unsplit small geometry,
    ragged tokens, odd K-step count; the tiles below take two K groups."""
    c = get_dense("d0", dev, T=1100, K=384, N=4096)
    log("[dense] small tile, unsplit: T1100 K384 N4096")
    xq, xs = moe.quant_act_mxfp8(c.x)
    y = moe.dense_forward(c.dw, xq, xs, PRE)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([sample_tokens(c.sh.T, 40, seed=6), np.arange(1090, 1100)])).astype(np.int32)
    check_y(y.float().cpu().numpy()[toks], c.ref(toks), "dense/small-unsplit")


def _unpack(packed: np.ndarray, N: int, K: int):
    """Read the packed layout back: per 32-row group and K-step, 2 tiles of 2 KiB
    (lane l = 16 g + r: row r, K [16 g, +16) then K [64 + 16 g, +16)), then the
    scales, 64 bytes per tile in the same grouping."""
    J = K // 128
    ng = N // 32
    tiles = packed[:ng * J * 4096].reshape(ng, J, 2, 2, 4, 16, 16)   # grp j tile half g r byte
    s_off = (ng * J * 4096 + 255) // 256 * 256
    sc = packed[s_off:s_off + ng * J * 128].reshape(ng, J, 2, 4, 16)   # grp j tile g r
    wq = np.empty((N, K), dtype=np.uint8)
    w4 = wq.reshape(ng, 2, 16, K)                                      # grp tile r K
    for half in range(2):
        for g in range(4):
            cols = np.arange(J)[:, None] * 128 + 64 * half + 16 * g + np.arange(16)[None, :]
            w4[:, :, :, cols] = tiles[:, :, :, half, g].transpose(0, 2, 3, 1, 4)   # grp tile r j byte
    ws = sc.transpose(0, 2, 4, 1, 3).reshape(N, K // 32)               # grp tile r j g
    return wq, ws


def test_dense_prepack_roundtrip(dev):
    c = get_dense("d0", dev, T=3, K=384, N=64)
    wq, ws = _unpack(c.dw.buffer.cpu().numpy(), 64, 384)
    assert np.array_equal(wq, c.inp.wq)
    assert np.array_equal(ws, c.inp.ws)


@pytest.mark.parametrize("flags", [DEC, PRE], ids=["decode", "prefill"])
def test_dense_one_hot_is_exact(flags, dev):
    T, K, N = 40, 384, 96
    inp = synth.make_dense_inputs("d0", T=T, K=K, N=N)
    wq = np.zeros((N, K), dtype=np.uint8)
    cols = (13 * np.arange(N) + 7) % K
    wq[np.arange(N), cols] = 0x38                       # +1.0
    ws = np.full((N, K // 32), 127, dtype=np.uint8)     # 2^0
    dw = moe.dense_prepack(to_dev(wq, dev), to_dev(ws, dev))
    x = to_dev(inp.x.view(np.int16), dev).view(torch.bfloat16)
    y = moe.dense_layer(dw, x, flags).float().cpu().numpy()
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    want = oracle.decode_mxfp8(xq, xs)[:, cols]         # 4 significant bits: exact in bf16
    assert np.array_equal(y, want.astype(np.float32))


@pytest.mark.parametrize("T", [17, 33, 96])
def test_dense_streaming_two_token_tiles_long_k(T, dev):
    """The weight-streaming kernel from 17 tokens takes two 16-token tiles per
    pass over the weights; with K = 8192 (64 K-steps, more than its 16 waves)
    every wave runs whole batches of its K loop, with a ragged (T = 17, 33) or
    full (T = 96) second tile.  All tokens against the oracle and against the
    tiled GEMM."""
    c = get_dense("d0", dev, T=T, K=8192, N=256)
    log(f"[dense] streaming, two token tiles, T{T} K8192 N256")
    xq, xs = moe.quant_act_mxfp8(c.x)
    y = moe.dense_forward(c.dw, xq, xs)            # the default path: streaming up to T = 96
    y_pre = moe.dense_forward(c.dw, xq, xs, PRE)
    torch.cuda.synchronize()
    toks = np.arange(T, dtype=np.int32)
    ref = c.ref(toks)
    check_y(y.float().cpu().numpy(), ref, f"dense/stream2/T{T}")
    check_y(y.float().cpu().numpy(), y_pre.float().cpu().numpy(), f"dense/stream2-vs-tiled/T{T}")
