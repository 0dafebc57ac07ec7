"""Helpers shared by the GPU tests: seeded cases on the device, the oracle's
expected values, the packed-layout reader, and the output tolerance check."""
from __future__ import annotations

import hashlib
import sys

import numpy as np
import torch

import fp4_routed_expert_amd as moe
import oracle
import synth


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def sha(a) -> str:
    if isinstance(a, torch.Tensor):
        a = a.cpu().numpy()
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


class Case:
    """One seeded layer on the device plus its oracle integer results."""

    def __init__(self, inp: synth.LayerInputs, dev, with_weights=True):
        self.inp = inp
        self.sh = inp.shape
        self.dev = dev
        self.x = to_dev(inp.x.view(np.int16), dev).view(torch.bfloat16)
        self.logits = to_dev(inp.logits, dev)
        self.pw = None
        if with_weights:
            w = [to_dev(getattr(inp, n), dev) for n in ("w1", "s1", "w3", "s3", "w2", "s2")]
            self.pw = moe.prepack_weights(*w)
            torch.cuda.synchronize()
            del w
        # oracle integer parts (cheap at every size)
        self.ids, self.gates = oracle.route(inp.logits, self.sh.k)
        self.counts, self.offsets, self.sorted_pair, self.pair_pos = oracle.sort(self.ids, self.sh.E)
        self.xq, self.xs = oracle.quant_mxfp8_bf16(inp.x)


_cache: dict = {}


def get_case(name_or_shape, dev, probe_w2=False, with_weights=True, **over) -> Case:
    key = (name_or_shape, probe_w2, with_weights, tuple(sorted(over.items())))
    if key not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        log(f"[case] building {key}")
        inp = synth.make_inputs(name_or_shape, probe_w2=probe_w2, with_weights=with_weights, **over)
        _cache[key] = Case(inp, dev, with_weights)
    return _cache[key]


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid])).astype(np.int32)


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "y"):
    """max|err| <= 1e-2 * max|ref| and cosine >= 0.9999 (fp32 outputs)."""
    g = y_gpu.astype(np.float64).ravel()
    r = y_ref.astype(np.float64).ravel()
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - r).max()
    ref = np.abs(r).max()
    cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r) + 1e-300))
    log(f"[{what}] max_err={err:.3e} max_ref={ref:.3e} ratio={err / max(ref, 1e-300):.3e} cos={cos:.7f}")
    assert err <= 1e-2 * ref, f"{what}: max|err| {err} > 1e-2 * {ref}"
    assert cos >= 0.9999, f"{what}: cosine {cos}"
    return err / max(ref, 1e-300), cos


def _a256(x: int) -> int:
    return (x + 255) & ~255


def unpack_layout(packed: np.ndarray, E: int, H: int, I: int):
    """Read the packed tile layout back into canonical w1, s1, w3, s3, w2, s2.

    Layout as documented with the kernels: 1 KiB MFMA B tiles (lane l holds
    row l%16 and the 32 K elements of block l//16 as 16 bytes); gate/up blocks
    of 4 tiles [W1 rows 0-15, W1 rows 16-31, W3 rows 0-15, W3 rows 16-31] per
    (expert, 32-row group, K-step of 128), then per (expert, group, K-step) one
    scale dword per lane (byte t = tile t); down blocks of 2 tiles and one
    16-bit scale pair per lane."""
    J, J2 = H // 128, I // 128
    QT, QT2 = I // 32, H // 32
    upw = E * QT * J * 4096
    ups = E * QT * J * 256
    dnw = E * QT2 * J2 * 2048
    dns = E * QT2 * J2 * 128
    o_ups = _a256(upw)
    o_dnw = _a256(o_ups + ups)
    o_dns = _a256(o_dnw + dnw)
    a = packed[:upw].reshape(E, QT, J, 4, 4, 16, 16)          # e q j t lg lr b
    w13 = a.transpose(0, 3, 1, 5, 2, 4, 6)                     # e t q lr j lg b
    w1 = w13[:, 0:2].transpose(0, 2, 1, 3, 4, 5, 6).reshape(E, I, H // 2)
    w3 = w13[:, 2:4].transpose(0, 2, 1, 3, 4, 5, 6).reshape(E, I, H // 2)
    s = packed[o_ups:o_ups + ups].reshape(E, QT, J, 4, 16, 4)   # e q j lg lr t
    s13 = s.transpose(0, 5, 1, 4, 2, 3)                          # e t q lr j lg
    s1 = s13[:, 0:2].transpose(0, 2, 1, 3, 4, 5).reshape(E, I, H // 32)
    s3 = s13[:, 2:4].transpose(0, 2, 1, 3, 4, 5).reshape(E, I, H // 32)
    d = packed[o_dnw:o_dnw + dnw].reshape(E, QT2, J2, 2, 4, 16, 16)  # e q2 j2 t lg lr b
    w2 = d.transpose(0, 1, 3, 5, 2, 4, 6).reshape(E, H, I // 2)
    ds = packed[o_dns:o_dns + dns].reshape(E, QT2, J2, 4, 16, 2)     # e q2 j2 lg lr t
    s2 = ds.transpose(0, 1, 5, 4, 2, 3).reshape(E, H, I // 32)
    return tuple(np.ascontiguousarray(v) for v in (w1, s1, w3, s3, w2, s2))
