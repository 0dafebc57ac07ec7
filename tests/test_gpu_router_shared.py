"""GPU parity of the router GEMM and the shared expert, through the C ABI.

* Router logits (bf16 x . bf16 Wg, fp32 accumulation on the matrix cores)
  against the oracle's exact fp64 sums: every logit within the fp32 error
  bound gamma_n * sum_h |x_h * Wg_h| (n = H plus a few), on decode shapes
  (many K slices), prefill shapes, ragged token and expert counts, shapes
  with no K split, and the full-size router of the large prefill workload on
  sampled tokens.
* The shared expert stage call: its bf16 output against the oracle's
  single-expert steps, and bit for bit against the routed stage calls on a
  one-expert routing (the entry is those kernels with pair = token).
* The whole layer from hidden states, with shared experts packed after the
  routed ones: bit for bit equal to the chain of single-stage calls on the
  same slots, to the separately packed shared expert's stage call, and within
  tolerance of the oracle's layer with shared expert, routed on the same fp32
  logits the GPU produced (so that the integer routing decision is taken on
  identical values on both sides)."""
import dataclasses

import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import oracle
import synth
from gpu_cases import check_y, get_case, log, sample_tokens, to_dev

pytestmark = pytest.mark.gpu

# Unit roundoff for the bound: the matrix cores' internal rounding of their
# fp32 adds is not specified as round-to-nearest, so the bound uses 2^-23, the
# unit roundoff of a directed rounding, which covers either.
U32 = 2.0 ** -23


def _gamma(n: int) -> float:
    return n * U32 / (1 - n * U32)


def _bf16_dev(bits: np.ndarray, dev) -> torch.Tensor:
    return to_dev(bits.view(np.int16), dev).view(torch.bfloat16)


def _check_logits(lg: np.ndarray, x_bits: np.ndarray, wg_bits: np.ndarray, what: str):
    ref, absum = oracle.router_logits(x_bits, wg_bits)
    H = x_bits.shape[1]
    bound = _gamma(H + 4) * absum
    err = np.abs(lg.astype(np.float64) - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    log(f"[{what}] max_err={err.max():.3e} worst err/bound={worst:.3f}")
    assert np.isfinite(lg).all(), what
    assert (err <= bound).all(), f"{what}: error beyond the fp32 bound (worst ratio {worst})"


ROUTER_SHAPES = [
    # (T, H, E) with the number of K slices the library picks in brackets:
    (1, 128, 8),         # tiny, one K slice of 4 chunks [1]
    (8, 4096, 64),       # decode [8]
    (16, 256, 8),        # largest one-tile token count [1]
    (17, 256, 8),        # 64-row token tiles, 17 valid rows [2]
    (33, 512, 200),      # ragged tokens and experts [4]
    (300, 512, 16),      # LDS-tiled GEMM from T = 128 on [2]
    (777, 1536, 200),    # tiled, ragged tokens and experts [6]
    (64, 7168, 256),     # decode batch: the LDS-tiled GEMM from T = 17 when E >= 256 [28]
    (16, 7168, 256),     # decode, wide [16]
    (1000, 1024, 96),    # [4]
    (4096, 256, 1024),   # LDS-DMA GEMM (E >= 256), four expert tiles, no K split [1]
    (20, 256, 1024),     # the largest expert count, medium T: tiled, 8 expert tiles [1]
    (300, 128, 1000),    # LDS-DMA, ragged experts, two 64-K stages, no split [1]
    (300, 512, 256),     # LDS-DMA, ragged tokens [2]
    (777, 1536, 300),    # LDS-DMA, ragged tokens and experts, two expert tiles [6]
    (100, 7168, 256),    # tiled below T = 128 (E >= 256), ragged tokens [28]
    (48, 4096, 512),     # tiled below T = 128, four expert tiles [16]
    (129, 128, 256),     # LDS-DMA, one valid row in the second token tile [1]
]


@pytest.mark.parametrize("T,H,E", ROUTER_SHAPES, ids=lambda v: str(v))
def test_router_logits_within_fp32_bound(T, H, E, dev):
    sh = synth.Shape(T=T, H=H, I=128, E=E, k=1, seed=70 + T % 13)
    log(f"[router] T{T} H{H} E{E}")
    x_bits, _ = synth.make_activations(sh)
    wg_bits = synth.make_router_weights(sh)
    lg = moe.router_logits(_bf16_dev(x_bits, dev), _bf16_dev(wg_bits, dev))
    torch.cuda.synchronize()
    _check_logits(lg.cpu().numpy(), x_bits, wg_bits, f"router T{T} H{H} E{E}")


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_router_logits_full_prefill_size_sampled(name, dev):
    """The prefill workloads' routers on sampled tokens: T 4604 (7 K slices)
    and T 16384 (2 K slices), H 7168, E 256."""
    sh = synth.CONFIGS[name]
    log(f"[router] {name} sampled")
    x_bits, _ = synth.make_activations(sh)
    wg_bits = synth.make_router_weights(sh)
    lg = moe.router_logits(_bf16_dev(x_bits, dev), _bf16_dev(wg_bits, dev))
    torch.cuda.synchronize()
    toks = sample_tokens(sh.T, 48, seed=9)
    _check_logits(lg.cpu().numpy()[toks], x_bits[toks], wg_bits, f"router {name}")
    # repeatable: the same call gives the same bits
    lg2 = moe.router_logits(_bf16_dev(x_bits, dev), _bf16_dev(wg_bits, dev))
    torch.cuda.synchronize()
    assert torch.equal(lg.cpu(), lg2.cpu())


@pytest.mark.parametrize("T,H,E", [(40, 256, 24), (200, 512, 256)], ids=lambda v: str(v))
def test_router_one_hot_weights_return_the_activations(T, H, E, dev):
    """Wg rows with a single +1: each logit is one activation, exactly (the
    register-staged and the LDS-DMA kernels)."""
    sh = synth.Shape(T=T, H=H, I=128, E=E, k=1, seed=77)
    x_bits, _ = synth.make_activations(sh)
    wg = np.zeros((E, H), dtype=np.uint16)
    cols = (7 * np.arange(E) + 2) % H
    wg[np.arange(E), cols] = 0x3F80
    lg = moe.router_logits(_bf16_dev(x_bits, dev), _bf16_dev(wg, dev)).cpu().numpy()
    assert np.array_equal(lg, synth.bf16_bits_to_f32(x_bits)[:, cols])


def _shared_pw(sh, Is, dev):
    sw = synth.make_shared_weights(sh, I_shared=Is)
    pws = moe.prepack_weights(*[to_dev(a, dev) for a in sw])
    torch.cuda.synchronize()
    return sw, pws


SHARED_CASES = [
    ("c0", 128, 0),
    ("c1", 1536, 0),
    (synth.Shape(T=300, H=512, I=256, E=16, k=4, seed=53), 384, moe.MOE_FLAG_FORCE_PREFILL),
    (synth.Shape(T=300, H=512, I=256, E=16, k=4, seed=53), 384, moe.MOE_FLAG_FORCE_DECODE),
]


def _sid(v):
    return v if isinstance(v, str) else f"T{v.T}H{v.H}I{v.I}E{v.E}k{v.k}"


@pytest.mark.parametrize("shape,Is,flags", SHARED_CASES,
                         ids=[f"{_sid(s)}-Is{i}-f{f}" for s, i, f in SHARED_CASES])
def test_shared_expert_output(shape, Is, flags, dev):
    c = get_case(shape, dev)
    sh = c.sh
    log(f"[shared] {_sid(shape)} Is={Is} flags={flags}")
    sw, pws = _shared_pw(sh, Is, dev)
    xq, xs = moe.quant_act_mxfp8(c.x)
    Os = moe.shared_expert(pws, xq, xs, flags)
    # the same kernels through the stage calls on a one-expert routing
    offs = torch.tensor([0, sh.T], dtype=torch.int32, device=dev)
    ident = torch.arange(sh.T, dtype=torch.int32, device=dev)
    hq, hs = moe.expert_up(pws, xq, xs, offs, ident, sh.T, 1, flags)
    O1 = moe.expert_down(pws, hq, hs, offs, sh.T, 1, flags)
    torch.cuda.synchronize()
    assert torch.equal(Os.view(torch.int16), O1.view(torch.int16))
    toks = sample_tokens(sh.T, 16, seed=3)
    ref = np.empty((toks.size, sh.H))
    for n, t in enumerate(toks):
        G, U = oracle.expert_gate_up(c.xq[t], c.xs[t], sw[0][0], sw[1][0], sw[2][0], sw[3][0])
        _, hq_r, hs_r = oracle.swiglu_requant(G, U)
        ref[n] = oracle.expert_down(hq_r, hs_r, sw[4][0], sw[5][0])
    check_y(Os.float().cpu().numpy()[toks], ref, f"shared/{_sid(shape)}/Is{Is}")


def _with_shared(c, sws, dev):
    """Packed weights of the routed experts followed by the shared ones (E_r + ns experts)."""
    names = ("w1", "s1", "w3", "s3", "w2", "s2")
    cat = [np.concatenate([getattr(c.inp, n)] + [sw[i] for sw in sws], axis=0) for i, n in enumerate(names)]
    pw = moe.prepack_weights(*[to_dev(a, dev) for a in cat])
    torch.cuda.synchronize()
    return pw


def _shared_list(sh, ns):
    return [synth.make_shared_weights(sh if i == 0 else dataclasses.replace(sh, seed=sh.seed + 1000 * i))
            for i in range(ns)]


def _oracle_shared_rows(c, sw, toks):
    out = np.empty((toks.size, c.sh.H))
    for n, t in enumerate(toks):
        G, U = oracle.expert_gate_up(c.xq[t], c.xs[t], sw[0][0], sw[1][0], sw[2][0], sw[3][0])
        _, hq_r, hs_r = oracle.swiglu_requant(G, U)
        out[n] = oracle.expert_down(hq_r, hs_r, sw[4][0], sw[5][0])
    return out


FULL_CASES = [
    # (shape, shared experts, flags, sampled tokens)
    ("c0", 1, 0, 16),
    ("c1", 1, 0, 8),
    ("c1", 0, 0, 8),
    (synth.Shape(T=300, H=512, I=256, E=16, k=4, seed=53), 1, moe.MOE_FLAG_FORCE_PREFILL, 24),
    (synth.Shape(T=300, H=512, I=256, E=16, k=4, seed=53), 2, moe.MOE_FLAG_FORCE_DECODE, 24),
    (synth.Shape(T=40, H=256, I=128, E=8, k=2, seed=54), 1, moe.MOE_FLAG_FORCE_DECODE, 40),
    ("c3", 1, 0, 16),
]


@pytest.mark.parametrize("shape,ns,flags,ntok", FULL_CASES,
                         ids=[f"{_sid(s)}-ns{n}-f{f}" for s, n, f, _ in FULL_CASES])
def test_layer_full(shape, ns, flags, ntok, dev):
    c = get_case(shape, dev)
    sh = c.sh
    log(f"[full] {_sid(shape)} ns={ns} flags={flags}")
    wg = _bf16_dev(synth.make_router_weights(sh), dev)
    sws = _shared_list(sh, ns)
    pw = _with_shared(c, sws, dev) if ns else c.pw
    y = moe.layer_forward_full(pw, ns, wg, c.x, sh.k, flags)
    # the chain of single-stage calls on the same slots: routed top-k, then the shared ids
    lg = moe.router_logits(c.x, wg)
    ids, gates = moe.route_topk(lg, sh.k)
    if ns:
        sh_ids = torch.arange(sh.E, sh.E + ns, dtype=torch.int32, device=dev).expand(sh.T, ns)
        ids = torch.cat([ids, sh_ids], dim=1).contiguous()
        gates = torch.cat([gates, torch.ones((sh.T, ns), device=dev)], dim=1).contiguous()
    counts, offsets, sp, pp = moe.sort_permute(ids, sh.E + ns)
    xq, xs = moe.quant_act_mxfp8(c.x)
    y_chain = moe.grouped_forward(pw, xq, xs, gates, offsets, sp, pp, flags)
    torch.cuda.synchronize()
    assert torch.equal(y, y_chain)
    if ns == 1 and flags:
        # the separately packed shared expert through its own stage call: same kernels, same bits
        pws = moe.prepack_weights(*[to_dev(a, dev) for a in sws[0]])
        ids_r, gates_r = moe.route_topk(lg, sh.k)
        _, off_r, sp_r, pp_r = moe.sort_permute(ids_r, sh.E)
        hq, hs = moe.expert_up(c.pw, xq, xs, off_r, sp_r, sh.T, sh.k, flags)
        O = moe.expert_down(c.pw, hq, hs, off_r, sh.T, sh.k, flags)
        Os = moe.shared_expert(pws, xq, xs, flags)
        y_sep = moe.combine_shared(O, gates_r, pp_r, Os, sh.T, sh.k, sh.H)
        torch.cuda.synchronize()
        assert torch.equal(y, y_sep)
    lg_np = lg.cpu().numpy()
    toks = sample_tokens(sh.T, ntok, seed=11)
    ref = oracle.layer_tokens_shared(c.inp, lg_np, sws[0] if ns else None, tokens=toks).astype(np.float64)
    for sw in sws[1:]:
        ref += _oracle_shared_rows(c, sw, toks)
    check_y(y.cpu().numpy()[toks], ref, f"full/{_sid(shape)}/ns{ns}")


def test_layer_full_repeatable_and_workspace_poison(dev):
    c = get_case("c1", dev)
    sh = c.sh
    wg = _bf16_dev(synth.make_router_weights(sh), dev)
    pw = _with_shared(c, _shared_list(sh, 1), dev)
    need = moe.layer_full_workspace_size(sh.T, sh.E + 1, sh.k, sh.H, sh.I, 1)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=dev)
    y1 = moe.layer_forward_full(pw, 1, wg, c.x, sh.k, workspace=ws)
    ws.fill_(0x3C)
    y2 = torch.full((sh.T, sh.H), float("nan"), device=dev)
    moe.layer_forward_full(pw, 1, wg, c.x, sh.k, y=y2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
