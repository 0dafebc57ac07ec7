"""GPU parity of the whole-layer entry point moe_fp4_layer_forward.

It must give bitwise the same y as the chain of single-stage calls (whose
integer outputs are checked bit-exactly against the oracle elsewhere), and y
within the output tolerance of the oracle.  Token counts up to 16 take the
fused front kernel (routing + sort in one workgroup, MXFP8 in the others);
larger ones the stand-alone kernels, so the shapes below straddle that limit
and cover every keys-per-lane variant of the routing (E <= 64, 128, 256, 512,
1024)."""
import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import oracle
import synth
from gpu_cases import Case, check_y, get_case, log, sample_tokens

pytestmark = pytest.mark.gpu

PATHS = {"decode": moe.MOE_FLAG_FORCE_DECODE, "prefill": moe.MOE_FLAG_FORCE_PREFILL}

SHAPES = [
    "c0",
    "c1",
    synth.Shape(T=1, H=128, I=128, E=1, k=1, seed=31),        # one token, one expert
    synth.Shape(T=16, H=256, I=128, E=100, k=7, seed=37),     # largest fused T, E in (64, 128]
    synth.Shape(T=17, H=256, I=128, E=100, k=7, seed=38),     # just past the fused limit
    synth.Shape(T=32, H=256, I=128, E=100, k=7, seed=32),     # stand-alone front, E in (64, 128]
    synth.Shape(T=16, H=384, I=256, E=256, k=8, seed=33),     # fused, E in (128, 256]
    synth.Shape(T=20, H=384, I=256, E=256, k=8, seed=40),     # stand-alone front, E in (128, 256]
    synth.Shape(T=9, H=128, I=128, E=400, k=5, seed=34),      # E in (256, 512]
    synth.Shape(T=16, H=128, I=128, E=1024, k=32, seed=39),   # fused, E = 1024, k = 32: P = 512
    synth.Shape(T=32, H=128, I=128, E=1024, k=32, seed=35),   # E = 1024, k = 32: P = 1024
    synth.Shape(T=33, H=256, I=128, E=65, k=7, seed=36),      # stand-alone front, E = 65
]


def _sid(s):
    return s if isinstance(s, str) else f"T{s.T}H{s.H}I{s.I}E{s.E}k{s.k}"


@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("shape", SHAPES, ids=_sid)
def test_layer_forward_matches_chain_and_oracle(shape, path, dev):
    c = get_case(shape, dev)
    log(f"[layer_forward] {_sid(shape)} {path}")
    y_chain = moe.moe_layer(c.pw, c.x, c.logits, c.sh.k, PATHS[path])
    y = moe.layer_forward(c.pw, c.x, c.logits, c.sh.k, PATHS[path])
    torch.cuda.synchronize()
    assert torch.equal(y, y_chain)
    toks = sample_tokens(c.sh.T, 24, seed=2)
    check_y(y.cpu().numpy()[toks], oracle.layer_tokens(c.inp, toks), f"layer/{_sid(shape)}/{path}")


@pytest.mark.parametrize("T", [16, 48])
def test_layer_forward_ties(T, dev):
    """Many exact ties in the logits, through both front variants."""
    sh = synth.Shape(T=T, H=256, I=128, E=16, k=4, seed=37)
    inp = synth.make_inputs(sh)
    inp.logits = (np.round(inp.logits * 2) / 2).astype(np.float32)
    inp.logits[:, 3] = inp.logits[:, 11] = 0.75                    # equal top candidates
    c = Case(inp, dev)
    y_chain = moe.moe_layer(c.pw, c.x, c.logits, sh.k)
    y = moe.layer_forward(c.pw, c.x, c.logits, sh.k)
    torch.cuda.synchronize()
    assert torch.equal(y, y_chain)
    check_y(y.cpu().numpy(), oracle.layer_tokens(c.inp), f"layer-ties/T{T}")


def test_layer_forward_poisoned_workspace(dev):
    c = get_case("c1", dev)
    T, k, E, H, I = c.sh.T, c.sh.k, c.sh.E, c.sh.H, c.sh.I
    y_ref = moe.layer_forward(c.pw, c.x, c.logits, k)
    need = moe.layer_workspace_size(T, E, k, H, I)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    moe.layer_forward(c.pw, c.x, c.logits, k, y=y, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
