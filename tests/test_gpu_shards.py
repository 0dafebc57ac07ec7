"""One GPU's share of the layer under expert and tensor parallelism (the
kernels at the shard's real shape; the exchanges between GPUs are not built).

* EP: for each shard of E/G experts, the gate/up and down calls over that
  shard's experts (re-based offsets, its pairs, its packed weights) give
  exactly the O rows the unsharded calls give for those experts, bit for bit.
* TP: the layer over each I/G slice of the weights yields a partial y; the
  partials, added in shard order, match the oracle's layer."""
import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import oracle
import synth
from fp4_routed_expert_amd import shard
from gpu_cases import check_y, get_case, log, sample_tokens, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("w1", "s1", "w3", "s3", "w2", "s2")

EP_CASES = [
    (synth.Shape(T=300, H=512, I=256, E=16, k=4, seed=91), 4, moe.MOE_FLAG_FORCE_PREFILL),
    (synth.Shape(T=300, H=512, I=256, E=16, k=4, seed=91), 4, moe.MOE_FLAG_FORCE_DECODE),
    ("c1", 8, moe.MOE_FLAG_FORCE_DECODE),
]


def _sid(v):
    return v if isinstance(v, str) else f"T{v.T}H{v.H}I{v.I}E{v.E}k{v.k}"


@pytest.mark.parametrize("shape,G,flags", EP_CASES, ids=[f"{_sid(s)}-G{g}-f{f}" for s, g, f in EP_CASES])
def test_ep_shards_give_the_same_rows(shape, G, flags, dev):
    c = get_case(shape, dev)
    sh = c.sh
    log(f"[ep] {_sid(shape)} G={G} flags={flags}")
    ids, gates = moe.route_topk(c.logits, sh.k)
    counts, offsets, sp, pp = moe.sort_permute(ids, sh.E)
    xq, xs = moe.quant_act_mxfp8(c.x)
    hq, hs = moe.expert_up(c.pw, xq, xs, offsets, sp, sh.T, sh.k, flags)
    O = moe.expert_down(c.pw, hq, hs, offsets, sh.T, sh.k, flags)
    torch.cuda.synchronize()
    w = [to_dev(getattr(c.inp, n), dev) for n in NAMES]
    per = sh.E // G
    for g in range(G):
        e0, e1 = g * per, (g + 1) * per
        o_g, sp_g, (r0, r1) = shard.ep_segment(offsets, sp, e0, e1)
        if r1 == r0:
            continue
        pw_g = moe.prepack_weights(*shard.ep_weights(*w, e0, e1))
        # the up call sizes its outputs from T and k; the shard's rows are the first r1 - r0
        hq_g, hs_g = moe.expert_up(pw_g, xq, xs, o_g, sp_g, sh.T, sh.k, flags)
        O_g = moe.expert_down(pw_g, hq_g, hs_g, o_g, sh.T, sh.k, flags)
        torch.cuda.synchronize()
        n = r1 - r0
        assert torch.equal(hq_g[:n], hq[r0:r1]) and torch.equal(hs_g[:n], hs[r0:r1]), f"shard {g} h"
        assert torch.equal(O_g[:n].view(torch.int16), O[r0:r1].view(torch.int16)), f"shard {g} O"


TP_CASES = [
    (synth.Shape(T=40, H=256, I=512, E=8, k=2, seed=92), 4, 0),
    ("c1", 3, 0),                                         # I = 1536: slices of 512
    (synth.Shape(T=300, H=512, I=512, E=16, k=4, seed=93), 2, moe.MOE_FLAG_FORCE_PREFILL),
]


@pytest.mark.parametrize("shape,G,flags", TP_CASES, ids=[f"{_sid(s)}-G{g}-f{f}" for s, g, f in TP_CASES])
def test_tp_partials_add_up(shape, G, flags, dev):
    c = get_case(shape, dev)
    sh = c.sh
    log(f"[tp] {_sid(shape)} G={G} flags={flags}")
    w = [to_dev(getattr(c.inp, n), dev) for n in NAMES]
    step = sh.I // G
    y = torch.zeros((sh.T, sh.H), dtype=torch.float32, device=dev)
    for g in range(G):
        pw_g = moe.prepack_weights(*shard.tp_slice(*w, g * step, (g + 1) * step))
        y += moe.layer_forward(pw_g, c.x, c.logits, sh.k, flags)   # the fixed-order reduction
    torch.cuda.synchronize()
    toks = sample_tokens(sh.T, 16, seed=17)
    check_y(y.cpu().numpy()[toks], oracle.layer_tokens(c.inp, toks), f"tp/{_sid(shape)}/G{G}")
