"""The whole layer (moe_fp4_layer_forward) captured into a HIP graph.

The library only enqueues kernels on the caller's stream (no allocation, no
memset, no host readback of device data), so one layer call can be captured
and replayed.  Each replay here follows eager work and new inputs written into
the captured buffers, and must equal an eager call on the same inputs bit for
bit: the graph holds the launches, the data stays live."""
import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import synth
from gpu_cases import get_case, log

pytestmark = pytest.mark.gpu

CASES = [
    ("c1", 0),                                                                   # decode, fused front
    (synth.Shape(T=300, H=512, I=256, E=16, k=4, seed=51), moe.MOE_FLAG_FORCE_PREFILL),  # prefill
    (synth.Shape(T=40, H=256, I=128, E=8, k=2, seed=52), moe.MOE_FLAG_FORCE_DECODE),    # T > 16: stand-alone front
]


def _sid(v):
    return v if isinstance(v, str) else f"T{v.T}H{v.H}I{v.I}E{v.E}k{v.k}"


@pytest.mark.parametrize("shape,flags", CASES, ids=lambda v: _sid(v) if not isinstance(v, int) else f"f{v}")
def test_layer_graph_replays_match_eager(shape, flags, dev):
    c = get_case(shape, dev)
    sh = c.sh
    log(f"[graph] {_sid(shape)} flags={flags}")
    x_buf = c.x.clone()
    l_buf = c.logits.clone()
    y = torch.empty((sh.T, sh.H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(moe.layer_workspace_size(sh.T, sh.E, sh.k, sh.H, sh.I, flags), 256),
                     dtype=torch.uint8, device=dev)
    moe.layer_forward(c.pw, x_buf, l_buf, sh.k, flags, y=y, workspace=ws)  # warm-up outside capture
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.layer_forward(c.pw, x_buf, l_buf, sh.k, flags, y=y, workspace=ws)

    rng = np.random.default_rng(7)
    for rep in range(4):
        if rep == 1:    # new activations
            x_buf.copy_(torch.roll(c.x, shifts=3, dims=0))
        elif rep == 2:  # new routing: logits of other tokens, different expert counts
            l_buf.copy_(torch.roll(c.logits, shifts=5, dims=0))
        elif rep == 3:  # both, with a token's logits tied
            perm = torch.from_numpy(rng.permutation(sh.T)).to(dev)
            x_buf.copy_(c.x[perm])
            l_buf.copy_(c.logits[perm])
            l_buf[0, :] = 0.25
        expected = moe.layer_forward(c.pw, x_buf, l_buf, sh.k, flags)      # eager, own buffers
        torch.cuda.synchronize()
        y.fill_(float("nan"))
        ws.fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, expected), f"replay {rep} differs from eager"


def test_full_layer_and_dense_graph_replays_match_eager(dev):
    """The layer from hidden states (router slice planes in the workspace, one
    shared expert) and the FP8 dense projection, captured and replayed with new
    inputs between replays; every replay equals an eager call bit for bit."""
    c = get_case("c1", dev)
    sh = c.sh
    names = ("w1", "s1", "w3", "s3", "w2", "s2")
    sw = synth.make_shared_weights(sh)
    pw = moe.prepack_weights(*[torch.from_numpy(np.concatenate([getattr(c.inp, n), sw[i]])).to(dev)
                               for i, n in enumerate(names)])
    wg = torch.from_numpy(synth.make_router_weights(sh).view(np.int16)).to(dev).view(torch.bfloat16)
    dn = synth.make_dense_inputs("d0", T=sh.T, K=sh.H, N=96)
    dw = moe.dense_prepack(torch.from_numpy(dn.wq).to(dev), torch.from_numpy(dn.ws).to(dev))
    x_buf = c.x.clone()
    y = torch.empty((sh.T, sh.H), dtype=torch.float32, device=dev)
    yd = torch.empty((sh.T, 96), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((sh.T, sh.H), dtype=torch.uint8, device=dev)
    xs = torch.empty((sh.T, sh.H // 32), dtype=torch.uint8, device=dev)
    ws = torch.empty(moe.layer_full_workspace_size(sh.T, sh.E + 1, sh.k, sh.H, sh.I, 1),
                     dtype=torch.uint8, device=dev)

    def run():
        moe.layer_forward_full(pw, 1, wg, x_buf, sh.k, y=y, workspace=ws)
        moe.quant_act_mxfp8(x_buf, xq, xs)
        moe.dense_forward(dw, xq, xs, y=yd)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        x_buf.copy_(torch.roll(c.x, shifts=rep + 1, dims=0))
        want_y = moe.layer_forward_full(pw, 1, wg, x_buf, sh.k)
        want_d = moe.dense_layer(dw, x_buf)
        torch.cuda.synchronize()
        y.fill_(float("nan"))
        yd.fill_(0)
        ws.fill_(0x77)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want_y), f"full layer replay {rep} differs from eager"
        assert torch.equal(yd.view(torch.int16), want_d.view(torch.int16)), f"dense replay {rep}"
