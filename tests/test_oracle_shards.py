"""The tensor-parallel split of the layer, pinned on the oracle (CPU only).

Splitting the intermediate size I into slices that are multiples of 32
keeps every MXFP8 block of h whole, so the layer over the full I equals the
sum of the layers over the slices (the down projection's sum over i split
into parts): exact in real arithmetic, here to fp64 rounding.  The slicing
helper used on the GPU side is checked against plain index arithmetic."""
import dataclasses

import numpy as np
import torch

import oracle
import synth
from fp4_routed_expert_amd import shard


def _slice_inputs(inp, i0, i1, w2_from=None):
    names = ("w1", "s1", "w3", "s3", "w2", "s2")
    w = shard.tp_slice(*[torch.from_numpy(getattr(inp, n)) for n in names], i0, i1)
    if w2_from is not None:   # W2 columns of another slice: a deliberate mistake
        v = shard.tp_slice(*[torch.from_numpy(getattr(inp, n)) for n in names], *w2_from)
        w = w[:4] + v[4:]
    return synth.LayerInputs(shape=dataclasses.replace(inp.shape, I=i1 - i0), x=inp.x, logits=inp.logits,
                             w1=w[0].numpy(), s1=w[1].numpy(), w3=w[2].numpy(), s3=w[3].numpy(),
                             w2=w[4].numpy(), s2=w[5].numpy())


def test_tp_partials_add_up_to_the_layer():
    inp = synth.make_inputs(synth.Shape(T=6, H=256, I=512, E=4, k=2, seed=81))
    y = oracle.layer_tokens(inp).astype(np.float64)
    parts = np.zeros_like(y)
    wrong = np.zeros_like(y)
    for g in range(4):
        i0, i1 = 128 * g, 128 * (g + 1)
        parts += oracle.layer_tokens(_slice_inputs(inp, i0, i1)).astype(np.float64)
        j = (g + 1) % 4
        wrong += oracle.layer_tokens(_slice_inputs(inp, i0, i1, (128 * j, 128 * (j + 1)))).astype(np.float64)
    # each partial and y are rounded to fp32 by the oracle
    np.testing.assert_allclose(parts, y, rtol=1e-6, atol=1e-6 * np.abs(y).max())
    assert not np.allclose(wrong, y, rtol=1e-3, atol=1e-3 * np.abs(y).max())


def test_tp_slice_indices():
    E, H, I = 2, 256, 384
    w1 = torch.arange(E * I * (H // 2)).reshape(E, I, H // 2)
    w2 = torch.arange(E * H * (I // 2)).reshape(E, H, I // 2)
    s2 = torch.arange(E * H * (I // 32)).reshape(E, H, I // 32)
    out = shard.tp_slice(w1, w1, w1, w1, w2, s2, 128, 256)
    assert torch.equal(out[0], w1[:, 128:256])
    assert torch.equal(out[4], w2[:, :, 64:128])       # two e2m1 values per byte along I
    assert torch.equal(out[5], s2[:, :, 4:8])          # one scale per 32 along I


def test_ep_segment_rebases_offsets():
    offsets = torch.tensor([0, 3, 3, 7, 12], dtype=torch.int32)
    sp = torch.arange(12, dtype=torch.int32) * 10
    o, s, (r0, r1) = shard.ep_segment(offsets, sp, 1, 3)
    assert o.tolist() == [0, 0, 4] and (r0, r1) == (3, 7)
    assert s.tolist() == [30, 40, 50, 60] + [0] * 8      # full length, valid pair ids past the shard
