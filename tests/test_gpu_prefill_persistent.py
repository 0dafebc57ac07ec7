"""GPU parity of the persistent prefill GEMMs when each workgroup runs many
work items (one workgroup per compute unit walks its XCD's share of the
(token tile, feature tile) items).

Two regimes of the item-to-item hand-off are exercised at sizes the oracle
checks on sampled tokens:
  * chained: K has >= 4 steps, so the next item's first three LDS stages are
    loaded during the current item's last three steps and its row sources two
    items ahead by LDS-DMA; J = 4 is the boundary where the first chained load
    is issued right after the step that makes those row sources visible;
  * cold: K has < 4 steps (H = 256: 2 steps), so every item refills the ring.
Both shapes have several hundred gate/up items, i.e. several per workgroup.
The stage outputs are also required to match the single-call layer entry
bit for bit."""
import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import oracle
import synth
from gpu_cases import check_y, get_case, log, sample_tokens

pytestmark = pytest.mark.gpu

SHAPES = {
    # gate/up: J = H/128 = 4 (chained, boundary), 384 tiles x 2 feature tiles
    "chain_J4": synth.Shape(T=8192, H=512, I=256, E=64, k=8, seed=41),
    # gate/up: J = 2 (cold hand-off), 192 tiles x 8 feature tiles;
    # down: J2 = 8 (chained)
    "cold_J2": synth.Shape(T=4096, H=256, I=1024, E=64, k=8, seed=42),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_prefill_many_items_per_workgroup(name, dev):
    c = get_case(SHAPES[name], dev)
    sh = c.sh
    log(f"[persistent] {name} T{sh.T} H{sh.H} I{sh.I} E{sh.E} k{sh.k}")
    flags = moe.MOE_FLAG_FORCE_PREFILL
    y_chain, it = moe.moe_layer(c.pw, c.x, c.logits, sh.k, flags, return_intermediates=True)
    y = moe.layer_forward(c.pw, c.x, c.logits, sh.k, flags)
    torch.cuda.synchronize()
    assert torch.equal(y, y_chain)
    # integer stages against the oracle, bit for bit
    assert np.array_equal(it["sorted_pair"].cpu().numpy(), c.sorted_pair)
    assert np.array_equal(it["expert_offsets"].cpu().numpy(), c.offsets)
    toks = sample_tokens(sh.T, 24, seed=5)
    check_y(y.cpu().numpy()[toks], oracle.layer_tokens(c.inp, toks), f"persistent/{name}")


def test_prefill_repeatable_across_calls(dev):
    """Items are taken in a fixed order per workgroup: two calls agree bitwise."""
    c = get_case(SHAPES["chain_J4"], dev)
    flags = moe.MOE_FLAG_FORCE_PREFILL
    y1 = moe.layer_forward(c.pw, c.x, c.logits, c.sh.k, flags)
    y2 = moe.layer_forward(c.pw, c.x, c.logits, c.sh.k, flags)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
