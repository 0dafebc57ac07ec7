"""One GPU's share of the layer under expert or tensor parallelism.

Only index and slicing work on the host side of the C ABI (no arithmetic of
the layer): a deployment that splits the layer over G GPUs runs the same
library calls on each GPU's share.

* Expert parallelism: GPU g owns experts [e0, e1).  After routing, the
  (token, slot) pairs routed to its experts arrive with their MXFP8 rows; it
  runs the gate/up and down GEMMs over its own experts with their real row
  counts and returns the O rows.  ``ep_segment`` cuts that share out of the
  full routing (offsets re-based to the shard, the pair ids unchanged).
* Tensor parallelism: GPU g owns the intermediate rows [i0, i1) of every
  expert: W1/W3 rows and the matching W2 columns.  Its layer output is a
  partial y; the G partials add up to y.  ``tp_slice`` cuts the canonical
  weights (i0, i1 multiples of 128, so MXFP8 blocks of h stay whole).
"""
from __future__ import annotations


def ep_segment(offsets, sorted_pair, e0: int, e1: int):
    """(offsets of experts e0..e1 re-based to 0, the shard's sorted pair ids,
    its row range in the full sorted order).  The pair ids keep the length of
    the full list (T*k), as the stage calls take it: the shard's own first,
    then pair 0 repeated (never computed: rows past the last offset are
    neither read as rows nor written)."""
    o = offsets[e0:e1 + 1]
    r0, r1 = int(o[0]), int(o[-1])
    sp = sorted_pair.new_zeros(sorted_pair.shape)
    sp[:r1 - r0] = sorted_pair[r0:r1]
    return (o - o[0]).contiguous(), sp, (r0, r1)


def ep_weights(w1, s1, w3, s3, w2, s2, e0: int, e1: int):
    """The canonical weights of experts [e0, e1)."""
    return tuple(a[e0:e1].contiguous() for a in (w1, s1, w3, s3, w2, s2))


def tp_slice(w1, s1, w3, s3, w2, s2, i0: int, i1: int):
    """Intermediate rows [i0, i1) of every expert: W1/W3 rows (and their
    scales), W2 columns (packed two per byte along I, one scale per 32)."""
    if i0 % 128 or i1 % 128:
        raise ValueError("TP slices must be multiples of 128 along I")
    return (w1[:, i0:i1].contiguous(), s1[:, i0:i1].contiguous(),
            w3[:, i0:i1].contiguous(), s3[:, i0:i1].contiguous(),
            w2[:, :, i0 // 2:i1 // 2].contiguous(), s2[:, :, i0 // 32:i1 // 32].contiguous())
