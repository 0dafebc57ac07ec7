"""Pins of the oracle's top-k routing, gates and expert sort/permute.

Routing compares fp32 scores with a fixed tie-break on expert id (pwwt.cn
review, section 4.1 precision table, row "MoE routing top-k"; section 4.2:
ties by expert_id, never by memory address, and no unstable sorting).
Gates are a softmax over the k selected logits.  The pins are brute-force
full sorts, closed forms and a hand-worked example.
"""
import math

import numpy as np
import pytest

import oracle


def brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (65, 1), (65, 65), (256, 8), (7, 7)])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_brute_force(E, k, ties):
    rng = np.random.default_rng(E * 100 + k)
    lg = rng.normal(0, 1, (40, E)).astype(np.float32)
    if ties:
        lg = (np.round(lg * 2) / 2).astype(np.float32)  # a 0.5 grid: many exact ties
    ids, gates = oracle.route(lg, k)
    for t in range(lg.shape[0]):
        assert list(ids[t]) == brute_topk(lg[t], k)
        assert abs(float(gates[t].astype(np.float64).sum()) - 1.0) < 1e-6
        assert all(gates[t][j] >= gates[t][j + 1] for j in range(k - 1))


def test_signed_zero_ties_go_to_lower_index():
    lg = np.array([[-1.0, 0.0, -0.0, -2.0], [-1.0, -0.0, 0.0, -2.0]], dtype=np.float32)
    ids, _ = oracle.route(lg, 2)
    assert ids.tolist() == [[1, 2], [1, 2]]


def test_gates_closed_form_k2():
    """For k = 2 the softmax reduces to the logistic of the logit gap."""
    rng = np.random.default_rng(5)
    lg = rng.normal(0, 2, (200, 16)).astype(np.float32)
    ids, gates = oracle.route(lg, 2)
    for t in range(200):
        d = float(lg[t, ids[t, 0]]) - float(lg[t, ids[t, 1]])
        g0 = 1.0 / (1.0 + math.exp(-d))
        assert abs(gates[t, 0] - g0) <= 1e-7 and abs(gates[t, 1] - (1 - g0)) <= 1e-7


def test_k1_gate_is_one():
    rng = np.random.default_rng(6)
    ids, gates = oracle.route(rng.normal(0, 1, (10, 9)).astype(np.float32), 1)
    assert (gates == 1.0).all()


def test_hand_worked_routing_and_sort():
    # t0: [0.5, 0.5, -1] -> the tie goes to expert 0, gates 1/2 each.
    # t1: [-1, 0, ln 3] -> experts 2 then 1, gates 3/4 and 1/4.
    lg = np.array([[0.5, 0.5, -1.0], [-1.0, 0.0, math.log(3.0)]], dtype=np.float32)
    ids, gates = oracle.route(lg, 2)
    assert ids.tolist() == [[0, 1], [2, 1]]
    assert gates[0].tolist() == [0.5, 0.5]
    assert abs(gates[1, 0] - 0.75) < 1e-7 and abs(gates[1, 1] - 0.25) < 1e-7
    # pairs p = t*k + j: (0 -> e0), (1 -> e1), (2 -> e2), (3 -> e1)
    counts, offsets, sp, pp = oracle.sort(ids, 3)
    assert counts.tolist() == [1, 2, 1]
    assert offsets.tolist() == [0, 1, 3, 4]
    assert sp.tolist() == [0, 1, 3, 2]
    assert pp.tolist() == [0, 1, 3, 2]


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (100, 64, 6), (513, 256, 8), (37, 5, 5), (9, 300, 1)])
def test_sort_brute_force_and_invariants(T, E, k):
    rng = np.random.default_rng(T + E + k)
    ids, _ = oracle.route(rng.normal(0, 1, (T, E)).astype(np.float32), k)
    flat = ids.reshape(-1)
    P = flat.size
    counts, offsets, sp, pp = oracle.sort(ids, E)
    assert sorted(range(P), key=lambda p: (flat[p], p)) == sp.tolist()
    assert counts.sum() == P
    assert (np.bincount(flat, minlength=E) == counts).all()
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all() and offsets[-1] == P
    assert sorted(sp.tolist()) == list(range(P))          # a bijection
    assert (pp[sp] == np.arange(P)).all()                 # exact inverse
    tok_hits = np.bincount(sp // k, minlength=T)
    assert (tok_hits == k).all()                          # each token exactly k times
    for e in range(E):
        seg = sp[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()  # stable within expert


def test_sort_all_to_one_expert_and_empty_experts():
    ids = np.full((20, 1), 3, dtype=np.int32)
    counts, offsets, sp, pp = oracle.sort(ids, 6)
    assert counts.tolist() == [0, 0, 0, 20, 0, 0]
    assert offsets.tolist() == [0, 0, 0, 0, 20, 20, 20]
    assert sp.tolist() == list(range(20))
