"""Pins of the router oracle (oracle/router.py) against facts fixed independently of it: the
selection by a threshold scan (no sort), closed forms of the renormalised softmax, invariances, tie
order, masked experts, and agreement with the workload's routing generator (a separate float32
argsort implementation)."""
import itertools

import numpy as np
import pytest

from oracle import route
from synth import gen_logits, gen_routing_softmax


def _threshold_select(row, k):
    """The k largest by repeated maximum scans, ties to the lower index: a second method."""
    taken = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None or v > row[best]:
                best = e
        taken.append(best)
    return taken


@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (384, 8)])
def test_selection_matches_repeated_max_scans(E, k):
    logits = gen_logits(6, E, 77 + E)
    ids, w = route(logits, k)
    for m in range(6):
        assert list(ids[m]) == _threshold_select([float(v) for v in logits[m]], k)
        chosen = set(ids[m].tolist())
        assert min(logits[m][list(chosen)]) >= max(np.delete(logits[m], list(chosen)))


def test_weights_sum_to_one_and_follow_the_logits():
    logits = gen_logits(20, 384, 5)
    ids, w = route(logits, 8)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (w > 0).all() and (np.diff(w, axis=1) <= 0).all()


def test_two_way_closed_form():
    """k = 2: the weights are the logistic function of the logit difference."""
    logits = np.array([[0.5, -1.25, 3.0, 2.0]], np.float32)
    ids, w = route(logits, 2)
    assert ids.tolist() == [[2, 3]]
    s = 1.0 / (1.0 + np.exp(-(3.0 - 2.0)))
    assert abs(w[0, 0] - s) < 1e-15 and abs(w[0, 1] - (1 - s)) < 1e-15


def test_equal_logits_give_uniform_weights_and_lowest_indices():
    ids, w = route(np.zeros((3, 10), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(w == 0.25)


def test_ties_at_the_boundary_take_the_lower_index():
    row = np.array([[1.0, 5.0, 2.0, 5.0, 2.0, 2.0, 0.0]], np.float32)
    ids, _ = route(row, 4)
    assert ids.tolist() == [[1, 3, 2, 4]]


def test_shift_invariance():
    """Adding a constant (exactly representable sums) changes neither ids nor weights."""
    rng = np.random.default_rng(3)
    logits = (rng.integers(-4096, 4096, size=(5, 64)) / 512.0).astype(np.float32)
    a = route(logits, 6)
    b = route(logits + np.float32(16.0), 6)
    assert np.array_equal(a[0], b[0]) and np.allclose(a[1], b[1], rtol=1e-15, atol=0)


def test_permutation_equivariance():
    """Relabelling the experts relabels the chosen ids (distinct logits, so no tie order involved)."""
    logits = gen_logits(4, 32, 9)
    perm = np.random.default_rng(1).permutation(32)
    a_ids, a_w = route(logits, 5)
    b_ids, b_w = route(logits[:, perm], 5)
    inv = np.argsort(perm)
    assert np.array_equal(perm[b_ids], a_ids) and np.array_equal(a_w, b_w)
    assert np.array_equal(b_ids, inv[a_ids])


def test_masked_experts():
    logits = np.full((2, 6), -np.inf, np.float32)
    logits[0, 4] = 0.5
    logits[1, [1, 2]] = [1.0, 1.0]
    ids, w = route(logits, 3)
    assert ids.tolist() == [[4, 0, 1], [1, 2, 0]]
    assert w.tolist() == [[1.0, 0.0, 0.0], [0.5, 0.5, 0.0]]


def test_k_equals_e_is_a_full_softmax():
    logits = np.array([[0.0, 1.0, 2.0]], np.float32)
    ids, w = route(logits, 3)
    e = np.exp([2.0, 1.0, 0.0])
    assert ids.tolist() == [[2, 1, 0]] and np.allclose(w[0], e / e.sum(), rtol=1e-15)


def test_agrees_with_the_routing_generator():
    """The workload generator routes the same logits with float32 softmax + argsort."""
    for seed in (2001, 2002, 2090):
        ids_g, w_g = gen_routing_softmax(16, 384, 8, seed)
        ids, w = route(gen_logits(16, 384, seed), 8)
        assert np.array_equal(ids, ids_g)
        assert np.allclose(w, w_g, rtol=2e-6, atol=1e-7)


def test_rejects_outside_the_domain():
    with pytest.raises(ValueError):
        route(np.array([[np.nan, 0.0]], np.float32), 1)
    with pytest.raises(ValueError):
        route(np.full((1, 4), -np.inf, np.float32), 2)
    with pytest.raises(ValueError):
        route(np.zeros((1, 4), np.float32), 5)


def test_brute_force_subsets_tiny():
    """E = 6, k = 3: the chosen set maximises the sum of logits over all 20 subsets."""
    logits = gen_logits(10, 6, 123)
    ids, _ = route(logits, 3)
    for m in range(10):
        best = max(itertools.combinations(range(6), 3), key=lambda c: float(sum(logits[m][list(c)])))
        assert set(best) == set(ids[m].tolist())
