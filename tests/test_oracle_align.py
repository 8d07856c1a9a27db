"""Pins of the oracle's token-to-expert alignment (no GPU): a brute-force re-derivation on small
inputs, the invariants the padded sort must satisfy, and special cases (one expert takes every
entry, every expert empty but one, a single token, duplicate ids within a token)."""
import numpy as np
import pytest

from oracle import moe_align
from synth import gen_routing_softmax, gen_routing_zipf


def _brute(flat, E, B):
    flat = [int(v) for v in flat]
    T = len(flat)
    sorted_ids, block_expert, counts, offsets = [], [], [], [0]
    for e in range(E):
        mine = [f for f in range(T) if flat[f] == e]          # ascending flat id
        counts.append(len(mine))
        padded = -(-len(mine) // B) * B
        sorted_ids += mine + [T] * (padded - len(mine))
        block_expert += [e] * (padded // B)
        offsets.append(offsets[-1] + padded)
    active = [e for e in range(E) if counts[e] > 0]
    return counts, offsets, sorted_ids, block_expert, active


def _check(ids, E, B):
    flat = np.asarray(ids).reshape(-1)
    T = flat.size
    got = moe_align(ids, E, B)
    counts, offsets, sorted_ids, block_expert, active = _brute(flat, E, B)
    assert got["counts"].tolist() == counts
    assert got["offsets"].tolist() == offsets
    assert got["sorted_ids"].tolist() == sorted_ids
    assert got["block_expert"].tolist() == block_expert
    assert got["active"].tolist() == active
    # invariants
    s = got["sorted_ids"]
    assert got["counts"].sum() == T
    assert np.array_equal(np.sort(s[s < T]), np.arange(T))
    assert np.all(got["offsets"] % B == 0)
    assert int((s == T).sum()) == got["offsets"][-1] - T
    return got


@pytest.mark.parametrize("B", [1, 16, 32, 64])
@pytest.mark.parametrize("M,E,k", [(1, 384, 8), (16, 8, 2), (90, 384, 8), (300, 384, 8)])
def test_align_matches_brute_force(M, E, k, B):
    ids, _ = gen_routing_softmax(M, E, k, 2000 + M)
    _check(ids, E, B)


@pytest.mark.parametrize("B", [1, 16])
def test_align_zipf(B):
    ids, _ = gen_routing_zipf(512, 384, 8, 77)
    got = _check(ids, 384, B)
    assert (got["counts"] == 0).any() and got["counts"].max() > 100


def test_align_special_cases():
    E = 16
    _check(np.full((40, 4), 5, np.int32), E, 16)                 # all entries to one expert
    _check(np.array([[3]], np.int32), E, 16)                      # one entry
    _check(np.array([[2, 2, 7], [7, 2, 2]], np.int32), E, 4)      # duplicates within a token
    _check(np.arange(E, dtype=np.int32).reshape(4, 4), E, 1)      # every expert exactly once
    _check(np.zeros((0, 8), np.int32), E, 16)                     # no tokens
    got = moe_align(np.array([[E - 1]], np.int32), E, 16)
    assert got["active"].tolist() == [E - 1] and got["offsets"][-1] == 16


def test_align_rejects_out_of_range_ids():
    with pytest.raises(RuntimeError):
        moe_align(np.array([[0, 16]], np.int32), 16, 16)
    with pytest.raises(RuntimeError):
        moe_align(np.array([[-1]], np.int32), 16, 16)
