"""Pair mode up to 128 routed entries takes the entries routed to the same expert two at a time, in
flat order, as one work item (the expert's weights stream once for both). Every output against the
oracle, under both pair plans, for routings that make items of every kind: many entries per expert
(odd and even counts, so some items hold one entry), the same expert twice within a token, dropped
ids among them, an expert shard, 8-bit codes and activation order; and the deduplicated result equal
to the per-entry one within the bar."""
import os
from dataclasses import replace

import numpy as np
import pytest

from oracle import moe_forward
from synth import CONFIGS, MoEDims, gen_hidden, gen_routing_softmax
from tests.gpu_common import gpu_forward, log, make_layer, make_layer_act_order, parity

pytestmark = pytest.mark.gpu
TINY = CONFIGS["tiny"]


def _routings(E, topk, M, seed):
    rng = np.random.default_rng(seed)
    cases = {}
    ids = rng.integers(0, 3, size=(M, topk)).astype(np.int32)          # three hot experts, odd counts
    cases["three experts"] = ids
    ids = np.repeat(rng.integers(0, E, size=(M, 1)), topk, axis=1).astype(np.int32)   # one expert per token, twice
    cases["same expert twice in a token"] = ids
    ids = rng.integers(0, E, size=(M, topk)).astype(np.int32)
    ids[::5, 0] = E + 3                                                   # dropped entries among the items
    ids[1::7, -1] = -1
    cases["dropped ids"] = ids
    ids, _ = gen_routing_softmax(M, E, topk, seed)
    cases["softmax"] = ids
    out = {}
    for k, v in cases.items():
        w = rng.dirichlet(np.ones(topk), size=M).astype(np.float32)
        out[k] = (np.ascontiguousarray(v), w)
    return out


@pytest.fixture(autouse=True)
def _shared_items(monkeypatch):
    """Items shared by two entries at every entry count (W4MOE_DEDUP=1, read when a layer is created;
    by default only from 48 routed entries on)."""
    monkeypatch.setenv("W4MOE_DEDUP", "1")


@pytest.mark.parametrize("M", [1, 7, 32, 50, 64])
def test_dedup_items_every_output(M):
    layer, store = make_layer(TINY, 41, max_tokens=64, tag="dedup tiny")
    try:
        x = gen_hidden(M, TINY.K, 4100 + M)
        for name, (ids, w) in _routings(TINY.E, TINY.topk, M, 4200 + M).items():
            bad = (ids < 0) | (ids >= TINY.E)
            dropped = bad.any()
            # a dropped slot adds nothing: the oracle's layer with that slot weighted 0 (any valid id)
            ref = moe_forward(TINY, x, np.where(bad, 0, ids).astype(np.int32),
                              np.where(bad, 0, w).astype(np.float32), store)
            for plan in (3, 5):
                log(f"[dedup] M={M} {name} plan={plan}")
                got = gpu_forward(layer, x, ids, w, plan)
                parity(got, ref, f"dedup M={M} {name} plan{plan}")
                assert layer.device_error() == (1 if dropped else 0)
    finally:
        layer.close()


@pytest.mark.parametrize("kind", ["w8", "act_order"])
def test_dedup_variants(kind):
    d = replace(TINY, bits=8) if kind == "w8" else TINY
    maker = make_layer_act_order if kind == "act_order" else make_layer
    layer, store = maker(d, 43, max_tokens=64, tag=f"dedup {kind}")
    try:
        M = 24
        x = gen_hidden(M, d.K, 4300)
        rng = np.random.default_rng(4301)
        ids = rng.integers(0, 4, size=(M, d.topk)).astype(np.int32)
        w = rng.dirichlet(np.ones(d.topk), size=M).astype(np.float32)
        ref = moe_forward(d, x, ids, w, store)
        for plan in (3, 5):
            log(f"[dedup {kind}] plan={plan}")
            parity(gpu_forward(layer, x, ids, w, plan), ref, f"dedup {kind} plan{plan}")
            assert layer.device_error() == 0
    finally:
        layer.close()


def test_dedup_expert_shard():
    """A shard holding experts 2..5 of the tiny layer, fed global ids mostly on its own experts."""
    from synth import ExpertStore
    from tests.shards import shard_ref
    from tests.test_gpu_expert_shard import make_shard
    layer = make_shard(TINY, 1, 2, 4, 64, "dedup shard")
    try:
        M = 24
        x = gen_hidden(M, TINY.K, 4400)
        rng = np.random.default_rng(4401)
        ids = rng.integers(0, TINY.E, size=(M, TINY.topk)).astype(np.int32)
        ids[::2, 0] = 3
        ids[1::3, 1] = 4
        w = rng.dirichlet(np.ones(TINY.topk), size=M).astype(np.float32)
        ref = shard_ref(TINY, x, ids, w, ExpertStore(TINY, 1), 2, 4)
        for plan in (3, 5):
            log(f"[dedup shard] plan={plan}")
            parity(gpu_forward(layer, x, ids, w, plan), ref, f"dedup shard plan{plan}")
            assert layer.device_error() == 0
    finally:
        layer.close()


@pytest.mark.parametrize("phases", [1, 2, 3, 8])
def test_single_launch_entry_groups(phases, monkeypatch):
    """The single-launch mode dispatched in 1, 2, 3 or 8 entry groups (each group's GEMM1 workgroups,
    then its GEMM2 ones; W4MOE_PHASES, read when the layer is created): every output against the
    oracle, and bitwise equal to the one-group launch."""
    monkeypatch.setenv("W4MOE_PHASES", str(phases))
    layer, store = make_layer(TINY, 47, max_tokens=64, tag=f"entry groups {phases}")
    monkeypatch.setenv("W4MOE_PHASES", "1")
    one, _ = make_layer(TINY, 47, max_tokens=64, tag="entry groups 1")
    try:
        for M in (1, 5, 32):
            x = gen_hidden(M, TINY.K, 4500 + M)
            ids, w = gen_routing_softmax(M, TINY.E, TINY.topk, 4600 + M)
            log(f"[entry groups {phases}] M={M}")
            got = gpu_forward(layer, x, ids, w, 3)
            parity(got, moe_forward(TINY, x, ids, w, store), f"entry groups {phases} M={M}")
            assert np.array_equal(got, gpu_forward(one, x, ids, w, 3))
            assert layer.device_error() == 0
    finally:
        layer.close()
        one.close()
