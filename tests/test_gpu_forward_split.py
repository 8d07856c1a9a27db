"""Kernel options selected at create through the environment, on a small layer with a longer
reduction (E=8, K=1024, N=256, top-2), every output compared with the oracle: pair mode with a
superblock's reduction split across workgroups (partial sums in slots, added in slot order by the
last arrival; split and unsplit runs agree to the parity bar, each split run is bitwise
reproducible), and the wide kernel with 32- and 64-row work items."""
import numpy as np
import pytest

from oracle import moe_forward
from synth import MoEDims, gen_hidden, gen_routing_softmax
from tests.gpu_common import gpu_forward, log, make_layer, parity

pytestmark = pytest.mark.gpu
D = MoEDims(E=8, K=1024, N=256, topk=2)   # GEMM1: 8 group quads, 8 superblocks; GEMM2: 2 quads


@pytest.fixture(scope="module")
def unsplit():
    layer, store = make_layer(D, 11, max_tokens=64, tag="split-ref")
    yield layer, store
    layer.close()


# (S1, X1, S2, X2): waves per superblock in a workgroup and workgroups per superblock
SPLITS = [(1, 8, 1, 2), (4, 2, 2, 1), (2, 4, 1, 2), (1, 2, 2, 1)]


@pytest.mark.parametrize("split", SPLITS, ids=lambda s: "S1=%d,X1=%d,S2=%d,X2=%d" % s)
def test_split_reduction_matches_oracle(unsplit, split, monkeypatch):
    s1, x1, s2, x2 = split
    for k, v in zip(("W4MOE_S1", "W4MOE_X1", "W4MOE_S2", "W4MOE_X2"), split):
        monkeypatch.setenv(k, str(v))
    layer, store = make_layer(D, 11, max_tokens=64, tag=f"split {split}")
    try:
        for M in (1, 5, 32):
            x = gen_hidden(M, D.K, 900 + M)
            ids, w = gen_routing_softmax(M, D.E, D.topk, 910 + M)
            ref = moe_forward(D, x, ids, w, store)
            base = gpu_forward(unsplit[0], x, ids, w, 3)
            for plan in (3, 5):
                log(f"[split {split}] M={M} plan={plan}")
                got = gpu_forward(layer, x, ids, w, plan)
                parity(got, ref, f"split {split} M={M} plan{plan}")
                assert np.array_equal(got, gpu_forward(layer, x, ids, w, plan))
                assert layer.device_error() == 0
                parity(got, base, f"split {split} vs unsplit M={M}")
    finally:
        layer.close()


def test_split_with_dropped_ids(monkeypatch):
    """Dropped ids under a split: each superblock is still counted once (no stale counters)."""
    for k, v in (("W4MOE_S1", 1), ("W4MOE_X1", 8), ("W4MOE_S2", 1), ("W4MOE_X2", 2)):
        monkeypatch.setenv(k, str(v))
    layer, store = make_layer(D, 11, max_tokens=64, tag="split dropped")
    try:
        M = 6
        x = gen_hidden(M, D.K, 950)
        ids, w = gen_routing_softmax(M, D.E, D.topk, 951)
        bad = ids.copy()
        bad[1, 0], bad[4, 1] = -1, D.E + 3
        keep = (bad >= 0) & (bad < D.E)
        ref = moe_forward(D, x, np.where(keep, bad, 0).astype(np.int32), np.where(keep, w, 0).astype(np.float32), store)
        for plan in (3, 5, 3):
            got = gpu_forward(layer, x, bad, w, plan)
            assert layer.device_error() == 1
            parity(got, ref, f"split dropped plan{plan}")
        # the next call with valid ids is unaffected
        good = gpu_forward(layer, x, ids, w, 3)
        assert layer.device_error() == 0
        parity(good, moe_forward(D, x, ids, w, store), "split after dropped")
    finally:
        layer.close()


@pytest.mark.parametrize("rows", [32, 64])
def test_wide_item_sizes(rows, monkeypatch):
    """The wide kernel with 32- and 64-row work items (ragged items of 1..64 rows, hot experts with
    several items, empty experts) matches the oracle on every output."""
    monkeypatch.setenv("W4MOE_WIDE_ROWS", str(rows))
    layer, store = make_layer(D, 11, max_tokens=256, tag=f"wide rows={rows}")
    try:
        for M in (3, 40, 256):
            x = gen_hidden(M, D.K, 960 + M)
            ids, w = gen_routing_softmax(M, D.E, D.topk, 970 + M)
            if M == 256:
                ids[:150, 0] = 5      # one expert with 150+ rows
            log(f"[wide rows={rows}] M={M}")
            got = gpu_forward(layer, x, ids, w, 4)
            parity(got, moe_forward(D, x, ids, w, store), f"wide rows={rows} M={M}")
            assert layer.device_error() == 0
    finally:
        layer.close()
