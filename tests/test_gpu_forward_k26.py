"""Forward parity at full size: the K2.6-shaped layer (E=384, K=7168, N=2048, top-8) over the
whole M sweep (1..1024) with uniform routing and at M = 256..1024 with Zipf routing, and one
tensor-parallel shard's shape (N=256), under every plan.

The oracle computes every output row at M <= 32 and at M = 90, and at larger M at least 32 token
rows chosen to cover the aligned plans' work-item edges (entries 0, 15, 16, 31, 32, 47, 48 and the
last of every expert with more than 16 entries); every plan's full output is compared with the default
plan's, which holds every row of each plan to the bar. Properties that hold at any size are checked
as well (finite, duplicate rows identical, run-to-run bitwise equality, independence from
never-routed experts)."""
import numpy as np
import pytest
import torch

from oracle import moe_forward
from synth import CONFIGS, gen_expert, gen_hidden, gen_routing_softmax, gen_routing_zipf
from tests.gpu_common import gpu_forward, log, make_layer, parity, prepack_experts

pytestmark = pytest.mark.gpu
K26 = CONFIGS["k26"]
TP8 = CONFIGS["k26_tp8"]


@pytest.fixture(scope="module")
def k26():
    layer, store = make_layer(K26, 2, max_tokens=1024, tag="k26")
    yield layer, store
    layer.close()


@pytest.fixture(scope="module")
def tp8():
    layer, store = make_layer(TP8, 5, max_tokens=1024, tag="tp8")
    yield layer, store
    layer.close()


def _rows(M, extra=()):
    return sorted(set([0, M // 2, M - 1, *[r % M for r in extra]]))


def _boundary_rows(ids, M, limit=64, seed=0):
    """Token rows that exercise the aligned plans' work items: for every expert with more than 16
    entries, the tokens of its entries 0, 15, 16, 31, 32, 47, 48 and last (in flat order, which is
    the sorted order within an expert: the edges of 16-, 32- and 48-row items), plus the first,
    middle and last token, topped up with seeded random rows to at least 32 (at most `limit`)."""
    flat = ids.reshape(-1)
    rows = {0, M // 2, M - 1}
    counts = np.bincount(flat, minlength=int(flat.max()) + 1)
    for e in np.argsort(-counts, kind="stable"):
        if counts[e] <= 16 or len(rows) >= limit:
            break
        ent = np.nonzero(flat == e)[0]
        for i in (0, 15, 16, 31, 32, 47, 48, len(ent) - 1):
            if i < len(ent):
                rows.add(int(ent[i]) // ids.shape[1])
    rng = np.random.default_rng(seed)
    while len(rows) < min(32, M):
        rows.add(int(rng.integers(0, M)))
    return sorted(rows)[:max(limit, 32)]


def _plans(M, topk=8):
    """Every plan at this size: plan 3 runs as plan 5 above 64 routed entries, so it is left out there."""
    return [0, 1, 2, 3, 4, 5] if M * topk <= 64 else [0, 1, 2, 4, 5]


def _sweep_check(layer, store, dims, M, kind, seed, plans, rows, tag):
    """Each plan's output against the oracle on `rows` (None: every row), and every plan's full
    output against the default plan's (the same bar: all of them are within it of the exact result)."""
    x = gen_hidden(M, dims.K, 1000 + M)
    ids, w = (gen_routing_softmax if kind == "softmax" else gen_routing_zipf)(M, dims.E, dims.topk, seed)
    outs = {}
    for plan in plans:
        log(f"[{tag}] M={M} routing={kind} seed={seed} plan={plan}")
        outs[plan] = gpu_forward(layer, x, ids, w, plan)
        assert np.isfinite(outs[plan]).all()
        assert layer.device_error() == 0
    log(f"[{tag}] M={M}: oracle on {'all' if rows is None else len(rows)} rows")
    ref = moe_forward(dims, x, ids, w, store, rows=None if rows is None else np.array(rows, np.int32))
    for plan, got in outs.items():
        parity(got if rows is None else got[rows], ref, f"{tag} M={M} {kind} plan{plan} vs oracle")
        parity(got, outs[plans[0]], f"{tag} M={M} {kind} plan{plan} vs plan{plans[0]}, every row")
    return outs, ids


@pytest.mark.parametrize("rep", [0, 1, 2])
def test_k26_decode_m1_all_columns(k26, rep):
    _sweep_check(*k26, K26, 1, "softmax", 2001 + rep, _plans(1), None, "k26 decode")


@pytest.mark.parametrize("M", [2, 4, 8, 9, 16, 32, 90])
def test_k26_every_row(k26, M):
    """Every output of every plan against the oracle (M = 90: about 12 s of oracle on 16 cores)."""
    _sweep_check(*k26, K26, M, "softmax", 2000 + M, _plans(M), None, "k26 every row")


@pytest.mark.parametrize("M", [64, 128, 256, 330, 512, 1024])
def test_k26_sampled_rows(k26, M):
    ids, _ = gen_routing_softmax(M, K26.E, K26.topk, 2000 + M)
    _sweep_check(*k26, K26, M, "softmax", 2000 + M, _plans(M), _boundary_rows(ids, M, seed=M), "k26 sampled")


@pytest.mark.parametrize("M", [256, 512, 1024])
def test_k26_plateau_zipf(k26, M):
    ids, _ = gen_routing_zipf(M, K26.E, K26.topk, 3000 + M)
    counts = np.bincount(ids.reshape(-1), minlength=K26.E)
    log(f"zipf M={M}: hottest expert with {counts.max()} rows, {int((counts == 0).sum())} experts unrouted")
    _sweep_check(*k26, K26, M, "zipf", 3000 + M, _plans(M), _boundary_rows(ids, M, seed=M), "k26 zipf")


@pytest.mark.parametrize("plan", [1, 2, 4, 5])
def test_k26_hot_experts(k26, plan):
    """Every token routed to the same 8 experts: 300 rows per expert, many work items each."""
    layer, store = k26
    M = 300
    x = gen_hidden(M, K26.K, 4242)
    ids = np.tile(np.arange(8, dtype=np.int32) * 47, (M, 1))
    w = np.random.default_rng(3).dirichlet(np.ones(8), size=M).astype(np.float32)
    got = gpu_forward(layer, x, ids, w, plan)
    rows = _boundary_rows(ids, M, seed=7)
    parity(got[rows], moe_forward(K26, x, ids, w, store, rows=np.array(rows, np.int32)), f"k26 hot plan{plan}")


def test_k26_properties_at_full_size(k26):
    layer, store = k26
    M = 90
    x = gen_hidden(M, K26.K, 5151)
    ids, w = gen_routing_softmax(M, K26.E, K26.topk, 5152)
    x[40] = x[11]
    ids[40], w[40] = ids[11], w[11]
    a = gpu_forward(layer, x, ids, w, 0)
    assert np.isfinite(a).all()
    assert np.array_equal(a[40], a[11])
    b = gpu_forward(layer, x, ids, w, 0)
    assert np.array_equal(a, b)
    unrouted = sorted(set(range(K26.E)) - set(ids.reshape(-1).tolist()))[:2]
    log(f"[k26] overwrite never-routed experts {unrouted} with extreme values")
    rng = np.random.default_rng(0)
    wild = {}
    for e in unrouted:
        w1, s1, w2, s2 = gen_expert(K26, e, 2)
        wild[e] = (rng.integers(-2**31, 2**31, size=w1.shape, dtype=np.int64).astype(np.int32), np.full_like(s1, 0x7F7F),
                   rng.integers(-2**31, 2**31, size=w2.shape, dtype=np.int64).astype(np.int32), np.full_like(s2, 0xFF7F))
    prepack_experts(layer, K26, 2, experts=unrouted, batch=1, override=wild)
    c = gpu_forward(layer, x, ids, w, 0)
    prepack_experts(layer, K26, 2, experts=unrouted, batch=1)
    assert np.array_equal(a, c)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1, 90, 330, 1024])
def test_tp8_shard_shape(tp8, M):
    ids, _ = gen_routing_softmax(M, TP8.E, TP8.topk, 2000 + M)
    rows = None if M <= 90 else _boundary_rows(ids, M, seed=M)
    _sweep_check(*tp8, TP8, M, "softmax", 2000 + M, _plans(M), rows, "tp8 shard")
