"""Forward parity at full size: the K2.6-shaped layer (E=384, K=7168, N=2048, top-8) over the
M sweep with uniform and Zipf routing, and one tensor-parallel shard's shape (N=256). The oracle
computes sampled token rows one by one (every column of those rows); the rest of each output is
checked through properties that hold at any size (finite, duplicate rows identical, run-to-run
bitwise equality, independence from never-routed experts)."""
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


def _check(layer, store, dims, M, kind, seed, plan=0, rows=None, tag=""):
    x = gen_hidden(M, dims.K, 1000 + M)
    gen = gen_routing_softmax if kind == "softmax" else gen_routing_zipf
    ids, w = gen(M, dims.E, dims.topk, seed)
    log(f"[{tag}] M={M} routing={kind} seed={seed} plan={plan}")
    got = gpu_forward(layer, x, ids, w, plan)
    assert np.isfinite(got).all()
    assert layer.device_error() == 0
    rows = _rows(M) if rows is None else rows
    ref = moe_forward(dims, x, ids, w, store, rows=np.array(rows, np.int32))
    parity(got[rows], ref, f"{tag} M={M} {kind} rows={rows}")
    return got, ids


@pytest.mark.parametrize("plan", [0, 1, 3, 5])
@pytest.mark.parametrize("rep", [0, 1, 2])
def test_k26_decode_m1_all_columns(k26, rep, plan):
    _check(*k26, K26, 1, "softmax", 2001 + rep, plan=plan, tag="k26 decode")


@pytest.mark.parametrize("plan", [3, 5])
@pytest.mark.parametrize("M", [2, 4, 8])
def test_k26_small_batches_pair_mode(k26, M, plan):
    _check(*k26, K26, M, "softmax", 2000 + M, plan=plan, tag="k26 pair")


@pytest.mark.parametrize("plan", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("M", [9, 32, 90])
def test_k26_verify_batches(k26, M, plan):
    _check(*k26, K26, M, "softmax", 2000 + M, plan=plan, tag="k26 verify")


@pytest.mark.parametrize("plan", [0, 1, 2, 4])
@pytest.mark.parametrize("M", [256, 512, 1024])
def test_k26_plateau_uniform(k26, M, plan):
    if plan in (1, 2) and M > 256:
        pytest.skip("plans 1 and 2 at M > 256 are covered by M = 256")
    _check(*k26, K26, M, "softmax", 2000 + M, plan=plan, tag="k26 plateau")


@pytest.mark.parametrize("M", [256, 512, 1024])
def test_k26_plateau_zipf(k26, M):
    layer, store = k26
    ids, _ = gen_routing_zipf(M, K26.E, K26.topk, 3000 + M)
    counts = np.bincount(ids.reshape(-1), minlength=K26.E)
    hot = int(np.argmax(counts))
    hot_row = int(np.nonzero((ids == hot).any(axis=1))[0][-1])
    log(f"zipf M={M}: hottest expert {hot} with {counts.max()} rows, {int((counts == 0).sum())} experts unrouted")
    _check(layer, store, K26, M, "zipf", 3000 + M, rows=_rows(M, [hot_row]), tag="k26 zipf")


@pytest.mark.parametrize("plan", [1, 2, 4])
def test_k26_hot_experts(k26, plan):
    """Every token routed to the same 8 experts: 300 rows per expert, many work items each."""
    layer, store = k26
    M = 300
    x = gen_hidden(M, K26.K, 4242)
    ids = np.tile(np.arange(8, dtype=np.int32) * 47, (M, 1))
    w = np.random.default_rng(3).dirichlet(np.ones(8), size=M).astype(np.float32)
    got = gpu_forward(layer, x, ids, w, plan)
    rows = _rows(M, [17, 33])
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
    _check(*tp8, TP8, M, "softmax", 2000 + M, tag="tp8 shard")
    if M >= 90:
        _check(*tp8, TP8, M, "softmax", 2000 + M, plan=2, tag="tp8 shard plan2")
    if M == 1:
        _check(*tp8, TP8, M, "softmax", 2000 + M, plan=3, tag="tp8 shard pair")
        _check(*tp8, TP8, M, "softmax", 2000 + M, plan=5, tag="tp8 shard pair, two launches")
