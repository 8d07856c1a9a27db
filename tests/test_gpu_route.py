"""Router on the GPU (w4moe_route and w4moe_forward_logits) against the router oracle: ids bit-exact
(both sides compare the same fp32 logits), weights to 2e-6, and the routed layer against the layer
oracle on the oracle's route; edge cases (ties, masked experts, NaN logits) and the single-launch
kernel's in-kernel routing against the router kernel."""
import numpy as np
import pytest
import torch

from oracle import moe_forward, route
from synth import CONFIGS, MoEDims, gen_hidden, gen_logits
from tests.gpu_common import bf16_dev, log, make_layer, parity, to_dev

pytestmark = pytest.mark.gpu
TINY = CONFIGS["tiny"]
K26 = CONFIGS["k26"]
W_TOL = 2e-6


@pytest.fixture(scope="module")
def tiny():
    layer, store = make_layer(TINY, 1, max_tokens=256, tag="route tiny")
    yield layer, store
    layer.close()


def _gpu_route(layer, logits):
    ids, w = layer.route(to_dev(logits))
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)


def _check_route(gids, gw, logits, k, tag):
    ids, w = route(logits, k)
    assert np.array_equal(gids, ids), f"{tag}: ids differ in rows {np.nonzero((gids != ids).any(axis=1))[0][:8]}"
    assert np.abs(gw - w).max() <= W_TOL, f"{tag}: max weight error {np.abs(gw - w).max():.2e}"


@pytest.mark.parametrize("M", [1, 5, 256])
def test_route_tiny(tiny, M):
    layer, _ = tiny
    logits = gen_logits(M, TINY.E, 3100 + M)
    _check_route(*_gpu_route(layer, logits), logits, TINY.topk, f"tiny M={M}")
    assert layer.device_error() == 0


def test_route_edge_cases(tiny):
    layer, _ = tiny
    E = TINY.E
    logits = np.zeros((6, E), np.float32)                      # row 0: all equal -> ids 0, 1
    logits[1] = [1, 5, 2, 5, 2, 2, 0, 0]                        # ties at the top
    logits[2] = -np.inf
    logits[2, 6] = 0.25                                         # one finite, the rest masked
    logits[3] = np.arange(E)[::-1]                              # strictly decreasing
    logits[4] = [-3, 7, 7, 7, -1, 0, 2, 7]                      # a four-way tie for first
    logits[5] = np.float32(1e30) * np.array([1, -1, 1, -1, 0, 0, 0, 0], np.float32)
    _check_route(*_gpu_route(layer, logits), logits, TINY.topk, "edge")
    assert layer.device_error() == 0


def test_route_nan_logits_drop_the_slot(tiny):
    layer, _ = tiny
    logits = np.full((2, TINY.E), np.nan, np.float32)
    logits[0, 3] = 1.0                       # one candidate for two slots
    logits[1, [2, 5]] = [0.5, -0.5]
    layer.device_error()
    ids, w = _gpu_route(layer, logits)
    assert ids.tolist() == [[3, -1], [2, 5]]
    assert w[0].tolist() == [1.0, 0.0] and abs(w[1, 0] - 1 / (1 + np.exp(-1.0))) < W_TOL
    assert layer.device_error() & 1


@pytest.mark.parametrize("plan", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("M", [1, 16, 100])
def test_forward_logits_tiny(tiny, M, plan):
    layer, store = tiny
    x = gen_hidden(M, TINY.K, 3200 + M)
    logits = gen_logits(M, TINY.E, 3300 + M)
    layer.set_plan(plan)
    out, gids, gw = layer.forward_logits(bf16_dev(x), to_dev(logits))
    torch.cuda.synchronize()
    _check_route(gids.cpu().numpy(), gw.cpu().numpy().astype(np.float64), logits, TINY.topk, f"M={M} plan{plan}")
    ids, w = route(logits, TINY.topk)
    ref = moe_forward(TINY, x, ids, w.astype(np.float32), store)
    parity(out.float().cpu().numpy().astype(np.float64), ref, f"tiny forward_logits M={M} plan{plan}")
    assert layer.device_error() == 0
    # the same layer fed the GPU's route gives the same output bits
    direct = layer.forward(bf16_dev(x), gids, gw)
    assert torch.equal(direct, out)


def test_route_k26(tiny):
    layer, _ = tiny
    from int4_weight_only_align_amd.w4moe import MoELayer
    big = MoELayer(K26.E, 256, 128, K26.topk, max_tokens=1024)   # routing needs no weights
    try:
        for M in (1, 90, 1024):
            logits = gen_logits(M, K26.E, 3400 + M)
            ids, w = big.route(to_dev(logits))
            torch.cuda.synchronize()
            _check_route(ids.cpu().numpy(), w.cpu().numpy().astype(np.float64), logits, K26.topk, f"E=384 M={M}")
    finally:
        big.close()


@pytest.mark.parametrize("M", [1, 4, 90])
def test_forward_logits_k26(M):
    layer, store = make_layer(K26, 2, max_tokens=128, tag="route k26")
    try:
        x = gen_hidden(M, K26.K, 3500 + M)
        logits = gen_logits(M, K26.E, 3600 + M)
        log(f"[route k26] M={M} plan={layer.resolved_plan(M)}")
        out, gids, gw = layer.forward_logits(bf16_dev(x), to_dev(logits))
        torch.cuda.synchronize()
        _check_route(gids.cpu().numpy(), gw.cpu().numpy().astype(np.float64), logits, K26.topk, f"k26 M={M}")
        rows = sorted({0, M // 2, M - 1})
        ids, w = route(logits, K26.topk)
        ref = moe_forward(K26, x, ids, w.astype(np.float32), store, rows=np.array(rows, np.int32))
        parity(out.float().cpu().numpy().astype(np.float64)[rows], ref, f"k26 forward_logits M={M}")
        assert layer.device_error() == 0
        assert torch.equal(layer.forward(bf16_dev(x), gids, gw), out)
    finally:
        layer.close()


def test_forward_logits_aligned_plans_many_tokens():
    """Routed calls of the aligned plans (router kernel, then alignment): up to 1024 tokens, repeated
    calls of different sizes, routes exact, and the layer fed the same route gives the same bits."""
    d = MoEDims(E=384, K=256, N=128, topk=8)
    layer, store = make_layer(d, 9, max_tokens=1024, tag="routed, aligned plans")
    try:
        for M in (9, 1024, 300, 1024, 17):
            logits = gen_logits(M, d.E, 3700 + M)
            x = gen_hidden(M, d.K, 3800 + M)
            for plan in (0, 1, 2):
                layer.set_plan(plan)
                log(f"[routed, aligned plans] M={M} plan={plan} (runs {layer.resolved_plan(M)})")
                out, gids, gw = layer.forward_logits(bf16_dev(x), to_dev(logits))
                torch.cuda.synchronize()
                _check_route(gids.cpu().numpy(), gw.cpu().numpy().astype(np.float64), logits, d.topk,
                             f"routed M={M} plan{plan}")
                assert torch.equal(layer.forward(bf16_dev(x), gids, gw), out), f"M={M} plan{plan}"
            rows = sorted({0, M // 2, M - 1})
            ids, w = route(logits, d.topk)
            ref = moe_forward(d, x, ids, w.astype(np.float32), store, rows=np.array(rows, np.int32))
            parity(out.float().cpu().numpy().astype(np.float64)[rows], ref, f"routed, aligned plans M={M}")
        assert layer.device_error() == 0
    finally:
        layer.close()
