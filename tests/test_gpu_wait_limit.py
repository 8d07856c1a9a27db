"""The single-launch pair mode's bounded hand-off wait, driven to its give-up path from the host.

`w4moe_set_wait_limit(h, 0)` makes every GEMM2 workgroup that does not find its entry's GEMM1 done at
the first look give up at once: every kernel still ends normally, the call raises device flag bit 1,
and the output columns served by a workgroup that gave up read NaN. Everything else in that call's
output, and every later call, must be exactly what the layer computes without a limit (the per-entry
hand-off state returns to zero within the call). The layer is eight experts at K2.6 width with top-4
routing: at M = 1 and 2 (4 and 8 routed entries) GEMM1 has 256 and 512 workgroups, fewer than the
768 the GPU holds at once, so GEMM2 workgroups are resident from the start and reach their wait
microseconds into a GEMM1 that streams 66 or 132 MB. Up to three calls with the zero limit are made
(each is checked); at least one of them must give up.
"""
from dataclasses import replace

import numpy as np
import pytest

from oracle import moe_forward
from synth import CONFIGS, gen_hidden, gen_routing_softmax
from tests.gpu_common import gpu_forward, log, make_layer, parity

pytestmark = pytest.mark.gpu
DIMS = replace(CONFIGS["k26"], E=8, topk=4)


@pytest.fixture(scope="module")
def layer8():
    layer, store = make_layer(DIMS, 2, max_tokens=8, tag="k26 width, 8 experts")
    yield layer, store
    layer.close()


@pytest.mark.parametrize("M", [1, 2])
def test_wait_limit_zero_poisons_and_recovers(layer8, M):
    layer, store = layer8
    x = gen_hidden(M, DIMS.K, 1000 + M)
    ids, w = gen_routing_softmax(M, DIMS.E, DIMS.topk, 7000 + M)
    assert layer.resolved_plan(M) == 3
    log(f"[wait limit] M={M}: reference call (default limit)")
    good = gpu_forward(layer, x, ids, w, 3)
    assert layer.device_error() == 0
    parity(good, moe_forward(DIMS, x, ids, w, store), f"wait limit M={M} reference")

    gave_up = False
    for attempt in range(3):
        log(f"[wait limit] M={M}: call {attempt} with a zero limit")
        layer.set_wait_limit(0)
        try:
            cut = gpu_forward(layer, x, ids, w, 3)
            flags = layer.device_error()
        finally:
            layer.set_wait_limit(-1)
        nan = np.isnan(cut)
        log(f"[wait limit] M={M}: flags={flags}, NaN outputs {int(nan.sum())} of {nan.size}")
        # NaN exactly when some wait gave up; a workgroup serves 64 output columns of one token, so
        # the poison covers whole column blocks; every value not poisoned is the layer's own
        assert bool(flags & 2) == bool(nan.any())
        blocks = nan.reshape(M, DIMS.K // 64, 64)
        assert (blocks.all(axis=2) | ~blocks.any(axis=2)).all()
        assert np.array_equal(cut[~nan], good[~nan])
        if flags & 2:
            gave_up = True
            break
    assert gave_up, "no wait gave up in three calls although GEMM2 workgroups start beside GEMM1"

    log(f"[wait limit] M={M}: next call with the default limit")
    again = gpu_forward(layer, x, ids, w, 3)
    assert layer.device_error() == 0
    assert np.array_equal(again, good)
    # a different routing right after, against the oracle
    ids2, w2 = gen_routing_softmax(M, DIMS.E, DIMS.topk, 7100 + M)
    nxt = gpu_forward(layer, x, ids2, w2, 3)
    assert layer.device_error() == 0
    parity(nxt, moe_forward(DIMS, x, ids2, w2, store), f"wait limit M={M} after")
