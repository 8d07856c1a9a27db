"""8-bit weights (W8A16): every plan against the oracle on a small layer at groups 32 and 128, and
the full K2.6 width (K=7168, N=2048) with 16 experts for the decode and wide paths."""
import numpy as np
import pytest

from oracle import moe_forward
from synth import MoEDims, gen_hidden, gen_routing_softmax
from tests.gpu_common import gpu_forward, log, make_layer, parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("group", [32, 128])
def test_w8_small_every_plan(group):
    d = MoEDims(E=8, K=512, N=256, topk=2, group=group, bits=8)
    layer, store = make_layer(d, 23, max_tokens=128, tag=f"w8 group {group}")
    try:
        for M in (1, 16, 100):
            x = gen_hidden(M, d.K, 6000 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 6100 + M)
            ref = moe_forward(d, x, ids, w, store)
            for plan in (0, 1, 2, 3, 4, 5):
                log(f"[w8 group {group}] M={M} plan={plan}")
                got = gpu_forward(layer, x, ids, w, plan)
                parity(got, ref, f"w8 group {group} M={M} plan{plan}")
            assert layer.device_error() == 0
    finally:
        layer.close()


def test_w8_full_width():
    d = MoEDims(E=16, K=7168, N=2048, topk=8, bits=8)
    layer, store = make_layer(d, 29, max_tokens=128, tag="w8 full width")
    try:
        for M, plans in ((1, (0, 5)), (100, (0, 1))):
            x = gen_hidden(M, d.K, 6200 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 6300 + M)
            rows = sorted({0, M // 2, M - 1})
            ref = moe_forward(d, x, ids, w, store, rows=np.array(rows, np.int32))
            for plan in plans:
                log(f"[w8 full width] M={M} plan={plan}")
                got = gpu_forward(layer, x, ids, w, plan)
                assert np.isfinite(got).all()
                parity(got[rows], ref, f"w8 full width M={M} plan{plan}")
            assert layer.device_error() == 0
    finally:
        layer.close()
