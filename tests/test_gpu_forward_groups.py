"""Scale groups of 64 and 128 rows (and 32 for reference) on a small layer (E=8, K=512, N=256,
top-2): every output of every plan against the oracle, ragged and multi-tile token counts."""
import numpy as np
import pytest

from oracle import moe_forward
from synth import MoEDims, gen_hidden, gen_routing_softmax
from tests.gpu_common import gpu_forward, log, make_layer, parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("group", [32, 64, 128])
def test_forward_group_sizes(group):
    d = MoEDims(E=8, K=512, N=256, topk=2, group=group)
    layer, store = make_layer(d, 17, max_tokens=128, tag=f"group {group}")
    try:
        for M in (1, 16, 100):
            x = gen_hidden(M, d.K, 5000 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 5100 + M)
            ref = moe_forward(d, x, ids, w, store)
            for plan in (0, 1, 2, 3, 4, 5):
                log(f"[group {group}] M={M} plan={plan}")
                parity(gpu_forward(layer, x, ids, w, plan), ref, f"group {group} M={M} plan{plan}")
            assert layer.device_error() == 0
    finally:
        layer.close()
