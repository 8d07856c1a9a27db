"""Reduction dimensions that are multiples of the scale group but not of the 128-row block (K and N
of 32 * odd, W2 widths not a multiple of 64): the library pads the packed weights to whole blocks
(zero codes, zero scales) and the hidden rows with zeros. Every output of every plan against the
oracle at M = 1, 16 and 100, for 4- and 8-bit codes, groups of 32 and 64, and activation order; and
the no-allocation forward on a padded shape."""
import numpy as np
import pytest
import torch

from oracle import moe_forward
from synth import MoEDims, gen_hidden, gen_routing_softmax
from tests.gpu_common import bf16_dev, gpu_forward, log, make_layer, make_layer_act_order, parity, to_dev

pytestmark = pytest.mark.gpu

SHAPES = {
    "K160-N96": MoEDims(E=8, K=160, N=96, topk=2),
    "K160-N96-w8": MoEDims(E=8, K=160, N=96, topk=2, bits=8),
    "K96-N32-top3": MoEDims(E=5, K=96, N=32, topk=3),
    "K192-N320-g64": MoEDims(E=6, K=192, N=320, topk=2, group=64),
    "K2080-N416": MoEDims(E=4, K=2080, N=416, topk=2),
}


def _run_all_plans(layer, store, d, tag):
    for M in (1, 16, 100):
        x = gen_hidden(M, d.K, 6000 + M)
        ids, w = gen_routing_softmax(M, d.E, d.topk, 6100 + M)
        ref = moe_forward(d, x, ids, w, store)
        outs = []
        for plan in (0, 1, 2, 3, 4, 5):
            log(f"[{tag}] M={M} plan={plan}")
            got = gpu_forward(layer, x, ids, w, plan)
            parity(got, ref, f"{tag} M={M} plan{plan}")
            outs.append(got)
        assert layer.device_error() == 0


@pytest.mark.parametrize("name", list(SHAPES))
def test_padded_shapes_every_plan(name):
    d = SHAPES[name]
    layer, store = make_layer(d, 23, max_tokens=128, tag=f"padded {name}")
    try:
        _run_all_plans(layer, store, d, f"padded {name}")
    finally:
        layer.close()


@pytest.mark.parametrize("bits", [4, 8])
def test_padded_shape_act_order(bits):
    d = MoEDims(E=8, K=160, N=96, topk=2, bits=bits)
    layer, store = make_layer_act_order(d, 29, max_tokens=128, tag=f"padded act order {bits}-bit")
    try:
        _run_all_plans(layer, store, d, f"padded act order {bits}-bit")
    finally:
        layer.close()


def test_padded_shape_noalloc():
    d = SHAPES["K160-N96"]
    layer, store = make_layer(d, 23, max_tokens=64, tag="padded noalloc")
    try:
        for M in (32, 5):
            x = gen_hidden(M, d.K, 6200 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 6300 + M)
            out = torch.full((M, d.K), float("nan"), dtype=torch.bfloat16, device="cuda")
            layer.forward_noalloc(bf16_dev(x), to_dev(ids), to_dev(w), out)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy().astype(np.float64)
            assert np.array_equal(got, gpu_forward(layer, x, ids, w, 3))
            parity(got, moe_forward(d, x, ids, w, store), f"padded noalloc M={M}")
    finally:
        layer.close()
