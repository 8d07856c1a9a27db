"""The no-allocation forward (w4moe_forward_noalloc): the same layer as w4moe_forward, with the call's
workspace in the library's static per-GPU scratch array instead of the handle's workspace.

Checked through the C-ABI against w4moe_forward on the same inputs (bit for bit: the same kernels in
the same order) and against the oracle (the layer's parity bar), on two calls in a row where the
second is smaller, for two shapes that lay the scratch array out differently; then interleaved with
w4moe_forward calls; then the sizes it must refuse, with their errors.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import moe_forward
from synth import CONFIGS, gen_hidden, gen_routing_softmax
from tests.gpu_common import bf16_dev, log, make_layer, parity, to_dev

pytestmark = pytest.mark.gpu
TINY = CONFIGS["tiny"]
WIDE8 = replace(CONFIGS["k26"], E=8)   # K2.6 width, eight experts


def _inputs(dims, M, seed):
    x = gen_hidden(M, dims.K, 1000 + seed)
    ids, w = gen_routing_softmax(M, dims.E, dims.topk, 9000 + seed)
    return x, ids, w


def _both(layer, dims, x, ids, w):
    """(no-allocation result, w4moe_forward result) as float64 arrays."""
    from int4_weight_only_align_amd.w4moe import W4MoEError  # noqa: F401
    M = x.shape[0]
    dx, di, dw = bf16_dev(x), to_dev(ids), to_dev(w)
    out_na = torch.full((M, dims.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    layer.forward_noalloc(dx, di, dw, out_na)
    torch.cuda.synchronize()
    layer.set_plan(3)
    out_ref = layer.forward(dx, di, dw)
    layer.set_plan(0)
    torch.cuda.synchronize()
    return (out_na.float().cpu().numpy().astype(np.float64), out_ref.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("name,dims,sizes,seed", [("tiny", TINY, (32, 3), 1), ("k26 width", WIDE8, (8, 1), 2)])
def test_noalloc_matches_forward_two_calls(name, dims, sizes, seed):
    layer, store = make_layer(dims, seed, max_tokens=64, tag=f"noalloc {name}")
    try:
        for M in sizes:   # the second call is smaller than the first
            log(f"[noalloc {name}] M={M}")
            x, ids, w = _inputs(dims, M, M)
            got, ref = _both(layer, dims, x, ids, w)
            assert np.array_equal(got, ref), f"{name} M={M}: differs from w4moe_forward"
            parity(got, moe_forward(dims, x, ids, w, store), f"noalloc {name} M={M}")
            assert layer.device_error() == 0
    finally:
        layer.close()


def test_noalloc_interleaved_with_forward():
    layer, store = make_layer(TINY, 1, max_tokens=64, tag="noalloc interleaved")
    try:
        for r, M in enumerate((5, 32, 1, 17)):
            log(f"[noalloc interleaved] round {r} M={M}")
            x, ids, w = _inputs(TINY, M, 40 + r)
            got, ref = _both(layer, TINY, x, ids, w)
            assert np.array_equal(got, ref)
            parity(got, moe_forward(TINY, x, ids, w, store), f"noalloc interleaved M={M}")
        assert layer.device_error() == 0
    finally:
        layer.close()


def test_noalloc_refuses_what_does_not_fit():
    from int4_weight_only_align_amd.w4moe import W4MoEError
    layer, _ = make_layer(TINY, 1, max_tokens=128, tag="noalloc limits")
    try:
        M = 40   # 80 routed entries > 64
        x, ids, w = _inputs(TINY, M, 3)
        out = torch.empty((M, TINY.K), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(W4MoEError) as ei:
            layer.forward_noalloc(bf16_dev(x), to_dev(ids), to_dev(w), out)
        assert ei.value.status == 2 and "64" in str(ei.value)
        x0 = torch.empty((0, TINY.K), dtype=torch.bfloat16, device="cuda")
        i0 = torch.empty((0, TINY.topk), dtype=torch.int32, device="cuda")
        w0 = torch.empty((0, TINY.topk), dtype=torch.float32, device="cuda")
        layer.forward_noalloc(x0, i0, w0, torch.empty((0, TINY.K), dtype=torch.bfloat16, device="cuda"))
    finally:
        layer.close()
    # rows too wide for the array's data zone: K = 22528, 64 entries need 64 * 22528 * 4 B of slot outputs
    big = replace(TINY, E=2, K=22528, N=128, topk=2)
    from int4_weight_only_align_amd.w4moe import MoELayer
    lb = MoELayer(big.E, big.K, big.N, big.topk, max_tokens=32)
    try:
        M = 32
        x = torch.zeros((M, big.K), dtype=torch.bfloat16, device="cuda")
        ids = torch.zeros((M, big.topk), dtype=torch.int32, device="cuda")
        ids[:, 1] = 1
        w = torch.full((M, big.topk), 0.5, dtype=torch.float32, device="cuda")
        out = torch.empty((M, big.K), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(W4MoEError) as ei:   # not prepacked: refused before the size check
            lb.forward_noalloc(x, ids, w, out)
        assert ei.value.status == 3
        z1 = torch.zeros((big.E, big.K // 8, 2 * big.N), dtype=torch.int32, device="cuda")
        s1 = torch.zeros((big.E, big.K // 32, 2 * big.N), dtype=torch.bfloat16, device="cuda")
        z2 = torch.zeros((big.E, big.N // 8, big.K), dtype=torch.int32, device="cuda")
        s2 = torch.zeros((big.E, big.N // 32, big.K), dtype=torch.bfloat16, device="cuda")
        lb.prepack(z1, s1, z2, s2)
        with pytest.raises(W4MoEError) as ei:
            lb.forward_noalloc(x, ids, w, out)
        assert ei.value.status == 2 and "scratch" in str(ei.value)
        lb.forward_noalloc(x[:4], ids[:4], w[:4], out[:4])   # 8 entries fit
        torch.cuda.synchronize()
        assert (out[:4].float() == 0).all()
    finally:
        lb.close()
