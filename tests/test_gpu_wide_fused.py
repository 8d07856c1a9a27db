"""The wide plan in one launch (4-bit codes, work items of up to 48 rows): GEMM1 and GEMM2 workgroups in
one grid, each GEMM2 workgroup waiting for its work item's GEMM1 workgroups. Its outputs must be
bitwise those of the wide plan in two launches (the same sums in the same order; only the hand-off
differs), which W4MOE_WIDE_FUSED=0 selects when a layer is created, and within the bar of the oracle
(W4MOE_WIDE_FUSED=1 takes the single launch also where GEMM2 is not the thin kernel, which by default
runs in two launches).
Shapes: a GEMM2 over several group quads (the wide GEMM2) and over one or two (the thin one), padded
sizes, items of one to three tiles, uniform and Zipf routing, and one GPU's share of a TP8 layer at
M = 1024.

The bounded wait is driven to its give-up path from the host with a zero wait limit: every kernel
still ends normally, the call raises device flag bit 1, the output columns served by a GEMM2
workgroup that gave up read NaN, everything else in the call is the layer's own output, and the next
call with the default limit is exact again (every flag returns to zero within the call).
"""
from dataclasses import replace

import numpy as np
import pytest

from oracle import moe_forward
from synth import CONFIGS, MoEDims, gen_hidden, gen_routing, gen_routing_softmax
from tests.gpu_common import gpu_forward, log, make_layer, parity

pytestmark = pytest.mark.gpu


def _pair_of_layers(d, seed, max_tokens, tag, monkeypatch):
    monkeypatch.setenv("W4MOE_WIDE_FUSED", "1")
    one, store = make_layer(d, seed, max_tokens, tag=f"{tag} one launch")
    monkeypatch.setenv("W4MOE_WIDE_FUSED", "0")
    try:
        two, _ = make_layer(d, seed, max_tokens, tag=f"{tag} two launches")
    finally:
        monkeypatch.delenv("W4MOE_WIDE_FUSED", raising=False)
    return one, two, store


@pytest.mark.parametrize("d", [
    MoEDims(E=12, K=1024, N=512, topk=4),   # GEMM2 over four group quads: the wide GEMM2
    MoEDims(E=12, K=1024, N=256, topk=4),   # two group quads: the thin GEMM2
    MoEDims(E=5, K=544, N=96, topk=2),      # padded hidden and intermediate sizes, one group quad
], ids=["wide-g2", "thin-g2", "padded"])
def test_one_launch_equals_two_launches(d, monkeypatch):
    one, two, store = _pair_of_layers(d, 71, 300, f"wide fused E={d.E} K={d.K} N={d.N}", monkeypatch)
    try:
        for M, kind in ((31, "softmax"), (100, "softmax"), (300, "softmax"), (300, "zipf")):
            if M * d.topk <= 120:
                continue   # the single-launch pair mode's range
            x = gen_hidden(M, d.K, 7300 + M)
            ids, w = gen_routing(kind, M, d.E, d.topk, 7400 + M)
            assert one.resolved_plan(M) == 4 and two.resolved_plan(M) == 4
            log(f"[wide fused E={d.E} K={d.K} N={d.N}] M={M} {kind}")
            a = gpu_forward(one, x, ids, w, 4)
            b = gpu_forward(two, x, ids, w, 4)
            assert one.device_error() == 0 and two.device_error() == 0
            assert np.array_equal(a, b), f"M={M} {kind}: one launch differs from two"
            parity(a, moe_forward(d, x, ids, w, store), f"wide fused N={d.N} M={M} {kind}")
    finally:
        one.close()
        two.close()


@pytest.mark.parametrize("kind", ["softmax", "zipf"])
def test_tp8_shard_m1024_one_launch_equals_two(kind, monkeypatch):
    d = CONFIGS["k26_tp8"]
    M = 1024
    one, two, store = _pair_of_layers(d, 5, M, f"TP8 shard {kind}", monkeypatch)
    try:
        x = gen_hidden(M, d.K, 7500)
        ids, w = gen_routing(kind, M, d.E, d.topk, 7600)
        log(f"[TP8 shard wide fused] M={M} {kind}")
        a = gpu_forward(one, x, ids, w, 4)
        b = gpu_forward(two, x, ids, w, 4)
        assert one.device_error() == 0 and two.device_error() == 0
        assert np.array_equal(a, b), f"TP8 M={M} {kind}: one launch differs from two"
        rows = [0, 511, M - 1]
        parity(a[rows], moe_forward(d, x[rows], ids[rows], w[rows], store), f"TP8 wide fused M={M} {kind} rows")
    finally:
        one.close()
        two.close()


@pytest.mark.parametrize("cfg", ["k26", "k26_tp8"])
def test_wide_wait_limit_zero_poisons_and_recovers(cfg, monkeypatch):
    # eight experts at K2.6 hidden width, top-4, M = 40: 160 routed entries (the wide plan), 8 items of
    # about 20 rows. K2.6: 128 GEMM1 and 224 GEMM2 workgroups (the wide GEMM2, in one launch only when
    # asked); TP8 shard (N = 256): 16 and 112 (the thin GEMM2, one launch by default). All are resident
    # at once, so GEMM2 workgroups reach their wait while GEMM1 streams.
    d = replace(CONFIGS[cfg], E=8, topk=4)
    M = 40
    if cfg == "k26":
        monkeypatch.setenv("W4MOE_WIDE_FUSED", "1")
    layer, store = make_layer(d, 2, max_tokens=M, tag=f"{cfg} width, 8 experts, wide plan")
    monkeypatch.delenv("W4MOE_WIDE_FUSED", raising=False)
    try:
        x = gen_hidden(M, d.K, 7700)
        ids, w = gen_routing_softmax(M, d.E, d.topk, 7800)
        assert layer.resolved_plan(M) == 4
        good = gpu_forward(layer, x, ids, w, 4)
        assert layer.device_error() == 0
        rows = [0, M - 1]
        parity(good[rows], moe_forward(d, x[rows], ids[rows], w[rows], store), "wide wait limit reference rows")
        gave_up = False
        for attempt in range(3):
            log(f"[wide wait limit] call {attempt} with a zero limit")
            layer.set_wait_limit(0)
            try:
                cut = gpu_forward(layer, x, ids, w, 4)
                flags = layer.device_error()
            finally:
                layer.set_wait_limit(-1)
            nan = np.isnan(cut)
            log(f"[wide wait limit] flags={flags}, NaN outputs {int(nan.sum())} of {nan.size}")
            # a GEMM2 workgroup serves whole 64-column superblocks of its item's tokens
            assert bool(flags & 2) == bool(nan.any())
            blocks = nan.reshape(M, d.K // 64, 64)
            assert (blocks.all(axis=2) | ~blocks.any(axis=2)).all()
            assert np.array_equal(cut[~nan], good[~nan])
            if flags & 2:
                gave_up = True
                break
        assert gave_up, "no wait gave up in three calls although GEMM2 workgroups start beside GEMM1"
        again = gpu_forward(layer, x, ids, w, 4)
        assert layer.device_error() == 0
        assert np.array_equal(again, good)
        ids2, w2 = gen_routing_softmax(M, d.E, d.topk, 7900)
        nxt = gpu_forward(layer, x, ids2, w2, 4)
        assert layer.device_error() == 0
        parity(nxt[rows], moe_forward(d, x[rows], ids2[rows], w2[rows], store), "wide wait limit after")
    finally:
        layer.close()
