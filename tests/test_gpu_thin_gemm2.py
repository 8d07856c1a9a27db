"""The aligned GEMM2 over a reduction of one or two group quads (N <= 256, a tensor-parallel shard's
width) walks several output superblocks per wave. Every output against the oracle, and bitwise equal
to the one-superblock-per-wave kernel (the same sums in the same order), for 4- and 8-bit codes, one
and two group quads, superblock counts that leave the last workgroup's waves ragged, and several
superblocks-per-wave settings (W4MOE_SBW, read when a layer is created; 1 selects the other kernel)."""
import numpy as np
import pytest

from oracle import moe_forward
from synth import MoEDims, gen_hidden, gen_routing_softmax
from tests.gpu_common import gpu_forward, log, make_layer, parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [96, 256])
@pytest.mark.parametrize("bits", [4, 8])
def test_thin_gemm2_matches_oracle_and_one_superblock_kernel(N, bits, monkeypatch):
    # K = 1472: 23 output superblocks of W2, so every setting below leaves a ragged last workgroup
    d = MoEDims(E=6, K=1472, N=N, topk=2, group=32, bits=bits)
    layers = {}
    try:
        for sbw in ("", "1", "3", "5"):
            if sbw:
                monkeypatch.setenv("W4MOE_SBW", sbw)
            else:
                monkeypatch.delenv("W4MOE_SBW", raising=False)
            layers[sbw], store = make_layer(d, 61, max_tokens=160, tag=f"thin N={N} w{bits} sbw={sbw or 'default'}")
        for M in (61, 150):   # 122 and 300 routed entries: past the single-launch limit, aligned plan
            x = gen_hidden(M, d.K, 6100 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 6200 + M)
            ref = moe_forward(d, x, ids, w, store)
            outs = {}
            for sbw, layer in layers.items():
                log(f"[thin N={N} w{bits}] M={M} sbw={sbw or 'default'}")
                outs[sbw] = gpu_forward(layer, x, ids, w, 4)
                assert layer.device_error() == 0
            parity(outs[""], ref, f"thin N={N} w{bits} M={M}")
            for sbw in ("", "3", "5"):
                assert np.array_equal(outs[sbw], outs["1"]), f"sbw={sbw or 'default'} M={M}"
    finally:
        for layer in layers.values():
            layer.close()
