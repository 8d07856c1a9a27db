"""Seeded shapes off the workloads' grid against the oracle: expert counts, hidden and intermediate
sizes that are any multiple of the scale group (so blocks, superblock groups and reduction splits
come out ragged and padded), top-k from 1 to 8, scale groups 32/64/128, 4- and 8-bit codes,
consecutive and activation-ordered groups, every plan, and token counts on both sides of the
single-launch limit."""
import numpy as np
import pytest

from oracle import moe_forward
from synth import MoEDims, gen_hidden, gen_routing_softmax
from tests.gpu_common import gpu_forward, log, make_layer, make_layer_act_order, parity

pytestmark = pytest.mark.gpu


def _cases(n=20, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([2, 3, 5, 12, 33, 64]))
        group = int(rng.choice([32, 64, 128]))
        K = group * int(rng.integers(1, 1024 // group + 1))   # 32 .. 1024: partial group quads padded
        N = group * int(rng.integers(1, 512 // group + 1))    # 32 .. 512: W1 superblocks 1 .. 16
        topk = int(rng.integers(1, min(E, 8) + 1))
        bits = int(rng.choice([4, 8]))
        act = bool(rng.integers(0, 2))
        Ms = sorted({1, int(rng.integers(2, 9)), int(rng.integers(9, 80)), int(rng.integers(80, 200))})
        out.append(pytest.param(MoEDims(E=E, K=K, N=N, topk=topk, group=group, bits=bits), act, Ms,
                                id=f"{i}-E{E}-K{K}-N{N}-k{topk}-g{group}-w{bits}{'-ao' if act else ''}"))
    return out


@pytest.mark.parametrize("d,act,Ms", _cases())
def test_random_shape_every_plan(d, act, Ms):
    tag = f"random E={d.E} K={d.K} N={d.N} k={d.topk} g={d.group} w{d.bits}{' act order' if act else ''}"
    maker = make_layer_act_order if act else make_layer
    layer, store = maker(d, 100 + d.E + d.K, max_tokens=max(Ms), tag=tag)
    try:
        for M in Ms:
            x = gen_hidden(M, d.K, 9000 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 9100 + M)
            ref = moe_forward(d, x, ids, w, store)
            for plan in (0, 1, 2, 3, 4, 5):
                log(f"[{tag}] M={M} plan={plan}")
                parity(gpu_forward(layer, x, ids, w, plan), ref, f"{tag} M={M} plan{plan}")
        assert layer.device_error() == 0
    finally:
        layer.close()
