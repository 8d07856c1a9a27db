"""Activation-ordered (GPTQ act-order) weights on the GPU: every plan against the oracle, which takes
the checkpoint's group index per row while the library takes the group-order permutation; the
prepacked layout; the routed call; the entry-point guards and the out-of-range flag."""
import numpy as np
import pytest
import torch

from oracle import moe_forward
from synth import MoEDims, gen_act_order, gen_expert, gen_hidden, gen_logits, gen_routing_softmax
from tests.gpu_common import (bf16_dev, gpu_forward, group_order, log, make_layer, make_layer_act_order, parity,
                              to_dev)
from tests.packing import decode_packed, unpack_codes

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("group,bits", [(32, 4), (128, 4), (64, 8)])
def test_act_order_small_every_plan(group, bits):
    d = MoEDims(E=8, K=512, N=256, topk=2, group=group, bits=bits)
    layer, store = make_layer_act_order(d, 31, max_tokens=128, tag=f"act order g{group} w{bits}")
    try:
        for M in (1, 16, 100):
            x = gen_hidden(M, d.K, 7000 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 7100 + M)
            ref = moe_forward(d, x, ids, w, store)
            for plan in (0, 1, 2, 3, 4, 5):
                log(f"[act order g{group} w{bits}] M={M} plan={plan}")
                parity(gpu_forward(layer, x, ids, w, plan), ref, f"act order g{group} w{bits} M={M} plan{plan}")
            assert layer.device_error() == 0
    finally:
        layer.close()


def test_act_order_full_width():
    d = MoEDims(E=16, K=7168, N=2048, topk=8)
    layer, store = make_layer_act_order(d, 37, max_tokens=128, tag="act order full width")
    try:
        for M, plans in ((1, (0, 5)), (100, (0, 1))):
            x = gen_hidden(M, d.K, 7200 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 7300 + M)
            rows = sorted({0, M // 2, M - 1})
            ref = moe_forward(d, x, ids, w, store, rows=np.array(rows, np.int32))
            for plan in plans:
                log(f"[act order full width] M={M} plan={plan}")
                got = gpu_forward(layer, x, ids, w, plan)[rows]
                parity(got, ref, f"act order full width M={M} plan{plan}")
        assert layer.device_error() == 0
    finally:
        layer.close()


def test_act_order_prepacked_layout():
    """Packed W1 row i / column c holds logical row perm1[i] of column perm2-mapped c; W2 row i holds
    logical row perm2[i]; the scales are those of the rows' groups."""
    d = MoEDims(E=3, K=256, N=128, topk=1, group=64)
    layer, store = make_layer_act_order(d, 41, max_tokens=4, tag="act order layout")
    try:
        dec = {}
        for which, kind, R, Cc in ((1, "w1", d.K, 2 * d.N), (2, "w2", d.N, d.K)):
            dec[kind] = decode_packed(layer.packed_bytes(which).cpu().numpy(), kind, d.E, R, Cc, d.N)
        for e in range(d.E):
            w1, s1, w2, s2, g1, g2 = store[e]
            p1, p2 = group_order(g1), group_order(g2)
            cols = np.concatenate([p2, d.N + p2])
            codes1, sc1 = dec["w1"][0][e], dec["w1"][1][e]
            assert np.array_equal(codes1, unpack_codes(w1)[p1][:, cols])
            assert np.array_equal(sc1, s1[(np.arange(d.K // 32) * 32) // d.group][:, cols])
            codes2, sc2 = dec["w2"][0][e], dec["w2"][1][e]
            assert np.array_equal(codes2, unpack_codes(w2)[p2])
            assert np.array_equal(sc2, s2[(np.arange(d.N // 32) * 32) // d.group])
        assert layer.device_error() == 0
    finally:
        layer.close()


def test_act_order_routed_layer_and_dropped_ids():
    d = MoEDims(E=8, K=512, N=256, topk=2)
    layer, store = make_layer_act_order(d, 43, max_tokens=128, tag="act order routed")
    try:
        for M in (1, 40, 100):
            logits = torch.from_numpy(gen_logits(M, d.E, 7400 + M)).cuda()
            x = gen_hidden(M, d.K, 7500 + M)
            for plan in (0, 3, 5, 4):
                layer.set_plan(plan)
                out, ids, w = layer.forward_logits(bf16_dev(x), logits)
                torch.cuda.synchronize()
                again = gpu_forward(layer, x, ids.cpu().numpy(), w.cpu().numpy(), plan)
                assert np.array_equal(out.float().cpu().numpy().astype(np.float64), again), f"M={M} plan={plan}"
                parity(again, moe_forward(d, x, ids.cpu().numpy(), w.cpu().numpy(), store),
                       f"act order routed M={M} plan{plan}")
        assert layer.device_error() == 0
        # a dropped id adds nothing: compare with the same slot routed anywhere at weight 0
        M = 20
        x = gen_hidden(M, d.K, 7600)
        ids, w = gen_routing_softmax(M, d.E, d.topk, 7601)
        bad = ids.copy()
        bad[3, 1] = -1
        ref_ids, ref_w = ids.copy(), w.copy()
        ref_w[3, 1] = 0.0
        ref = moe_forward(d, x, ref_ids, ref_w, store)
        for plan in (0, 3, 4):
            parity(gpu_forward(layer, x, bad, w, plan), ref, f"act order dropped id plan{plan}")
            assert layer.device_error() & 1
    finally:
        layer.close()


def test_act_order_entry_point_guards_and_range_flag():
    from int4_weight_only_align_amd.w4moe import W4MoEError
    d = MoEDims(E=2, K=256, N=128, topk=1)
    plain, _ = make_layer(d, 47, max_tokens=4, tag="plain layer guard")
    layer, _ = make_layer_act_order(d, 47, max_tokens=4, tag="act order guard")
    try:
        w1, s1, w2, s2 = gen_expert(d, 0, 47)
        g1, g2 = gen_act_order(d, 0, 47)
        args = (to_dev(w1[None]), bf16_dev(s1[None]), to_dev(w2[None]), bf16_dev(s2[None]))
        perms = (to_dev(group_order(g1)[None]), to_dev(group_order(g2)[None]))
        with pytest.raises(W4MoEError) as ei:
            layer.prepack(*args)
        assert ei.value.status == 1
        with pytest.raises(W4MoEError) as ei:
            plain.prepack_act_order(args[0], args[1], perms[0], args[2], args[3], perms[1])
        assert ei.value.status == 1
        # a value outside [0, K) is read as row 0 and flagged; nothing is read out of bounds
        p1 = group_order(g1)
        p1[5] = d.K + 3
        layer.prepack_act_order(args[0], args[1], to_dev(p1[None]), args[2], args[3], perms[1])
        torch.cuda.synchronize()
        assert layer.device_error() & 4
        assert layer.device_error() == 0
    finally:
        layer.close()
        plain.close()
