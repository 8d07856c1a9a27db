"""Expert parallelism, one GPU's share: a layer holding experts [first, first + E_s) of a larger layer
(w4moe_set_expert_range) and fed global routing ids. Its output must be the shard's partial sum, i.e.
the oracle's layer with every slot routed to another shard weighted 0 (those slots add exactly
nothing), and the shards' outputs must add up to the whole layer. Other shards' ids raise no flag;
ids outside the whole layer still do. Tiny workload (E = 8, top-2) over every plan, shards of
activation-ordered and 8-bit layers, the router under a range, the alignment's local histogram, and
one EP8 share of the K2.6 layer (48 of 384 experts)."""
import numpy as np
import pytest
import torch

from oracle import moe_align, moe_forward
from synth import (CONFIGS, ExpertStore, MoEDims, gen_act_order, gen_expert, gen_hidden, gen_logits, gen_routing_softmax,
                   gen_routing_zipf)
from tests.gpu_common import bf16_dev, gpu_forward, group_order, log, parity, to_dev
from tests.shards import shard_ref

pytestmark = pytest.mark.gpu
D = CONFIGS["tiny"]
K26 = CONFIGS["k26"]
# (first expert, experts held): four even shards of the tiny layer
SHARDS = [(0, 2), (2, 2), (4, 2), (6, 2)]


def make_shard(dims, seed, first, n, max_tokens, tag, act_order=False):
    """A layer holding the seeded experts [first, first + n) of `dims` at local indices 0 .. n-1 (with
    act_order, prepacked with their seeded group orders, as the caller of the library does)."""
    from int4_weight_only_align_amd.w4moe import MoELayer
    log(f"[{tag}] shard: experts {first}..{first + n - 1} of {dims.E}")
    layer = MoELayer(n, dims.K, dims.N, dims.topk, max_tokens, group_size=dims.group, num_bits=dims.bits,
                     act_order=act_order)
    for e0 in range(0, n, 16):
        es = range(first + e0, first + min(n, e0 + 16))
        parts = [gen_expert(dims, e, seed) for e in es]
        st = [np.stack([p[k] for p in parts]) for k in range(4)]
        if act_order:
            orders = [gen_act_order(dims, e, seed) for e in es]
            p1 = np.stack([group_order(o[0]) for o in orders])
            p2 = np.stack([group_order(o[1]) for o in orders])
            layer.prepack_act_order(to_dev(st[0]), bf16_dev(st[1]), to_dev(p1), to_dev(st[2]), bf16_dev(st[3]),
                                    to_dev(p2), first_expert=e0)
        else:
            layer.prepack(to_dev(st[0]), bf16_dev(st[1]), to_dev(st[2]), bf16_dev(st[3]), first_expert=e0)
        torch.cuda.synchronize()
    layer.set_expert_range(first, dims.E)
    return layer


@pytest.fixture(scope="module")
def tiny_shards():
    layers = [make_shard(D, 1, f, n, 256, "tiny") for f, n in SHARDS]
    yield layers
    for layer in layers:
        layer.close()


@pytest.mark.parametrize("plan", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("M", [1, 16, 100])
def test_tiny_shards_match_oracle_and_add_up(tiny_shards, M, plan):
    store = ExpertStore(D, 1)
    x = gen_hidden(M, D.K, 700 + M)
    ids, w = gen_routing_softmax(M, D.E, D.topk, 710 + M)
    total = np.zeros((M, D.K))
    for (first, n), layer in zip(SHARDS, tiny_shards):
        layer.device_error()
        got = gpu_forward(layer, x, ids, w, plan)
        assert layer.device_error() == 0, "another shard's ids raised the flag"
        parity(got, shard_ref(D, x, ids, w, store, first, n), f"tiny shard {first}+{n} M={M} plan{plan}")
        total += got
    parity(total, moe_forward(D, x, ids, w, store), f"tiny shards summed M={M} plan{plan}")


def test_tiny_uneven_shard_and_unrouted_tokens():
    """Three experts (5..7); tokens routed only to other shards come out exactly zero."""
    store = ExpertStore(D, 1)
    layer = make_shard(D, 1, 5, 3, 64, "tiny uneven")
    M = 24
    x = gen_hidden(M, D.K, 720)
    ids, w = gen_routing_softmax(M, D.E, D.topk, 721)
    ids[3] = [0, 1]
    ids[10] = [2, 4]
    for plan in (1, 2, 3, 4, 5):
        got = gpu_forward(layer, x, ids, w, plan)
        assert layer.device_error() == 0
        assert not got[3].any() and not got[10].any(), f"plan {plan}: a token with no local slot is not zero"
        parity(got, shard_ref(D, x, ids, w, store, 5, 3), f"tiny uneven shard plan{plan}")
    layer.close()


@pytest.mark.parametrize("act_order,bits,group", [(True, 4, 32), (False, 8, 64), (True, 8, 128)])
def test_shards_with_activation_order_and_eight_bit_codes(act_order, bits, group):
    """The expert range through the act-order gathers (pair-mode staging, the aligned plans' gather
    kernel) and the 8-bit decode: two shards of 3 and 5 experts, every plan, M = 1, 16, 100."""
    d = MoEDims(E=8, K=512, N=256, topk=2, group=group, bits=bits)
    store = ExpertStore(d, 33, act_order=act_order)
    shards = [(0, 3), (3, 5)]
    layers = [make_shard(d, 33, f, n, 128, f"shard ao={act_order} w{bits} g{group}", act_order) for f, n in shards]
    try:
        for M in (1, 16, 100):
            x = gen_hidden(M, d.K, 760 + M)
            ids, w = gen_routing_softmax(M, d.E, d.topk, 770 + M)
            full = moe_forward(d, x, ids, w, store)
            for plan in (0, 1, 2, 3, 4, 5):
                total = np.zeros_like(full)
                for (first, n), layer in zip(shards, layers):
                    got = gpu_forward(layer, x, ids, w, plan)
                    assert layer.device_error() == 0
                    parity(got, shard_ref(d, x, ids, w, store, first, n), f"shard {first}+{n} M={M} plan{plan}")
                    total += got
                parity(total, full, f"shards summed M={M} plan{plan}")
    finally:
        for layer in layers:
            layer.close()


def test_tiny_shard_flags_only_ids_outside_the_whole_layer():
    store = ExpertStore(D, 1)
    layer = make_shard(D, 1, 2, 2, 64, "tiny flags")
    M = 12
    x = gen_hidden(M, D.K, 730)
    ids, w = gen_routing_softmax(M, D.E, D.topk, 731)
    bad = ids.copy()
    bad[1, 0], bad[4, 1], bad[7, 0] = D.E, -1, 1 << 30
    ok = (bad >= 0) & (bad < D.E)
    ref = shard_ref(D, x, np.where(ok, bad, 0).astype(np.int32), np.where(ok, w, 0).astype(np.float32), store, 2, 2)
    for plan in (1, 2, 3, 4, 5):
        layer.device_error()
        got = gpu_forward(layer, x, bad, w, plan)
        assert layer.device_error() == 1, f"plan {plan}"
        parity(got, ref, f"tiny shard, ids outside the layer, plan{plan}")
    layer.close()


def test_tiny_shard_alignment_is_the_local_histogram(tiny_shards):
    """moe_align under a range: local expert e is global first + e, other shards' ids are dropped --
    bit-exact against the oracle's alignment with every remote entry given to one extra expert n
    placed after the local ones (which leaves the local counts, offsets, flat ids and the sentinel T
    as they are)."""
    for M in (1, 16, 100, 256):
        ids, _ = gen_routing_softmax(M, D.E, D.topk, 740 + M)
        for (first, n), layer in zip(SHARDS, tiny_shards):
            local = ids.astype(np.int64) - first
            local = np.where((local >= 0) & (local < n), local, n).astype(np.int32)
            for B in (1, 16):
                got = layer.moe_align(to_dev(ids), B)
                ref = moe_align(local, n + 1, B)
                P = int(ref["offsets"][n])
                assert np.array_equal(got["counts"].cpu().numpy(), ref["counts"][:n])
                assert np.array_equal(got["offsets"].cpu().numpy(), ref["offsets"][:n + 1])
                assert np.array_equal(got["sorted_ids"].cpu().numpy()[:P], ref["sorted_ids"][:P])
                assert np.array_equal(got["block_expert"].cpu().numpy()[:P // B], ref["block_expert"][:P // B])
                active = ref["active"][ref["active"] < n]
                assert int(got["n_active"][0]) == active.size
                assert np.array_equal(got["active"].cpu().numpy()[:active.size], active)


def test_tiny_shard_routes_over_the_whole_layer(tiny_shards):
    """The router under a range reads logits of all experts and writes global ids; the routed call
    equals forward fed that route."""
    M = 16
    x = bf16_dev(gen_hidden(M, D.K, 750))
    logits = to_dev(gen_logits(M, D.E, 751))
    for layer in tiny_shards:
        for plan in (3, 4):
            layer.set_plan(plan)
            out, ids, w = layer.forward_logits(x, logits)
            ref_ids, ref_w = layer.route(logits)
            assert torch.equal(ids, ref_ids) and torch.equal(w, ref_w)
            assert int(ids.max()) < D.E and int(ids.min()) >= 0
            assert torch.equal(out, layer.forward(x, ids, w))
    for layer in tiny_shards:
        layer.set_plan(0)


@pytest.mark.parametrize("plan,M", [(3, 16), (5, 40), (4, 100)])
def test_tiny_shard_graph_replays_match_eager(tiny_shards, plan, M):
    """A shard's calls captured in a HIP graph and replayed, with eager calls on other inputs in
    between: on a shard the single-launch mode's other-shard workgroups skip the ready-flag hand-off,
    and every replay must still match the eager result bit for bit."""
    layer = tiny_shards[2]
    layer.set_plan(plan)
    x = bf16_dev(gen_hidden(M, D.K, 780 + M))
    ids, w = (to_dev(a) for a in gen_routing_softmax(M, D.E, D.topk, 781 + M))
    ox = bf16_dev(gen_hidden(M, D.K, 790 + M))
    oids, ow = (to_dev(a) for a in gen_routing_softmax(M, D.E, D.topk, 791 + M))
    out = torch.empty((M, D.K), dtype=torch.bfloat16, device="cuda")
    eager = layer.forward(x, ids, w).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x, ids, w, out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, ids, w, out)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"plan {plan} replay {rep}"
        layer.forward(ox, oids, ow)
        torch.cuda.synchronize()
    assert layer.device_error() == 0
    layer.set_plan(0)


def test_set_expert_range_rejects_bad_ranges(tiny_shards):
    from int4_weight_only_align_amd.w4moe import W4MoEError
    layer = tiny_shards[1]
    for first, total in ((-1, 8), (7, 8), (2, 3), (0, 1), (0, 2000)):
        with pytest.raises(W4MoEError):
            layer.set_expert_range(first, total)
    layer.set_expert_range(2, 8)


@pytest.mark.parametrize("first", [144, 0])
def test_k26_ep8_share(first):
    """One GPU's share of an EP8 K2.6 layer (48 of the 384 experts): sampled rows of every column
    against the oracle's shard sum, M = 1, 90, 1024 with uniform routing and M = 256, 1024 with
    Zipf(1.2) routing (hot experts of hundreds of rows on some shards), the default plans."""
    store = ExpertStore(K26, 2)
    n = 48
    layer = make_shard(K26, 2, first, n, 1024, "k26 ep8")
    for M, kind in ((1, "softmax"), (90, "softmax"), (1024, "softmax"), (256, "zipf"), (1024, "zipf")):
        x = gen_hidden(M, K26.K, 1000 + M)
        gen = gen_routing_softmax if kind == "softmax" else gen_routing_zipf
        ids, w = gen(M, K26.E, K26.topk, 2000 + M)
        local = (ids >= first) & (ids < first + n)
        got = gpu_forward(layer, x, ids, w, 0)
        assert np.isfinite(got).all() and layer.device_error() == 0
        assert not got[~local.any(axis=1)].any(), "a token with no local slot is not zero"
        with_local = np.nonzero(local.any(axis=1))[0]
        counts = np.bincount(ids[local].reshape(-1) - first, minlength=n)
        hot_rows = np.nonzero((ids == first + int(np.argmax(counts))).any(axis=1))[0] if counts.max() else []
        rows = sorted(set([0, M - 1] + with_local[:2].tolist() + list(hot_rows[-1:])))
        log(f"[k26 ep8 {first}] M={M} {kind}: plan {layer.resolved_plan(M)}, {int(local.sum())} local slots "
            f"(hottest local expert {int(counts.max())} rows), rows {rows}")
        ref = shard_ref(K26, x, ids, w, store, first, n, rows=np.array(rows, np.int32))
        if np.abs(ref).max() == 0:
            assert not got[rows].any()
        else:
            parity(got[rows], ref, f"k26 ep8 {first} M={M} {kind}")
    layer.close()

