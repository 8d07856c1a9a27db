"""Pins of the oracle's activation-order path (explicit group index per reduction row), no GPU.

  * consecutive group indices given explicitly reproduce the pinned consecutive-group oracle bit for
    bit (the special case that reduces to it);
  * permutation equivalence: an activation-ordered layer equals the consecutive-group layer whose w1
    rows, w2 rows and intermediate features (w1 gate and up columns) are put in group-sorted order,
    fed the hidden state permuted the same way -- so a group index read for the wrong row, the wrong
    matrix or through the inverse permutation fails;
  * brute force: dense numpy fp64 with every row's scale gathered through its group index;
  * a single hidden feature and single-row codes isolate the scale row one index selects;
  * the generator's group indices hold exactly `group` rows per group and differ per expert.
"""
import numpy as np
import pytest

from oracle import expert_ffn, moe_forward
from synth import ExpertStore, MoEDims, bf16_bits, gen_act_order, gen_hidden, gen_routing_softmax
from tests.packing import bf16_f64, pack_codes, pack_codes8, unpack_codes, unpack_codes8


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _unpack(words, bits):
    return unpack_codes(words) if bits == 4 else unpack_codes8(words)


def _pack(q, bits):
    return pack_codes(q) if bits == 4 else pack_codes8(q)


def _dense(words, scales, gidx, bits):
    """[R, C] fp64: code * scale of the row's recorded group."""
    return _unpack(words, bits).astype(np.float64) * bf16_f64(scales)[gidx]


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 128), (8, 64)])
def test_consecutive_groups_given_explicitly_are_the_plain_layer(bits, group):
    d = MoEDims(E=4, K=256, N=128, topk=2, group=group, bits=bits)
    st = ExpertStore(d, 41)
    x = gen_hidden(6, d.K, 42)
    ids, w = gen_routing_softmax(6, d.E, d.topk, 43)
    g1 = (np.arange(d.K) // group).astype(np.int32)
    g2 = (np.arange(d.N) // group).astype(np.int32)
    act = {e: st[e] + (g1, g2) for e in range(d.E)}
    assert np.array_equal(moe_forward(d, x, ids, w, act), moe_forward(d, x, ids, w, st))


def _sorted_equivalent(d, parts):
    """The consecutive-group expert that computes what the activation-ordered one does once the
    hidden features are put in w1's group-sorted order (perm1) and the intermediate features in w2's
    (perm2): w1 rows permuted by perm1 and its gate / up columns by perm2, w2 rows permuted by perm2."""
    w1, s1, w2, s2, g1, g2 = parts
    p1 = np.argsort(g1, kind="stable")
    p2 = np.argsort(g2, kind="stable")
    q1 = _unpack(w1, d.bits)[p1]
    q1 = np.concatenate([q1[:, :d.N][:, p2], q1[:, d.N:][:, p2]], axis=1)
    s1p = np.concatenate([s1[:, :d.N][:, p2], s1[:, d.N:][:, p2]], axis=1)
    q2 = _unpack(w2, d.bits)[p2]
    return (_pack(q1, d.bits), s1p, _pack(q2, d.bits), s2), p1


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 64), (8, 32)])
def test_permutation_equivalence_with_the_plain_layer(bits, group):
    d = MoEDims(E=3, K=256, N=128, topk=2, group=group, bits=bits)
    st = ExpertStore(d, 51, act_order=True)
    x = gen_hidden(1, d.K, 52)[0]
    for e in range(d.E):
        plain, p1 = _sorted_equivalent(d, st[e])
        ref = expert_ffn(d, x[p1], *plain)
        got = expert_ffn(d, x, *st[e])
        assert _rel(got, ref) < 1e-12, f"expert {e}"
        # and it is not the consecutive-group reading of the same codes
        assert _rel(expert_ffn(d, x, *st[e][:4]), ref) > 1e-3


def test_brute_force_dense_gather():
    d = MoEDims(E=5, K=256, N=128, topk=3, group=32)
    st = ExpertStore(d, 61, act_order=True)
    x = gen_hidden(7, d.K, 62)
    ids, w = gen_routing_softmax(7, d.E, d.topk, 63)
    xf = bf16_f64(x)
    G = np.zeros((7, d.E))
    np.add.at(G, (np.repeat(np.arange(7), d.topk), ids.reshape(-1)), w.reshape(-1).astype(np.float64))
    ref = np.zeros((7, d.K))
    for e in range(d.E):
        w1, s1, w2, s2, g1, g2 = st[e]
        H = xf @ _dense(w1, s1, g1, d.bits)
        A = _silu(H[:, :d.N]) * H[:, d.N:]
        ref += G[:, e:e + 1] * (A @ _dense(w2, s2, g2, d.bits))
    assert _rel(moe_forward(d, x, ids, w, st), ref) < 1e-12


def test_one_feature_selects_the_scale_row_of_its_group():
    """Hidden state one-hot at feature r0, w1 codes 1 in row r0 only, w2 codes 1 on the diagonal:
    gate_n = up_n = s1[g1[r0], n], so out_c = SiLU(s) * s * s2[g2[c], c] for c < N."""
    d = MoEDims(E=1, K=128, N=128, topk=1, group=32)
    rng = np.random.default_rng(71)
    r0 = 77
    q1 = np.zeros((d.K, 2 * d.N), np.int64)
    q1[r0, :] = 1
    q2 = np.eye(d.N, d.K, dtype=np.int64)
    s1 = bf16_bits(rng.uniform(0.5, 2.0, size=(d.K // 32, 2 * d.N)).astype(np.float32))
    s1[:, d.N:] = s1[:, :d.N]
    s2 = bf16_bits(rng.uniform(0.5, 2.0, size=(d.N // 32, d.K)).astype(np.float32))
    g1, g2 = gen_act_order(d, 0, 72)
    x = np.zeros(d.K, np.uint16)
    x[r0] = bf16_bits(np.array([1.0], np.float32))[0]
    y = expert_ffn(d, x, pack_codes(q1), s1, pack_codes(q2), s2, g1, g2)
    s = bf16_f64(s1[g1[r0], :d.N])
    expect = np.zeros(d.K)
    expect[:d.N] = _silu(s) * s * bf16_f64(s2[g2[:d.N], np.arange(d.N)])
    assert _rel(y, expect) < 1e-14
    # the consecutive reading picks row r0 // 32 instead, which differs here
    assert g1[r0] != r0 // 32


def test_generator_groups_hold_group_rows_and_differ_per_expert():
    d = MoEDims(E=4, K=512, N=256, topk=2, group=64)
    a = [gen_act_order(d, e, 81) for e in range(d.E)]
    for g1, g2 in a:
        assert np.array_equal(np.bincount(g1), np.full(d.K // 64, 64))
        assert np.array_equal(np.bincount(g2), np.full(d.N // 64, 64))
    assert not np.array_equal(a[0][0], a[1][0])
    assert np.array_equal(gen_act_order(d, 2, 81)[1], a[2][1])   # reproducible per expert


def test_group_index_out_of_range_is_rejected():
    d = MoEDims(E=1, K=128, N=128, topk=1)
    st = ExpertStore(d, 91, act_order=True)
    w1, s1, w2, s2, g1, g2 = st[0]
    bad = g1.copy()
    bad[5] = d.K // d.group
    with pytest.raises(RuntimeError):
        moe_forward(d, gen_hidden(1, d.K, 1), np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                    {0: (w1, s1, w2, s2, bad, g2)})
    with pytest.raises(ValueError):
        expert_ffn(d, gen_hidden(1, d.K, 1)[0], w1, s1, w2, s2, bad, g2)
