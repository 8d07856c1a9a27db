"""Pins of the CPU oracle against things other than itself (no GPU).

Each test is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign, a wrong
nibble or group index, gate and up swapped, a transposed operand, the routing weight applied to the
wrong slot) fails at least one of them:
  * element unpacking vs an independent packer, including the edge codes -8, 0 and 7;
  * dequantisation equals value * scale exactly;
  * brute force: every expert computed densely for every token (numpy fp64 matmuls on weights
    unpacked by an independent byte-view decoder), combined through a dense gate matrix;
  * closed form 1: unit scales and one-hot codes make the layer SiLU(x_c) * x_c on the first N
    features and 0 elsewhere;
  * closed form 2: all codes 1 and unit scales make every output N * SiLU(S) * S with S = sum(x);
  * experts that no token routes to do not change the output, whatever their weights;
  * the output is linear in the routing weights, and a one-hot routing weight gives one dense
    SwiGLU expert (numpy).
"""
import numpy as np
import pytest

from oracle import code, dequant, expert_ffn, moe_forward
from synth import CONFIGS, ExpertStore, MoEDims, bf16_bits, gen_hidden, gen_routing_softmax, gen_routing_zipf
from tests.packing import bf16_f64, dequant as np_dequant, pack_codes, pack_codes8, unpack_codes, unpack_codes8

TINY = CONFIGS["tiny"]


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_unpack_matches_independent_packer():
    rng = np.random.default_rng(7)
    q = rng.integers(-8, 8, size=(64, 24))
    q[0, 0], q[1, 0], q[7, 3], q[8, 5] = -8, 7, 0, -8
    words = pack_codes(q)
    assert np.array_equal(unpack_codes(words), q)
    for r in range(q.shape[0]):
        for c in range(q.shape[1]):
            assert code(words, r, c) == q[r, c]


def test_dequant_is_value_times_scale():
    rng = np.random.default_rng(8)
    q = rng.integers(-8, 8, size=(64, 16))
    words = pack_codes(q)
    s = bf16_bits(rng.uniform(0.005, 0.02, size=(2, 16)).astype(np.float32))
    for r in range(0, 64, 5):
        for c in range(16):
            expect = float(q[r, c]) * float(bf16_f64(s[r // 32, c]))
            assert dequant(words, s, 32, r, c) == expect


def _dense_moe(dims, x_bits, ids, w, experts):
    """Brute force: all experts on all tokens, combined through a dense [M, E] gate matrix."""
    x = bf16_f64(x_bits)
    M = x.shape[0]
    G = np.zeros((M, dims.E))
    np.add.at(G, (np.repeat(np.arange(M), dims.topk), ids.reshape(-1)), w.reshape(-1).astype(np.float64))
    out = np.zeros((M, dims.K))
    for e in range(dims.E):
        w1, s1, w2, s2 = experts[e]
        W1 = np_dequant(w1, s1, dims.group, dims.bits)      # [K, 2N]
        W2 = np_dequant(w2, s2, dims.group, dims.bits)      # [N, K]
        H = x @ W1
        A = _silu(H[:, :dims.N]) * H[:, dims.N:]
        out += G[:, e:e + 1] * (A @ W2)
    return out


def test_brute_force_dense_tiny_config():
    st = ExpertStore(TINY, 1)
    x = gen_hidden(16, TINY.K, 101)
    ids, w = gen_routing_softmax(16, TINY.E, TINY.topk, 201)
    ref = _dense_moe(TINY, x, ids, w, st)
    got = moe_forward(TINY, x, ids, w, st)
    assert _rel(got, ref) < 1e-12


def _dense_shard(dims, x_bits, ids, w, experts, first, n):
    """Brute force of one expert-parallel shard: only experts [first, first + n) of the dense gate
    matrix's columns, each on every token."""
    x = bf16_f64(x_bits)
    M = x.shape[0]
    G = np.zeros((M, dims.E))
    np.add.at(G, (np.repeat(np.arange(M), dims.topk), ids.reshape(-1)), w.reshape(-1).astype(np.float64))
    out = np.zeros((M, dims.K))
    for e in range(first, first + n):
        w1, s1, w2, s2 = experts[e]
        H = x @ np_dequant(w1, s1, dims.group, dims.bits)
        out += G[:, e:e + 1] * ((_silu(H[:, :dims.N]) * H[:, dims.N:]) @ np_dequant(w2, s2, dims.group, dims.bits))
    return out


def test_expert_shards_brute_force_and_add_up_to_the_layer():
    """The reference of one GPU's expert-parallel share (the oracle with other shards' slots weighted
    0) equals a brute force over the shard's experts alone, and the shards add up to the layer."""
    from tests.shards import shard_ref
    st = ExpertStore(TINY, 1)
    for M in (1, 16):
        x = gen_hidden(M, TINY.K, 700 + M)
        ids, w = gen_routing_softmax(M, TINY.E, TINY.topk, 710 + M)
        full = moe_forward(TINY, x, ids, w, st)
        total = np.zeros_like(full)
        for first, n in ((0, 2), (2, 2), (4, 1), (5, 3)):
            part = shard_ref(TINY, x, ids, w, st, first, n)
            dense = _dense_shard(TINY, x, ids, w, st, first, n)
            assert np.abs(part - dense).max() <= 1e-12 * max(np.abs(dense).max(), 1e-300)
            total += part
        assert _rel(total, full) < 1e-12


def test_brute_force_with_duplicate_ids_and_odd_shapes():
    d = MoEDims(E=3, K=64, N=32, topk=3)
    st = ExpertStore(d, 99)
    x = gen_hidden(5, d.K, 5)
    ids = np.array([[0, 0, 2], [1, 2, 1], [2, 2, 2], [0, 1, 2], [1, 1, 0]], np.int32)
    w = np.random.default_rng(3).uniform(-1, 1, size=ids.shape).astype(np.float32)
    ref = _dense_moe(d, x, ids, w, st)
    assert _rel(moe_forward(d, x, ids, w, st), ref) < 1e-12
    rows = np.array([4, 1], np.int32)
    assert _rel(moe_forward(d, x, ids, w, st, rows=rows), ref[rows]) < 1e-12


def _unit_scale_experts(d, q1, q2):
    s1 = bf16_bits(np.ones((d.K // 32, 2 * d.N), np.float32))
    s2 = bf16_bits(np.ones((d.N // 32, d.K), np.float32))
    return {e: (pack_codes(q1), s1, pack_codes(q2), s2) for e in range(d.E)}


def test_closed_form_identity_scale():
    d = TINY  # K = 256 > N = 128
    q1 = np.zeros((d.K, 2 * d.N), np.int64)
    q2 = np.zeros((d.N, d.K), np.int64)
    for n in range(d.N):
        q1[n, n] = 1          # gate column n picks x_n
        q1[n, d.N + n] = 1    # up column n picks x_n
        q2[n, n] = 1          # down row n writes feature n
    ex = _unit_scale_experts(d, q1, q2)
    x = gen_hidden(6, d.K, 17)
    ids, w = gen_routing_softmax(6, d.E, d.topk, 18)
    got = moe_forward(d, x, ids, w, ex)
    xf = bf16_f64(x)
    ref = np.zeros((6, d.K))
    ref[:, :d.N] = _silu(xf[:, :d.N]) * xf[:, :d.N] * w.astype(np.float64).sum(axis=1, keepdims=True)
    assert _rel(got, ref) < 1e-12
    assert np.all(got[:, d.N:] == 0.0)


def test_closed_form_unit_weights():
    d = TINY
    ex = _unit_scale_experts(d, np.ones((d.K, 2 * d.N), np.int64), np.ones((d.N, d.K), np.int64))
    x = gen_hidden(4, d.K, 23)
    ids, w = gen_routing_softmax(4, d.E, d.topk, 24)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    got = moe_forward(d, x, ids, w, ex)
    S = bf16_f64(x).sum(axis=1)
    ref = (d.N * _silu(S) * S * w.astype(np.float64).sum(axis=1))[:, None] * np.ones((1, d.K))
    assert _rel(got, ref) < 1e-12


def test_unrouted_experts_do_not_contribute():
    d = TINY
    st = ExpertStore(d, 1)
    x = gen_hidden(3, d.K, 31)
    ids = np.array([[1, 4], [4, 6], [6, 1]], np.int32)
    w = np.full(ids.shape, 0.5, np.float32)
    base = moe_forward(d, x, ids, w, st)
    wild = {e: st[e] for e in (1, 4, 6)}
    rng = np.random.default_rng(0)
    for e in (0, 2, 3, 5, 7):
        w1, s1, w2, s2 = st[e]
        wild[e] = (np.full_like(w1, -1), np.full_like(s1, 0x7F00),   # all codes 7, scale 2^127
                   rng.integers(-2**31, 2**31, size=w2.shape, dtype=np.int64).astype(np.int32),
                   np.full_like(s2, 0xFF00))                          # scale -2^127
    assert np.array_equal(moe_forward(d, x, ids, w, wild), base)


def test_linear_in_routing_weights_and_one_hot():
    d = TINY
    st = ExpertStore(d, 1)
    x = gen_hidden(8, d.K, 41)
    ids, _ = gen_routing_softmax(8, d.E, d.topk, 42)
    rng = np.random.default_rng(43)
    # multiples of 2^-10 in [0, 1): wa + wb is exact in fp32, so only fp64 rounding separates the sides
    wa = (rng.integers(0, 1024, size=ids.shape) / 1024.0).astype(np.float32)
    wb = (rng.integers(0, 1024, size=ids.shape) / 1024.0).astype(np.float32)
    fa, fb = moe_forward(d, x, ids, wa, st), moe_forward(d, x, ids, wb, st)
    fab = moe_forward(d, x, ids, wa + wb, st)
    assert _rel(fab, fa + fb) < 1e-12
    one = np.zeros(ids.shape, np.float32)
    one[:, 0] = 1.0
    got = moe_forward(d, x, ids, one, st)
    xf = bf16_f64(x)
    for m in range(8):
        w1, s1, w2, s2 = st[int(ids[m, 0])]
        H = xf[m] @ np_dequant(w1, s1)
        ref = (_silu(H[:d.N]) * H[d.N:]) @ np_dequant(w2, s2)
        assert _rel(got[m], ref) < 1e-12
        assert _rel(expert_ffn(d, x[m], w1, s1, w2, s2), ref) < 1e-12


def test_scaling_weights_by_two_doubles_output():
    d = TINY
    st = ExpertStore(d, 1)
    x = gen_hidden(4, d.K, 51)
    ids, w = gen_routing_softmax(4, d.E, d.topk, 52)
    base = moe_forward(d, x, ids, w, st)
    # doubling the down-projection scales doubles every expert output (exact power of two)
    st2 = {e: (st[e][0], st[e][1], st[e][2], (st[e][3].astype(np.uint32) + (1 << 7)).astype(np.uint16))
           for e in range(d.E)}
    assert np.array_equal(moe_forward(d, x, ids, w, st2), 2.0 * base)


def test_generator_routing_properties():
    ids, w = gen_routing_softmax(64, 384, 8, 2001)
    assert ids.min() >= 0 and ids.max() < 384
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6) and np.all(w > 0)
    zi, zw = gen_routing_zipf(1024, 384, 8, 7)
    assert all(len(set(r)) == 8 for r in zi.tolist())
    assert np.allclose(zw.sum(axis=1), 1.0, atol=1e-6)
    counts = np.bincount(zi.reshape(-1), minlength=384)
    assert counts.max() > 300 and (counts == 0).sum() > 0     # hot experts and never-routed experts


@pytest.mark.parametrize("name", ["k26"])
def test_full_size_single_pair_vs_numpy(name):
    """One K2.6-sized expert on one token: oracle vs numpy fp64 (catches stride/shape slips that
    only show at full size)."""
    d = CONFIGS[name]
    w1, s1, w2, s2 = ExpertStore(d, 2)[5]
    x = gen_hidden(1, d.K, 1001)[0]
    H = bf16_f64(x) @ np_dequant(w1, s1)
    ref = (_silu(H[:d.N]) * H[d.N:]) @ np_dequant(w2, s2)
    assert _rel(expert_ffn(d, x, w1, s1, w2, s2), ref) < 1e-11


@pytest.mark.parametrize("group", [64, 128])
def test_brute_force_larger_groups(group):
    """Scale groups of 64 and 128 rows: the oracle against the dense numpy model on the same
    experts, and the group boundary falls where the group size puts it."""
    d = MoEDims(E=4, K=256, N=128, topk=2, group=group)
    st = ExpertStore(d, 7)
    x = gen_hidden(6, d.K, 8)
    ids, w = gen_routing_softmax(6, d.E, d.topk, 9)
    assert _rel(moe_forward(d, x, ids, w, st), _dense_moe(d, x, ids, w, st)) < 1e-12
    w1, s1, _, _ = st[0]
    assert s1.shape == (d.K // group, 2 * d.N)
    for r, c in ((group - 1, 3), (group, 3), (2 * group - 1, 200)):
        q = code(w1, r, c)
        assert dequant(w1, s1, group, r, c) == np.float32(q) * np.float32(bf16_f64(s1[r // group, c]))



def test_unpack8_matches_independent_packer():
    rng = np.random.default_rng(17)
    q = rng.integers(-128, 128, size=(32, 12))
    q[0, 0], q[1, 0], q[3, 3], q[4, 5] = -128, 127, 0, -1
    words = pack_codes8(q)
    assert np.array_equal(unpack_codes8(words), q)
    for r in range(q.shape[0]):
        for c in range(q.shape[1]):
            assert code(words, r, c, bits=8) == q[r, c]
            assert dequant(words, bf16_bits(np.full((1, 12), 0.25, np.float32)), 32, r, c, bits=8) == q[r, c] * 0.25


@pytest.mark.parametrize("group", [32, 128])
def test_brute_force_eight_bit_codes(group):
    """8-bit codes: the oracle against the dense numpy model (its own byte-view unpacker)."""
    d = MoEDims(E=4, K=256, N=128, topk=2, group=group, bits=8)
    st = ExpertStore(d, 21)
    assert st[0][0].shape == (d.K // 4, 2 * d.N)
    x = gen_hidden(5, d.K, 22)
    ids, w = gen_routing_softmax(5, d.E, d.topk, 23)
    assert _rel(moe_forward(d, x, ids, w, st), _dense_moe(d, x, ids, w, st)) < 1e-12


def test_eight_bit_closed_form_unit_codes():
    """All 8-bit codes +1 and unit scales behave exactly like the 4-bit closed form N*SiLU(S)*S."""
    d = MoEDims(E=2, K=128, N=128, topk=1, bits=8)
    ones1 = pack_codes8(np.ones((d.K, 2 * d.N), np.int64))
    ones2 = pack_codes8(np.ones((d.N, d.K), np.int64))
    s1 = bf16_bits(np.ones((d.K // 32, 2 * d.N), np.float32))
    s2 = bf16_bits(np.ones((d.N // 32, d.K), np.float32))
    ex = {e: (ones1, s1, ones2, s2) for e in range(d.E)}
    x = bf16_bits((np.random.default_rng(5).standard_normal((3, d.K)) * 0.05).astype(np.float32))
    ids = np.array([[0], [1], [0]], np.int32)
    w = np.ones((3, 1), np.float32)
    S = bf16_f64(x).sum(axis=1)
    ref = (d.N * S / (1 + np.exp(-S)) * S)[:, None] * np.ones((1, d.K))
    assert _rel(moe_forward(d, x, ids, w, ex), ref) < 1e-12
