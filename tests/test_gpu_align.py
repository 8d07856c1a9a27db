"""The HIP alignment kernel against the oracle, bit-exact (counts, padded offsets, sorted flat ids,
block experts, active list), on the workloads' routings and the degenerate cases."""
import numpy as np
import pytest
import torch

from oracle import moe_align
from synth import gen_routing_softmax, gen_routing_zipf
from tests.gpu_common import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layers():
    from int4_weight_only_align_amd.w4moe import MoELayer
    # the alignment needs no weights; small K, N keep the handles light
    big = MoELayer(384, 128, 128, 8, max_tokens=1024)
    tiny = MoELayer(8, 128, 128, 2, max_tokens=64)
    yield {384: big, 8: tiny}
    big.close()
    tiny.close()


def _compare(layer, ids, E, B, tag):
    log(f"[align {tag}] M={ids.shape[0]} E={E} B={B}")
    r = layer.moe_align(to_dev(ids), B)
    torch.cuda.synchronize()
    ref = moe_align(ids, E, B)
    P = ref["padded_rows"]
    got = {k: v.cpu().numpy() for k, v in r.items()}
    assert np.array_equal(got["counts"], ref["counts"]), tag
    assert np.array_equal(got["offsets"], ref["offsets"]), tag
    assert np.array_equal(got["sorted_ids"][:P], ref["sorted_ids"]), tag
    assert np.array_equal(got["block_expert"][:P // B], ref["block_expert"]), tag
    n = int(got["n_active"][0])
    assert n == ref["active"].size and np.array_equal(got["active"][:n], ref["active"]), tag


@pytest.mark.parametrize("B", [16, 1, 64])
@pytest.mark.parametrize("M", [1, 9, 32, 90, 256, 330, 512, 1024])
def test_align_softmax_routing(layers, M, B):
    ids, _ = gen_routing_softmax(M, 384, 8, 2000 + M)
    _compare(layers[384], ids, 384, B, "softmax")


@pytest.mark.parametrize("M", [256, 512, 1024])
def test_align_zipf_routing(layers, M):
    ids, _ = gen_routing_zipf(M, 384, 8, 3000 + M)
    _compare(layers[384], ids, 384, 16, "zipf")


def test_align_block_of_forward(layers):
    """The block forward's alignment uses, as the handle reports it: the MFMA token tile."""
    assert layers[384].align_block() == 16


def test_align_tiny_config(layers):
    ids, _ = gen_routing_softmax(16, 8, 2, 201)
    for B in (1, 4, 16):
        _compare(layers[8], ids, 8, B, "tiny")


def test_align_degenerate_cases(layers):
    big = layers[384]
    _compare(big, np.full((1024, 8), 5, np.int32), 384, 16, "all entries to one expert")
    _compare(big, np.full((1024, 8), 383, np.int32), 384, 1, "all entries to the last expert")
    _compare(big, np.arange(384, dtype=np.int32).reshape(48, 8), 384, 16, "each expert once")
    _compare(big, np.array([[7, 7, 7, 1, 1, 7, 0, 7]], np.int32), 384, 16, "duplicates within a token")
    rng = np.random.default_rng(5)
    _compare(big, rng.integers(0, 3, size=(777, 8)).astype(np.int32), 384, 16, "three hot experts, ragged M")
    r = big.moe_align(torch.zeros((0, 8), dtype=torch.int32, device="cuda"), 16)
    torch.cuda.synchronize()
    assert int(r["offsets"][-1]) == 0 and int(r["counts"].sum()) == 0 and int(r["n_active"][0]) == 0


def test_align_drops_out_of_range_ids(layers):
    big = layers[384]
    ids = np.array([[0, 384, 5, -1, 5, 7, 1000, 2]], np.int32)
    log("[align] out-of-range ids")
    big.device_error()   # clear
    r = big.moe_align(to_dev(ids), 16)
    flags = big.device_error()
    assert flags & 1
    valid = ids.reshape(-1)
    got = r["sorted_ids"].cpu().numpy()
    counts = r["counts"].cpu().numpy()
    assert counts.sum() == 5 and counts[5] == 2
    offs = r["offsets"].cpu().numpy()
    assert got[offs[5]:offs[5] + 2].tolist() == [2, 4]
    assert set(got[:offs[-1]].tolist()) - {8} == {0, 2, 4, 5, 7}
    assert valid.size == 8


def test_align_several_scatter_rounds():
    """Entries beyond one scatter round (65,536): E = 1024 (all ten id bits), a ragged last round,
    uniform and one-hot-heavy routings; bit-exact against the oracle."""
    from int4_weight_only_align_amd.w4moe import MoELayer
    layer = MoELayer(1024, 128, 128, 8, max_tokens=17000)
    try:
        rng = np.random.default_rng(11)
        ids = rng.integers(0, 1024, size=(16999, 8)).astype(np.int32)
        _compare(layer, ids, 1024, 16, "two rounds and a ragged third, uniform")
        ids[:9000] = 1023
        _compare(layer, ids, 1024, 1, "first round entirely one expert")
        ids = np.repeat(rng.integers(0, 1024, size=(17000, 1)), 8, axis=1).astype(np.int32)
        _compare(layer, ids, 1024, 64, "every token's slots to one expert")
    finally:
        layer.close()


def test_align_drops_out_of_range_ids_in_chunks(layers):
    """Out-of-range ids spread over several 1024-entry chunks (the two-launch alignment from 4096
    entries): dropped from every output, flag bit 0 raised, the rest bit-exact against the oracle
    fed the same ids with the dropped ones moved to an expert of their own past the last."""
    big = layers[384]
    rng = np.random.default_rng(5)
    ids, _ = gen_routing_softmax(1000, 384, 8, 5000)
    ids = ids.copy()
    bad = rng.random(ids.shape) < 0.02
    ids[bad] = rng.choice([-1, 384, 1 << 20], size=int(bad.sum()))
    log(f"[align] {int(bad.sum())} out-of-range ids among {ids.size} entries")
    big.device_error()
    r = big.moe_align(to_dev(ids), 16)
    assert big.device_error() & 1
    ref = moe_align(np.where(bad, 384, ids).astype(np.int32), 385, 16)
    P = int(ref["offsets"][384])          # rows of the real experts; the extra expert's rows follow
    got = {k: v.cpu().numpy() for k, v in r.items()}
    assert np.array_equal(got["counts"], ref["counts"][:384])
    assert np.array_equal(got["offsets"], ref["offsets"][:385])
    assert np.array_equal(got["sorted_ids"][:P], ref["sorted_ids"][:P])   # padding rows hold T in both
    assert np.array_equal(got["block_expert"][:P // 16], ref["block_expert"][:P // 16])
