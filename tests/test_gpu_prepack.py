"""The prepack kernel is a bijection: decoding the packed buffer with the test-side decoder of the
documented layout gives back the logical codes and scales bit for bit."""
import numpy as np
import pytest
import torch

from synth import MoEDims, gen_expert
from tests.gpu_common import log, prepack_experts
from tests.packing import decode_packed, unpack_codes

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dims", [MoEDims(E=8, K=256, N=128, topk=2), MoEDims(E=2, K=7168, N=2048, topk=2),
                                  MoEDims(E=3, K=7168, N=256, topk=2), MoEDims(E=3, K=384, N=640, topk=3)],
                         ids=["tiny", "k26-2experts", "tp8-3experts", "odd-superblocks"])
def test_prepack_round_trip(dims):
    from int4_weight_only_align_amd.w4moe import MoELayer
    log(f"[prepack] E={dims.E} K={dims.K} N={dims.N}")
    layer = MoELayer(dims.E, dims.K, dims.N, dims.topk, max_tokens=4)
    # experts in reverse order, one at a time, to exercise first_expert offsets
    prepack_experts(layer, dims, seed=11, experts=list(range(dims.E))[::-1], batch=1)
    for which, kind, R, Cc in ((1, "w1", dims.K, 2 * dims.N), (2, "w2", dims.N, dims.K)):
        buf = layer.packed_bytes(which).cpu().numpy()
        assert buf.size == dims.E * R * Cc // 2 + dims.E * (R // 32) * Cc * 2
        codes, scales = decode_packed(buf, kind, dims.E, R, Cc, dims.N)
        for e in range(dims.E):
            w1, s1, w2, s2 = gen_expert(dims, e, 11)
            wq, sc = (w1, s1) if which == 1 else (w2, s2)
            assert np.array_equal(codes[e], unpack_codes(wq)), (kind, e)
            assert np.array_equal(scales[e], sc), (kind, e)
    torch.cuda.synchronize()
    layer.close()


@pytest.mark.parametrize("group", [64, 128])
def test_prepack_round_trip_larger_groups(group):
    """Groups of 64 or 128 rows: the packed layout keeps one scale per 32 rows, each being the scale
    of the group those rows belong to; the codes are untouched."""
    from int4_weight_only_align_amd.w4moe import MoELayer
    dims = MoEDims(E=3, K=512, N=256, topk=2, group=group)
    layer = MoELayer(dims.E, dims.K, dims.N, dims.topk, max_tokens=4, group_size=group)
    prepack_experts(layer, dims, seed=13)
    for which, kind, R, Cc in ((1, "w1", dims.K, 2 * dims.N), (2, "w2", dims.N, dims.K)):
        codes, scales = decode_packed(layer.packed_bytes(which).cpu().numpy(), kind, dims.E, R, Cc, dims.N)
        for e in range(dims.E):
            w1, s1, w2, s2 = gen_expert(dims, e, 13)
            wq, sc = (w1, s1) if which == 1 else (w2, s2)
            assert np.array_equal(codes[e], unpack_codes(wq)), (kind, e)
            assert np.array_equal(scales[e], np.repeat(sc, group // 32, axis=0)), (kind, e)
    torch.cuda.synchronize()
    layer.close()


@pytest.mark.parametrize("group", [32, 128])
def test_prepack_round_trip_eight_bit(group):
    """8-bit codes: the low- and high-nibble planes give back every code, the scales their groups'."""
    from int4_weight_only_align_amd.w4moe import MoELayer
    from tests.packing import unpack_codes8
    dims = MoEDims(E=3, K=512, N=256, topk=2, group=group, bits=8)
    layer = MoELayer(dims.E, dims.K, dims.N, dims.topk, max_tokens=4, group_size=group, num_bits=8)
    prepack_experts(layer, dims, seed=19, experts=[2, 0, 1], batch=1)
    for which, kind, R, Cc in ((1, "w1", dims.K, 2 * dims.N), (2, "w2", dims.N, dims.K)):
        buf = layer.packed_bytes(which).cpu().numpy()
        assert buf.size == dims.E * (R // 128) * (Cc // 64) * 8704
        codes, scales = decode_packed(buf, kind, dims.E, R, Cc, dims.N, bits=8)
        for e in range(dims.E):
            w1, s1, w2, s2 = gen_expert(dims, e, 19)
            wq, sc = (w1, s1) if which == 1 else (w2, s2)
            assert np.array_equal(codes[e], unpack_codes8(wq)), (kind, e)
            assert np.array_equal(scales[e], np.repeat(sc, group // 32, axis=0)), (kind, e)
    torch.cuda.synchronize()
    layer.close()


@pytest.mark.parametrize("dims", [MoEDims(E=3, K=160, N=96, topk=2), MoEDims(E=2, K=2080, N=416, topk=2),
                                  MoEDims(E=3, K=160, N=96, topk=2, bits=8),
                                  MoEDims(E=2, K=192, N=320, topk=2, group=64)],
                         ids=["K160-N96", "K2080-N416", "K160-N96-w8", "K192-N320-g64"])
def test_prepack_round_trip_padded(dims):
    """Reduction rows padded up to whole 128-row blocks and W2 columns up to whole 64-column blocks:
    the data region decodes to the logical codes and scales, the padding to the code of 0 and the
    scale 0."""
    from int4_weight_only_align_amd.w4moe import MoELayer
    from tests.packing import unpack_codes8
    bits = dims.bits
    layer = MoELayer(dims.E, dims.K, dims.N, dims.topk, max_tokens=4, group_size=dims.group, num_bits=bits)
    prepack_experts(layer, dims, seed=31, experts=list(range(dims.E))[::-1], batch=1)
    up = lambda v, m: (v + m - 1) // m * m
    for which, kind, R, Cc, Rp, Cp in ((1, "w1", dims.K, 2 * dims.N, up(dims.K, 128), 2 * dims.N),
                                        (2, "w2", dims.N, dims.K, up(dims.N, 128), up(dims.K, 64))):
        buf = layer.packed_bytes(which).cpu().numpy()
        assert buf.size == dims.E * (Rp // 128) * (Cp // 64) * (4096 * bits // 4 + 512)
        codes, scales = decode_packed(buf, kind, dims.E, Rp, Cp, dims.N, bits=bits)
        for e in range(dims.E):
            w1, s1, w2, s2 = gen_expert(dims, e, 31)
            wq, sc = (w1, s1) if which == 1 else (w2, s2)
            want = unpack_codes(wq) if bits == 4 else unpack_codes8(wq)
            assert np.array_equal(codes[e][:R, :Cc], want), (kind, e)
            assert np.array_equal(scales[e][:R // 32, :Cc], np.repeat(sc, dims.group // 32, axis=0)), (kind, e)
            pad = np.ones((Rp, Cp), bool)
            pad[:R, :Cc] = False
            assert (codes[e][pad] == 0).all(), (kind, e)
            spad = np.ones((Rp // 32, Cp), bool)
            spad[:R // 32, :Cc] = False
            assert (scales[e][spad] == 0).all(), (kind, e)
    torch.cuda.synchronize()
    layer.close()
