"""Shared helpers of the GPU tests: building prepacked layers from the seeded generators, running the
HIP forward through the C-ABI, and the parity bar against the oracle.

Parity bar for the bf16 output (floating point): every value finite,
  max |out - ref| <= 2e-2 * max |ref|   and   sum |out - ref| / sum |ref| <= 1e-2,
with ref the oracle's fp64 result. The GPU rounds the SwiGLU intermediate and the output to bf16
(relative 2^-9 each) and accumulates in fp32, so its error sits an order of magnitude below this bar.
"""
import sys
import time

import numpy as np
import torch

from synth import ExpertStore, gen_act_order, gen_expert

MAX_REL = 2e-2
L1_REL = 1e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def bf16_dev(bits):
    return to_dev(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)


def prepack_experts(layer, dims, seed, experts=None, batch=16, override=None):
    """Generate experts (not cached) and prepack them in batches. `override` maps an expert to
    replacement logical tensors."""
    ids = list(range(dims.E)) if experts is None else list(experts)
    t0 = time.time()
    i = 0
    while i < len(ids):
        # a run of consecutive expert ids
        j = i
        while j + 1 < len(ids) and ids[j + 1] == ids[j] + 1 and j + 1 - i < batch:
            j += 1
        parts = [override[e] if override and e in override else gen_expert(dims, e, seed) for e in ids[i:j + 1]]
        st = [np.stack([p[k] for p in parts]) for k in range(4)]
        layer.prepack(to_dev(st[0]), bf16_dev(st[1]), to_dev(st[2]), bf16_dev(st[3]), first_expert=ids[i])
        torch.cuda.synchronize()
        if (i // batch) % 8 == 0 and len(ids) > batch:
            log(f"  prepacked experts up to {ids[j]} of {dims.E} ({time.time() - t0:.1f}s)")
        i = j + 1


def make_layer(dims, seed, max_tokens, tag):
    from int4_weight_only_align_amd.w4moe import MoELayer
    log(f"[{tag}] create + prepack E={dims.E} K={dims.K} N={dims.N} top{dims.topk} max_tokens={max_tokens}")
    layer = MoELayer(dims.E, dims.K, dims.N, dims.topk, max_tokens, group_size=dims.group, num_bits=dims.bits)
    prepack_experts(layer, dims, seed)
    return layer, ExpertStore(dims, seed)


def group_order(g_idx):
    """The caller's side of activation order: a checkpoint's group index per row -> the rows in group
    order (a stable argsort), the permutation w4moe_prepack_act_order takes."""
    return np.argsort(np.asarray(g_idx), kind="stable").astype(np.int32)


def make_layer_act_order(dims, seed, max_tokens, tag, batch=16):
    """Activation-ordered layer: the seeded experts plus seeded group indices, prepacked with the
    group-order permutations; the oracle's store holds the group indices themselves."""
    from int4_weight_only_align_amd.w4moe import MoELayer
    log(f"[{tag}] create + prepack (act order) E={dims.E} K={dims.K} N={dims.N} top{dims.topk} group {dims.group} "
        f"bits {dims.bits}")
    layer = MoELayer(dims.E, dims.K, dims.N, dims.topk, max_tokens, group_size=dims.group, num_bits=dims.bits,
                     act_order=True)
    for e0 in range(0, dims.E, batch):
        es = range(e0, min(dims.E, e0 + batch))
        parts = [gen_expert(dims, e, seed) + gen_act_order(dims, e, seed) for e in es]
        st = [np.stack([p[k] for p in parts]) for k in range(4)]
        p1 = np.stack([group_order(p[4]) for p in parts])
        p2 = np.stack([group_order(p[5]) for p in parts])
        layer.prepack_act_order(to_dev(st[0]), bf16_dev(st[1]), to_dev(p1), to_dev(st[2]), bf16_dev(st[3]), to_dev(p2),
                                first_expert=e0)
        torch.cuda.synchronize()
    return layer, ExpertStore(dims, seed, act_order=True)


def gpu_forward(layer, x_bits, ids, w, plan=0):
    layer.set_plan(plan)
    out = layer.forward(bf16_dev(x_bits), to_dev(ids), to_dev(w))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def parity(got, ref, tag):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{tag}: non-finite output"
    err = np.abs(got - ref)
    max_rel = float(err.max() / max(np.abs(ref).max(), 1e-30))
    l1_rel = float(err.sum() / max(np.abs(ref).sum(), 1e-30))
    log(f"[{tag}] max|err|/max|ref| = {max_rel:.2e}  sum|err|/sum|ref| = {l1_rel:.2e}")
    assert max_rel <= MAX_REL and l1_rel <= L1_REL, f"{tag}: max_rel={max_rel:.3e} l1_rel={l1_rel:.3e}"
    return max_rel, l1_rel
