"""Seeded synthetic inputs shaped like the pages' INT4 MoE benchmark.

Source pages: "The Pivot to Real Hardware: Diagnosing Throughput and Building the INT4 MoE
Benchmark for Kimi K2.6" (Step 1: Understanding the Weight Format; Step 4: the benchmark script;
Assumption 1: weight values do not change the work) and "The Weight-Streaming Threshold"
(Assumption 2: uniform expert activation).

What is drawn here, all with numpy's PCG64:
  * hidden states: float32 N(0,1) rounded to bfloat16 (round-to-nearest-even), stored as uint16 bits;
  * INT4 weights: raw uniform 32-bit words. Each word holds 8 four-bit codes, so every code is an
    independent uniform draw from 0..15, i.e. a uniform signed value in [-8, 7] under the
    offset-binary reading (code = value + 8);
  * group scales: float32 U[0.005, 0.02] rounded to bfloat16;
  * routing ("softmax"): float32 N(0,1) logits over all experts, softmax, top-k, renormalised;
  * routing ("zipf"): expert popularity p_r proportional to r^-s over a seeded permutation of the
    experts; k distinct ids per token drawn without replacement with Gumbel-top-k keys
    (Efraimidis & Spirakis 2006); weights are a softmax over k N(0,1) logits.

  * activation order (GPTQ act-order checkpoints): per expert and matrix a uniformly random
    quantisation order of the reduction rows; the row quantised i-th belongs to group i // group,
    which gives the group index g_idx of every row (each group holds exactly `group` rows).

Each expert's weights come from their own seed sequence (seed, expert), so any single expert can be
regenerated on its own, e.g. by the CPU side of a sampled parity check at full size.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "gen_logits", "gen_act_order",
    "MoEDims", "CONFIGS", "bf16_bits", "bf16_to_f32", "gen_hidden", "gen_expert",
    "gen_routing_softmax", "gen_routing_zipf", "gen_routing", "ExpertStore",
]


@dataclass(frozen=True)
class MoEDims:
    """Layer shape: E experts, hidden size K, per-expert intermediate size N, top-k, group size, code
    width (4: 8 codes per int32; 8: 4 codes per int32)."""
    E: int
    K: int
    N: int
    topk: int
    group: int = 32
    bits: int = 4

    @property
    def w1_shape(self):  # int32 words, packed along the reduction (hidden) dimension
        return (self.K * self.bits // 32, 2 * self.N)

    @property
    def s1_shape(self):
        return (self.K // self.group, 2 * self.N)

    @property
    def w2_shape(self):  # int32 words, packed along the reduction (intermediate) dimension
        return (self.N * self.bits // 32, self.K)

    @property
    def s2_shape(self):
        return (self.N // self.group, self.K)

    @property
    def expert_bytes(self) -> int:
        """Bytes of one expert in the logical layout: the codes plus bf16 scales."""
        n = 0
        for shp, item in ((self.w1_shape, 4), (self.s1_shape, 2), (self.w2_shape, 4), (self.s2_shape, 2)):
            n += shp[0] * shp[1] * item
        return n


# The workloads the layer is checked and measured on (sizes from the pages; distributions as stated
# in each generator below).
CONFIGS = {
    "tiny": MoEDims(E=8, K=256, N=128, topk=2),
    "k26": MoEDims(E=384, K=7168, N=2048, topk=8),
    "k26_tp8": MoEDims(E=384, K=7168, N=256, topk=8),
}

# Seeds: weights per configuration, activations and routing per M (and repetition).
WEIGHT_SEED = {"tiny": 1, "k26": 2, "k26_tp8": 5}
ZIPF_PERM_SEED = 3


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(*seed_parts: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_parts))))


def gen_hidden(M: int, K: int, seed: int) -> np.ndarray:
    """bf16 bits [M, K] of N(0,1) activations."""
    x = _rng(seed, 11).standard_normal((M, K), dtype=np.float32)
    return bf16_bits(x)


def gen_expert(dims: MoEDims, e: int, seed: int):
    """Logical (GPTQ-style) tensors of expert e: w1_q int32 [K*bits/32, 2N], s1 bf16 [K/g, 2N],
    w2_q int32 [N*bits/32, K], s2 bf16 [N/g, K]. Columns [0, N) of w1 are the gate projection and
    columns [N, 2N) the up projection."""
    r = _rng(seed, 1000 + e)
    w1 = r.integers(0, 2**32, size=dims.w1_shape, dtype=np.uint32).view(np.int32)
    s1 = bf16_bits(r.uniform(0.005, 0.02, size=dims.s1_shape).astype(np.float32))
    w2 = r.integers(0, 2**32, size=dims.w2_shape, dtype=np.uint32).view(np.int32)
    s2 = bf16_bits(r.uniform(0.005, 0.02, size=dims.s2_shape).astype(np.float32))
    return w1, s1, w2, s2


def gen_act_order(dims: MoEDims, e: int, seed: int):
    """Group indices of an activation-ordered expert e: g_idx1 int32 [K] for the rows of w1 and
    g_idx2 int32 [N] for the rows of w2. Row order[i] of a uniformly random quantisation order gets
    group i // group."""
    r = _rng(seed, 3000 + e)
    out = []
    for R in (dims.K, dims.N):
        order = r.permutation(R)
        g = np.empty(R, np.int32)
        g[order] = np.arange(R, dtype=np.int32) // dims.group
        out.append(g)
    return tuple(out)


class ExpertStore:
    """Lazily generated experts of one configuration, cached by index: (w1, s1, w2, s2), plus
    (g_idx1, g_idx2) when act_order is set."""

    def __init__(self, dims: MoEDims, seed: int, act_order: bool = False):
        self.dims, self.seed, self.act_order, self._cache = dims, seed, act_order, {}

    def __getitem__(self, e: int):
        if e not in self._cache:
            parts = gen_expert(self.dims, int(e), self.seed)
            if self.act_order:
                parts = parts + gen_act_order(self.dims, int(e), self.seed)
            self._cache[e] = parts
        return self._cache[e]

    def stacked(self):
        """All experts stacked: w1 [E,K/8,2N], s1 [E,K/32,2N], w2 [E,N/8,K], s2 [E,N/32,K]."""
        parts = [self[e] for e in range(self.dims.E)]
        return tuple(np.stack([p[i] for p in parts]) for i in range(4))


def gen_logits(M: int, E: int, seed: int) -> np.ndarray:
    """Router logits: fp32 N(0,1), [M, E] (the draw gen_routing_softmax routes from)."""
    return _rng(seed, 21).standard_normal((M, E), dtype=np.float32)


def gen_routing_softmax(M: int, E: int, topk: int, seed: int):
    """Softmax over N(0,1) fp32 logits, top-k (largest first), weights renormalised to sum 1."""
    logits = gen_logits(M, E, seed)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z, dtype=np.float32)
    p /= p.sum(axis=1, keepdims=True, dtype=np.float32)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :topk].astype(np.int32)
    w = np.take_along_axis(p, ids, axis=1)
    w = (w / w.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)


def gen_routing_zipf(M: int, E: int, topk: int, seed: int, s: float = 1.2, perm_seed: int = ZIPF_PERM_SEED):
    """Skewed routing: expert perm[r] has popularity proportional to (r+1)^-s; k distinct ids per
    token by Gumbel-top-k; weights = softmax of k N(0,1) fp32 logits."""
    perm = _rng(perm_seed, 31).permutation(E)
    logp = np.empty(E, dtype=np.float64)
    logp[perm] = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    r = _rng(seed, 41)
    keys = logp[None, :] + r.gumbel(size=(M, E))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :topk].astype(np.int32)
    lg = r.standard_normal((M, topk), dtype=np.float32)
    lg = np.exp(lg - lg.max(axis=1, keepdims=True), dtype=np.float32)
    w = (lg / lg.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)


def gen_routing(kind: str, M: int, E: int, topk: int, seed: int):
    if kind == "softmax":
        return gen_routing_softmax(M, E, topk, seed)
    if kind == "zipf":
        return gen_routing_zipf(M, E, topk, seed)
    raise ValueError(f"unknown routing kind {kind!r}")
