"""The benchmark's bookkeeping on the CPU: the algorithmic bytes and flops that the roofline fractions
divide by, checked against their closed forms at the K2.6 dims (one routed expert = its int4 codes
plus one bf16 scale per 32 rows and column, for W1 [K, 2N] and W2 [N, K]), the counting of distinct
and shard-local experts, and the refusal to run on more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import bench
from synth import CONFIGS

K26 = CONFIGS["k26"]
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _expert_bytes(K, N, group=32):
    w1 = K * 2 * N // 2 + (K // group) * 2 * N * 2      # codes (4 bits) + bf16 scales
    w2 = N * K // 2 + (N // group) * K * 2
    return w1 + w2


def test_expert_bytes_closed_form():
    assert _expert_bytes(7168, 2048) == 24_772_608
    assert K26.expert_bytes == 24_772_608
    assert CONFIGS["k26_tp8"].expert_bytes == _expert_bytes(7168, 256)


def test_layer_bytes_decode_call():
    """M=1, eight distinct experts: 8 experts + hidden in + out + ids and weights = 198,209,600 B."""
    ids = np.arange(8, dtype=np.int32).reshape(1, 1, 8) * 7
    nbytes, active = bench.layer_bytes(K26, 1, ids)
    assert active == 8
    assert nbytes == 8 * 24_772_608 + 2 * 7168 * 2 + 8 * 8 == 198_209_600


def test_layer_bytes_counts_each_expert_once_and_averages_over_sets():
    a = np.array([[[0, 1, 2, 3, 4, 5, 6, 7], [0, 1, 2, 3, 8, 9, 10, 11]]], np.int32)   # 12 distinct
    b = np.array([[[5] * 8, [5] * 8]], np.int32)                                        # 1 distinct
    nbytes, active = bench.layer_bytes(K26, 2, np.concatenate([a, b]))
    assert active == (12 + 1) / 2
    assert nbytes == 6.5 * 24_772_608 + 2 * 2 * 7168 * 2 + 2 * 8 * 8


def test_layer_bytes_of_a_shard_counts_local_experts_only():
    ids = np.array([[[143, 144, 150, 191, 192, 300, 0, 150]]], np.int32)
    nbytes, active = bench.layer_bytes(K26, 1, ids, shard=(144, 48))
    assert active == 3                                  # 144, 150, 191
    assert nbytes == 3 * 24_772_608 + 2 * 7168 * 2 + 8 * 8


def test_layer_flops():
    """2 flops per multiply-add: per routed slot K x 2N (GEMM1) + N x K (GEMM2)."""
    per_slot = 2 * (7168 * 4096 + 2048 * 7168)
    assert bench.layer_flops(K26, 1) == 8 * per_slot == 704_643_072
    assert bench.layer_flops(K26, 1024) == 1024 * 8 * per_slot
    assert bench.layer_flops(K26, 4, slots=3.5) == 3.5 * per_slot


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
