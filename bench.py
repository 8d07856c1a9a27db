"""Benchmark of the W4A16 MoE layer on one MI355X.

A step is one forward call of the whole layer (alignment, GEMM1 + SwiGLU, GEMM2, top-k combine)
on one batch that is already resident in HBM. The headline workload is the K2.6-shaped decode
layer (E=384, K=7168, N=2048, top-8, group 32) at M=1 token, with the routing rotated over 64
seeded sets so that consecutive calls stream different experts (the 256 MB last-level cache cannot
serve repeated weights). Prints one JSON line on stdout.

Also reported: per-kernel times from HIP events recorded on the launch stream by the library
(same workload, a second timed region of the same length), the dominant kernel's roofline, the
M sweep 1..1024 (uniform and Zipf routing), the same layer with 8-bit codes and with
activation-ordered weights, one GPU's share of a tensor-parallel layer (N = 256) and of an
expert-parallel one (48 of the 384 experts, global routing ids), and the CPU oracle on a bounded
sample of the headline workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer ms/call & tokens/s vs M=1..1024; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PAGES_TOKS_M1 = 6642.0     # the pages' single-GPU figure at M=1 (another machine: context)
SWEEP_M = [1, 2, 4, 8, 9, 16, 32, 64, 90, 128, 256, 330, 512, 1024]
GEMM_SRC = os.path.join(ROOT, "int4_weight_only_align_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_pair_fused_k26_decode_m1_traffic.md")
EP8_SHARD = (144, 48)   # one GPU's expert-parallel share of the K2.6 layer: experts 144..191 of 384


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def build_layer(dims, seed, max_tokens, act_order=False, shard=None):
    """A prepacked layer of seeded experts. With act_order, each expert also gets seeded group indices
    (a GPTQ act-order checkpoint) and is prepacked with the rows in group order (a stable argsort of
    the group indices, as a caller of the library computes it). With shard = (first, n), the layer
    holds experts [first, first + n) of dims.E (one GPU's expert-parallel share) and reads global ids."""
    import torch
    from int4_weight_only_align_amd.w4moe import MoELayer
    from synth import gen_act_order, gen_expert

    first, n_exp = shard if shard else (0, dims.E)
    layer = MoELayer(n_exp, dims.K, dims.N, dims.topk, max_tokens, group_size=dims.group, num_bits=dims.bits,
                     act_order=act_order)
    t0 = time.time()
    batch = 16

    def gen(e):
        parts = gen_expert(dims, first + e, seed)
        if act_order:
            parts = parts + tuple(np.argsort(g, kind="stable").astype(np.int32) for g in gen_act_order(dims, e, seed))
        return parts

    with ThreadPoolExecutor(max_workers=8) as ex:
        for e0 in range(0, n_exp, batch):
            parts = list(ex.map(gen, range(e0, min(n_exp, e0 + batch))))
            st = [np.stack([p[k] for p in parts]) for k in range(len(parts[0]))]
            dev = [torch.from_numpy(st[0]).cuda(), torch.from_numpy(st[1].view(np.int16)).view(torch.bfloat16).cuda(),
                   torch.from_numpy(st[2]).cuda(), torch.from_numpy(st[3].view(np.int16)).view(torch.bfloat16).cuda()]
            if act_order:
                p1, p2 = torch.from_numpy(st[4]).cuda(), torch.from_numpy(st[5]).cuda()
                layer.prepack_act_order(dev[0], dev[1], p1, dev[2], dev[3], p2, first_expert=e0)
            else:
                layer.prepack(*dev, first_expert=e0)
            torch.cuda.synchronize()
            if e0 % 128 == 0:
                log(f"prepacked experts {first + e0}..{first + e0 + len(parts) - 1} of {dims.E} "
                    f"({time.time() - t0:.1f}s)")
    if shard:
        layer.set_expert_range(first, dims.E)
    return layer


def make_batches(dims, M, R, kind, seed0):
    import torch
    from synth import gen_hidden, gen_routing
    x = gen_hidden(M, dims.K, 1000 + M)
    ids, ws = [], []
    for r in range(R):
        i, w = gen_routing(kind, M, dims.E, dims.topk, seed0 + M + r)
        ids.append(i)
        ws.append(w)
    dx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    dids = torch.from_numpy(np.stack(ids)).cuda()
    dws = torch.from_numpy(np.stack(ws)).cuda()
    return x, np.stack(ids), np.stack(ws), dx, dids, dws


def layer_bytes(dims, M, ids_np, shard=None):
    """Algorithmic bytes of one call: int4 codes + bf16 scales of the distinct experts routed (those
    of the shard [first, first + n) only, for an expert-parallel share), plus hidden in, out, ids and
    weights."""
    per_expert = dims.expert_bytes
    first, n = shard if shard else (0, dims.E)
    act = [len(np.unique(i[(i >= first) & (i < first + n)])) for i in ids_np]
    return float(np.mean(act)) * per_expert + 2 * M * dims.K * 2 + M * dims.topk * 8, float(np.mean(act))


def gemm1_bytes(dims, M, ids_np):
    """Algorithmic bytes of one GEMM1 launch: W1 codes + scales of the routed experts, hidden in,
    the bf16 SwiGLU rows out."""
    w1 = dims.K * 2 * dims.N // 2 + (dims.K // 32) * 2 * dims.N * 2
    act = np.mean([len(np.unique(i)) for i in ids_np])
    return float(act) * w1 + M * dims.K * 2 + M * dims.topk * dims.N * 2


def layer_flops(dims, M, slots=None):
    """2 flops per multiply-add of every routed slot (`slots`: the mean count, default M * topk)."""
    slots = M * dims.topk if slots is None else slots
    return 2.0 * slots * (dims.K * 2 * dims.N + dims.N * dims.K)


def measured_traffic():
    """HBM bytes per launch of the M=1 kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads for a plain copy of known size).
    None when the summary is missing or was taken on another revision of the kernel source."""
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_FILE).read().split("```")[-2].strip().splitlines())
    except (OSError, IndexError, ValueError):
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    src = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    if fields.get("gemm_source_sha256") != src:
        return None
    return float(fields["hbm_bytes_per_launch"])


def copy_calibration(mib):
    """Plain device-to-device copies of a known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 copies of {n} bytes")


def time_calls(layer, dx, dids, dws, out, steps, warmup):
    import torch
    R = dids.shape[0]
    for s in range(warmup):
        layer.forward(dx, dids[s % R], dws[s % R], out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        layer.forward(dx, dids[s % R], dws[s % R], out)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def profile_calls(layer, dx, dids, dws, out, steps):
    import torch
    R = dids.shape[0]
    layer.set_profiling(True)
    for s in range(steps):
        layer.forward(dx, dids[s % R], dws[s % R], out)
    torch.cuda.synchronize()
    ms, calls = layer.read_profile()
    layer.set_profiling(False)
    return [m / max(calls, 1) for m in ms], calls


def graph_us_per_call(layer, dx, dids, dws, out, replays=10):
    """Per-call time when the R rotating calls are captured once in a HIP graph and the graph is
    replayed: the device-side cost without host launch overhead."""
    import torch
    R = dids.shape[0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(R):
            layer.forward(dx, dids[r], dws[r], out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            layer.forward(dx, dids[r], dws[r], out)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / (replays * R) * 1e6
    del g
    return round(dt, 2)


def call_latency_us(layer, dx, dids, dws, out, steps):
    """Per-call latency percentiles from the library's timing-only events (before the first kernel
    to after the last, one call at a time on the stream of back-to-back calls)."""
    import torch
    R = dids.shape[0]
    layer.set_profiling(True)
    for s in range(steps):
        layer.forward(dx, dids[s % R], dws[s % R], out)
    torch.cuda.synchronize()
    per_call = np.array(layer.read_profile_calls(steps)) * 1e3
    layer.set_profiling(False)
    return {q: round(float(np.percentile(per_call, p)), 2) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}


def scrubbed_latency_us(layer, dx, dids, dws, out, steps, scrub_mib=512, kind="read"):
    """Per-call latency (library events around the layer's kernels only) when a plain device pass over
    scrub_mib MiB runs before every call, evicting the weights of earlier calls from the 256 MB
    last-level cache: the cold time, beside the rotating-routing time of the other measurements.
    kind "read" scrubs with a reduction (the cache is left holding clean lines); "copy" with a copy,
    which leaves it full of dirty lines that the layer's own reads then write back to HBM."""
    import torch
    R = dids.shape[0]
    n = scrub_mib * 1024 * 1024
    src = torch.ones(n // 8, dtype=torch.int64, device="cuda")
    dst = torch.empty_like(src) if kind == "copy" else None
    acc = torch.zeros((), dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    layer.set_profiling(True)
    for s in range(steps):
        if kind == "copy":
            dst.copy_(src)
        else:
            torch.sum(src, dim=0, out=acc)
        layer.forward(dx, dids[s % R], dws[s % R], out)
    torch.cuda.synchronize()
    per_call = np.array(layer.read_profile_calls(steps)) * 1e3
    layer.set_profiling(False)
    del src, dst
    return {"p10": round(float(np.percentile(per_call, 10)), 2), "p50": round(float(np.percentile(per_call, 50)), 2),
            "p90": round(float(np.percentile(per_call, 90)), 2), "scrub": f"{kind} of {scrub_mib} MiB",
            "calls": int(steps)}


def rotations_for(dims, M, kind, seed0, min_sets=16, max_sets=128, shard=None):
    """Routing sets to cycle through so that one cycle streams at least 1 GB of weights (four times the
    256 MB last-level cache), so that repeated calls cannot be served from it."""
    from synth import gen_routing
    ids = np.stack([gen_routing(kind, M, dims.E, dims.topk, seed0 + M + r)[0] for r in range(min_sets)])
    per_call = layer_bytes(dims, M, ids, shard)[0]
    return int(min(max_sets, max(min_sets, np.ceil(1e9 / per_call))))


def sweep_point(layer, dims, M, kind, seed0, R=None, min_time=0.15, shard=None):
    import torch
    R = R or rotations_for(dims, M, kind, seed0, shard=shard)
    x, ids, ws, dx, dids, dws = make_batches(dims, M, R, kind, seed0)
    out = torch.empty((M, dims.K), dtype=torch.bfloat16, device="cuda")
    ms0 = time_calls(layer, dx, dids, dws, out, steps=3, warmup=2)
    steps = int(max(10, min(400, min_time * 1e3 / max(ms0, 1e-3))))
    ms = time_calls(layer, dx, dids, dws, out, steps=steps, warmup=3)
    nbytes, act = layer_bytes(dims, M, ids, shard)
    first, n = shard if shard else (0, dims.E)
    flops = layer_flops(dims, M, float(np.mean([((i >= first) & (i < first + n)).sum() for i in ids])))
    t_star = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    return {"M": M, "routing": kind, "ms_per_call": round(ms, 5), "tokens_per_s": round(M / (ms * 1e-3), 1),
            "us_per_token": round(ms * 1e3 / M, 3), "active_experts": round(act, 1), "alg_GB": round(nbytes / 1e9, 4),
            "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "roofline_ms": round(t_star, 5),
            "roofline_frac": round(t_star / ms, 4), "routing_sets": R}


def router_point(layer, dims, M, R=64, steps=200):
    """Router timings at M tokens, rotating R logit sets: the router kernel alone, and the routed layer
    (w4moe_forward_logits) against the layer fed a precomputed route (w4moe_forward)."""
    import torch
    from synth import gen_hidden, gen_logits
    dx = torch.from_numpy(gen_hidden(M, dims.K, 1000 + M).view(np.int16)).view(torch.bfloat16).cuda()
    dl = torch.from_numpy(np.stack([gen_logits(M, dims.E, 5000 + M + r) for r in range(R)])).cuda()
    out = torch.empty((M, dims.K), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((R, M, dims.topk), dtype=torch.int32, device="cuda")
    ws = torch.empty((R, M, dims.topk), dtype=torch.float32, device="cuda")
    for r in range(R):
        ids[r], ws[r] = layer.route(dl[r])

    def timed(fn):
        for s in range(10):
            fn(s % R)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            fn(s % R)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    from int4_weight_only_align_amd.w4moe import w4moe_forward_logits
    t_route = timed(lambda r: layer.route(dl[r]))
    t_layer = timed(lambda r: layer.forward(dx, ids[r], ws[r], out))
    t_both = timed(lambda r: w4moe_forward_logits(layer.handle, dx, M, dl[r], ids[r], ws[r], out))
    return {"M": M, "route_us": round(t_route, 2), "layer_us": round(t_layer, 2),
            "routed_layer_us": round(t_both, 2), "plan": layer.resolved_plan(M)}


def cpu_info():
    """The host CPU as lscpu names it, its logical CPU count (nproc --all) and how many of them this
    process may run on (its affinity mask)."""
    import subprocess
    model = "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        model = next(l.split(":", 1)[1].strip() for l in out.splitlines() if l.startswith("Model name"))
    except (OSError, StopIteration, subprocess.SubprocessError):
        try:
            model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
        except (OSError, StopIteration):
            pass
    return {"cpu_model": model, "nproc_all": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(dims, n_tokens, sweep_m=(1, 9, 90, 256, 1024), rows_per_m=6):
    """The oracle, unchanged, using the threads OMP_NUM_THREADS allows (else every CPU of the
    affinity mask). Headline: n_tokens decode calls (M=1) of the headline workload, each with its own
    routing (seeds of the headline rotation, extended). Sweep: for each M, the oracle on rows_per_m
    token rows (spread over the batch) of that M's first sweep batch, timed alone; the oracle's cost
    per row does not depend on M (each row is its top-k experts' FFNs), so its tokens/s is the rate
    at which it would produce the whole batch."""
    from oracle import moe_forward
    from synth import ExpertStore, gen_hidden, gen_routing_softmax
    x = gen_hidden(1, dims.K, 1001)
    routes = [gen_routing_softmax(1, dims.E, dims.topk, 2001 + r) for r in range(n_tokens)]
    store = ExpertStore(dims, 2)
    needed = sorted({int(e) for ids, _ in routes for e in ids.reshape(-1)})
    sweep_in = []
    for M in sweep_m:
        ids, w = gen_routing_softmax(M, dims.E, dims.topk, 2000 + M)
        rows = np.unique(np.linspace(0, M - 1, min(rows_per_m, M)).round().astype(np.int32))
        sweep_in.append((M, gen_hidden(M, dims.K, 1000 + M), ids, w, rows))
        needed = sorted(set(needed) | {int(e) for e in ids[rows].reshape(-1)})
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(lambda e: store[e], needed))
    nthreads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    for ids, w in routes:
        moe_forward(dims, x, ids, w, store, nthreads=nthreads)
    dt = time.perf_counter() - t0
    sweep = []
    for M, xs, ids, w, rows in sweep_in:
        t1 = time.perf_counter()
        moe_forward(dims, xs, ids, w, store, rows=rows, nthreads=nthreads)
        ds = time.perf_counter() - t1
        sweep.append({"M": M, "rows_timed": int(rows.size), "seconds": round(ds, 3),
                      "tokens_per_s": round(rows.size / ds, 3), "ms_per_call_extrapolated": round(ds / rows.size * M * 1e3, 1)})
    info = cpu_info()
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{n_tokens} decode calls (M=1, K2.6 dims, each its own routing), fp64 oracle, "
                      f"{dt:.1f} s wall; sweep: {rows_per_m} token rows of each M's uniform batch",
            **info, "sweep": sweep}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # a few milliseconds of back-to-back calls before the timed region: fewer leave the clocks
    # ramping (20 warmup calls measured 44.8 us/call where 200 measured 43.2 on the same box)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotations", type=int, default=64)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=128)
    ap.add_argument("--sweep-m", default="", metavar="M,M,...",
                    help="sweep only these token counts (one layer, one routing; no other sweep points)")
    ap.add_argument("--sweep-config", default="k26", choices=("k26", "k26_tp8", "k26_ep8"),
                    help="with --sweep-m: the layer swept (k26_tp8: one GPU's share of a TP8 layer, N=256; "
                         "k26_ep8: one GPU's share of an EP8 layer, experts 144..191 of 384)")
    ap.add_argument("--sweep-routing", default="softmax", choices=("softmax", "zipf"),
                    help="with --sweep-m: uniform (softmax) or Zipf(1.2)-skewed routing")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed regions, run three plain copies of MIB MiB (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a single MI355X "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import __graft_entry__
    __graft_entry__._ensure_built()
    import torch
    from synth import CONFIGS

    torch.cuda.set_device(0)
    dims = CONFIGS["k26"]
    log(f"device: {torch.cuda.get_device_name(0)}")
    layer = build_layer(dims, 2, max_tokens=1024)

    M = 1
    x, ids, ws, dx, dids, dws = make_batches(dims, M, args.rotations, "softmax", 2000)
    out = torch.empty((M, dims.K), dtype=torch.bfloat16, device="cuda")
    # timed region: W warmup calls, then exactly K calls between two device synchronisations
    ms = time_calls(layer, dx, dids, dws, out, args.steps, args.warmup)
    value = M / (ms * 1e-3)
    prof_steps = min(args.steps, 1024)   # the library keeps the events of the last 1024 calls
    stage_ms, calls = profile_calls(layer, dx, dids, dws, out, prof_steps)
    latency = call_latency_us(layer, dx, dids, dws, out, prof_steps)
    latency["graph_replay_us_per_call"] = graph_us_per_call(layer, dx, dids, dws, out)
    latency["cold_scrubbed"] = scrubbed_latency_us(layer, dx, dids, dws, out, min(prof_steps, 300))
    latency["cold_scrubbed_by_copy"] = scrubbed_latency_us(layer, dx, dids, dws, out, min(prof_steps, 300), kind="copy")
    timed_ids = ids[:min(args.steps, args.rotations)]
    lb, act = layer_bytes(dims, M, ids)
    if layer.resolved_plan(M) == 3:
        # one launch does the whole layer; its event interval is the GEMM1 stage
        kname, kbytes = "gemm_pair_fused (W1 gate|up + SwiGLU, W2, top-k combine)", layer_bytes(dims, M, timed_ids)[0]
    else:
        kname, kbytes = "gemm1 (W1 gate|up + SwiGLU)", gemm1_bytes(dims, M, timed_ids)
    achieved = kbytes / (stage_ms[1] * 1e-3) / 1e9
    traffic = measured_traffic() if kname.startswith("gemm_pair_fused") else None
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": kname, "alg_bytes_per_launch": round(kbytes), "avg_launch_ms": round(stage_ms[1], 5)}
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": round(value / PAGES_TOKS_M1, 3), "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "K2.6 W4A16 MoE decode: E=384 K=7168 N=2048 top-8 g32, M=1, "
                               f"{args.rotations} rotating softmax routings", "M": M, "E": dims.E, "K": dims.K,
                   "N": dims.N, "topk": dims.topk, "group": 32, "parallelism": "single GPU"},
        "roofline": roof,
        "latency_us": latency,
        "per_kernel_ms": {"align": round(stage_ms[0], 5), "gemm1": round(stage_ms[1], 5),
                          "gemm2": round(stage_ms[2], 5), "combine": round(stage_ms[3], 5), "calls": calls},
        "layer_alg_GB_per_call": round(lb / 1e9, 4), "layer_GB_per_s": round(lb / (ms * 1e-3) / 1e9, 1),
        "layer_hbm_frac": round(lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    log(f"headline M=1: {ms * 1e3:.1f} us/call, {value:.0f} tok/s; per-kernel ms {stage_ms}")

    if not args.no_sweep:
        res["router"] = [router_point(layer, dims, Mr) for Mr in (1, 8, 256)]
        for r in res["router"]:
            log(json.dumps(r))

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    if args.sweep_m and not args.no_sweep:
        sdims, slayer, shard = dims, layer, None
        if args.sweep_config == "k26_tp8":
            sdims = CONFIGS[args.sweep_config]
            slayer = build_layer(sdims, 5, max_tokens=1024)
        elif args.sweep_config == "k26_ep8":
            shard = EP8_SHARD
            slayer = build_layer(sdims, 2, max_tokens=1024, shard=shard)
        res["sweep_config"] = args.sweep_config
        res["sweep"] = []
        seed0 = 2000 if args.sweep_routing == "softmax" else 3000
        for Ms in (int(v) for v in args.sweep_m.split(",")):
            res["sweep"].append(sweep_point(slayer, sdims, Ms, args.sweep_routing, seed0, shard=shard))
            log(json.dumps(res["sweep"][-1]))
        if slayer is not layer:
            slayer.close()
    elif not args.no_sweep:
        sweep = []
        for Ms in SWEEP_M:
            sweep.append(sweep_point(layer, dims, Ms, "softmax", 2000))
            log(json.dumps(sweep[-1]))
        for Ms in (256, 512, 1024):
            sweep.append(sweep_point(layer, dims, Ms, "zipf", 3000))
            log(json.dumps(sweep[-1]))
        res["sweep"] = sweep
        layer.close()
        del layer
        torch.cuda.empty_cache()
        # the same layer with 8-bit codes (W8A16): twice the code bytes per expert
        from dataclasses import replace as _replace
        w8 = _replace(dims, bits=8)
        wl = build_layer(w8, 2, max_tokens=1024)
        res["sweep_w8"] = [sweep_point(wl, w8, Ms, "softmax", 2000) for Ms in (1, 90, 256, 1024)]
        for r in res["sweep_w8"]:
            log(json.dumps(r))
        wl.close()
        del wl
        torch.cuda.empty_cache()
        # activation-ordered weights (GPTQ act-order): the same layer plus the per-entry row gather
        al = build_layer(dims, 2, max_tokens=1024, act_order=True)
        res["sweep_act_order"] = [sweep_point(al, dims, Ms, "softmax", 2000) for Ms in (1, 90, 256, 1024)]
        for r in res["sweep_act_order"]:
            log(json.dumps(r))
        al.close()
        del al
        torch.cuda.empty_cache()
        tp = CONFIGS["k26_tp8"]
        tl = build_layer(tp, 5, max_tokens=1024)
        res["sweep_tp8_shard"] = []
        for Ms in (1, 90, 330, 1024):
            res["sweep_tp8_shard"].append(sweep_point(tl, tp, Ms, "softmax", 2000))
            log(json.dumps(res["sweep_tp8_shard"][-1]))
        tl.close()
        del tl
        torch.cuda.empty_cache()
        # one GPU's share of an EP8 layer: 48 of the 384 experts, fed global routing ids
        el = build_layer(dims, 2, max_tokens=1024, shard=EP8_SHARD)
        res["sweep_ep8_shard"] = []
        for Ms in (1, 90, 330, 1024):
            res["sweep_ep8_shard"].append(sweep_point(el, dims, Ms, "softmax", 2000, shard=EP8_SHARD))
            log(json.dumps(res["sweep_ep8_shard"][-1]))
        el.close()

    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(dims, args.cpu_tokens)
        log(f"cpu baseline: {res['cpu_baseline']}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
