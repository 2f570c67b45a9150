#!/usr/bin/env python3
"""Benchmark: one decode step = one paged_decode_attention call (split kernel +
combine) over one batch of synthetic input, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C2]

Prints ONE JSON line.  ``value`` is the effective KV-cache bandwidth (bytes of
K and V rows the step must read / time per step) in GB/s; ``ms_per_step`` is
the time per step.  Inputs are resident in HBM before the timed region.  To
measure HBM rather than the 256 MB Infinity Cache, the step cycles over R
device replicas of the cache (R x bytes >= 1 GiB), and the K steps are
replayed from one HIP graph, timed with HIP events on the launch stream.

``roofline`` describes the dominant kernel (the split kernel): algorithmic KV
bytes per launch / its average duration (HIP events around a graph of K
partial-only launches on the same stream), against the 8 TB/s HBM peak.
``traffic`` is filled from the committed rocprofv3 counter summary
(profiles/) when it was taken on the current kernel source, else null.
``cpu_baseline`` times the FP64 oracle on the host cores on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense FP16 MFMA (the contractions run in FP16)
METRIC = "µs/decode step and effective KV-cache GB/s (% of MI355X HBM peak)"
KERNEL_SRC = os.path.join(ROOT, "quantized_paged_kv_amd", "csrc", "pkv_kernels.hip")
WRITER_SRC = os.path.join(ROOT, "quantized_paged_kv_amd", "csrc", "pkv_cache_write.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel: str, workload: str, src: str = KERNEL_SRC):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    if it was taken on this kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, budget_s: float = 12.0):
    """Time the FP64 oracle (as it stands) on the host cores on a bounded sample:
    whole steps of the workload if one step fits the budget, else a subset of
    its rows.  Returns the dict for the JSON line."""
    import numpy as np

    import oracle
    from workloads import live_token_counts

    p = inp.problem
    cores = os.cpu_count() or 1
    counts = live_token_counts(inp)
    row_bytes = (p.head_size if p.layout == "latent" else p.head_size + p.v_head_size) * p.cache_itemsize
    # probe one row to size the sample
    t0 = time.perf_counter()
    oracle.paged_decode(inp, threads=cores, rows=[0])
    t_row = max(time.perf_counter() - t0, 1e-4)
    rows_fit = max(1, int(budget_s / t_row))
    if rows_fit >= p.rows:
        reps = max(1, int(budget_s / (t_row * p.rows)))
        rows = None
        nrows = p.rows
        sample = f"{reps} full step(s) of the workload ({p.rows} rows)"
    else:
        reps = 1
        rows = list(range(min(p.rows, rows_fit)))
        nrows = len(rows)
        sample = f"{nrows} of {p.rows} rows of one step"
    units = nrows * p.kv_heads
    used = min(cores, units)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.paged_decode(inp, threads=cores, rows=rows)
    dt = time.perf_counter() - t0
    sel = counts if rows is None else counts[rows]
    kv_bytes = int(sel.sum()) * p.kv_heads * row_bytes * reps
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle",
            "sample": f"{sample}; FP64 C oracle, {used} threads over (row, KV head) units; "
                      f"{dt:.1f} s wall; {dt / reps * 1e3 * p.rows / nrows:.1f} ms per full step"}


def bench_write(args, dev):
    """The cache writer alone: --write-tokens new rows of the workload's
    cache format (KV heads, head sizes, dtype, scale granularity) written at
    distinct random slots, cycling over device replicas (inputs and caches)
    of >= --replica-bytes so the traffic reaches HBM.  Algorithmic bytes per
    call: the FP16 rows read, the codes written, the slot indices and the
    per-channel scales."""
    import dataclasses

    import numpy as np
    import torch

    import quantized_paged_kv_amd as pkv
    import workloads
    from workloads.device import problem_kwargs

    base = workloads.workload(args.workload).problem
    T = args.write_tokens
    p = dataclasses.replace(base, num_pool_blocks=-(-T // base.block_size))
    nt = workloads.new_tokens(p, T, seed=31, skip_fraction=0.0)
    prob = pkv.make_problem(**problem_kwargs(p))
    latent = p.layout == "latent"
    item = p.cache_itemsize
    dims = p.head_size + (0 if latent else p.v_head_size)
    scale_bytes = sum(4 * (p.kv_heads * d if q == "channel" else (1 if q == "tensor" else 0))
                      for q, d in ([(p.k_quant, p.head_size)] if latent else
                                   [(p.k_quant, p.head_size), (p.v_quant, p.v_head_size)]))
    algo = T * p.kv_heads * dims * (2 + item) + 8 * T + scale_bytes

    def dev_t(a):
        if a is None:
            return None
        if a.dtype == np.float16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.float16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    key, val = dev_t(nt.key), dev_t(nt.value)
    slots, ks, vs = dev_t(nt.slot_mapping), dev_t(nt.k_scale), dev_t(nt.v_scale)
    cdt = torch.float16 if p.cache_dtype == "f16" else torch.uint8
    kc = torch.zeros((p.num_pool_blocks, p.block_size, p.kv_heads, p.head_size), dtype=cdt,
                     device=dev)
    vc = None if latent else torch.zeros((p.num_pool_blocks, p.block_size, p.kv_heads,
                                          p.v_head_size), dtype=cdt, device=dev)
    R = max(1, min(args.steps, math.ceil(args.replica_bytes / max(algo, 1))))
    keys = [key] + [key.clone() for _ in range(R - 1)]
    vals = [val] + ([val.clone() for _ in range(R - 1)] if val is not None else [None] * (R - 1))
    kcs = [kc] + [kc.clone() for _ in range(R - 1)]
    vcs = [vc] + ([vc.clone() for _ in range(R - 1)] if vc is not None else [None] * (R - 1))
    log(f"writer {args.workload} format: {T} tokens, {algo} bytes/call, replicas {R}")

    def call(i):
        pkv.reshape_and_cache(prob, keys[i % R], vals[i % R], slots, ks, vs, kcs[i % R],
                              vcs[i % R])

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    K = args.steps
    if args.eager:
        def replay():
            for i in range(K):
                call(i)
    else:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(K):
                call(i)
        replay = g.replay
        replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    gbs = algo / (ms * 1e-3) / 1e9
    traffic = read_traffic("cache_write_kernel", f"{args.workload}_T{T}", WRITER_SRC)
    log(f"writer {ms * 1e3:.2f} us per call ({gbs:.0f} GB/s)")
    print(json.dumps({
        "metric": "cache-writer GB/s (FP16 rows read + codes written, % of MI355X HBM peak)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"reshape_and_cache, {T} tokens in the {args.workload} cache "
                               f"format ({p.cache_dtype}, k {p.k_quant}, v {p.v_quant}, "
                               f"{p.layout})",
                   "cold_cache_replicas": R,
                   "timing": ("K eager launches" if args.eager else
                              "one HIP-graph replay of K calls") + ", HIP events"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "cache_write_kernel",
                     "kernel_us": round(ms * 1e3, 3), "algorithmic_bytes_per_launch": algo},
    }), flush=True)
    return 0


def workloads_names():
    import workloads

    return list(workloads.WORKLOADS)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="C2", choices=sorted(workloads_names()),
                    help="C1..C5: the decode configurations; P<rows>: the dynamic-sparse "
                         "prefill shape (rows x 2048 gathered candidates, MFMA-bound); "
                         "X<ctx>b<batch><dtype>: the PagedAttention page's isolated decode "
                         "shapes (64q/8kv, head 64, block 256)")
    ap.add_argument("--replica-bytes", type=float, default=1.0 * (1 << 30),
                    help="cold-cache protocol: replicate the cache until this many bytes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="split-count override (0 = automatic)")
    ap.add_argument("--min-chunk", type=int, default=0, help="geometry min_chunk (0 = default)")
    ap.add_argument("--waves", type=int, default=0, help="geometry target waves (0 = default)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step eagerly instead of from a HIP graph (for "
                         "per-dispatch hardware counters)")
    ap.add_argument("--op", default="decode", choices=["decode", "write"],
                    help="decode: the decode step (default); write: the quantise-on-write "
                         "cache writer (reshape_and_cache) on the workload's cache format")
    ap.add_argument("--write-tokens", type=int, default=16384,
                    help="new tokens per writer call (--op write)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 4 plain device-to-device copies of this many bytes and exit "
                         "(calibrates the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has "
              "no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import quantized_paged_kv_amd as pkv
    import workloads
    from workloads.device import to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_bytes > 0:
        a = torch.ones(args.copy_bytes, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.copy_bytes} bytes 4 times")
        return 0
    pkv.load()
    if args.op == "write":
        return bench_write(args, dev)

    log(f"generating {args.workload}")
    inp = workloads.workload(args.workload)
    p = inp.problem
    kv_bytes = inp.effective_kv_bytes()
    d = to_device(inp, dev)
    prob = pkv.make_problem(**d.problem_kwargs)
    geo = pkv.split_geometry(prob, splits_override=args.splits, min_chunk=args.min_chunk,
                             waves=args.waves)
    ws = pkv.workspace_for(geo, dev)

    # cold-cache replicas of the caches (the block table, lengths, Q, scales are shared)
    cache_bytes = d.key_cache.numel() * d.key_cache.element_size()
    if d.value_cache is not None:
        cache_bytes += d.value_cache.numel() * d.value_cache.element_size()
    R = max(1, min(args.steps, math.ceil(args.replica_bytes / max(cache_bytes, 1))))
    log(f"{args.workload}: kv bytes/step {kv_bytes}, cache bytes {cache_bytes}, replicas {R}, "
        f"splits {geo.num_splits}")
    keys = [d.key_cache] + [d.key_cache.clone() for _ in range(R - 1)]
    vals = [d.value_cache] + ([d.value_cache.clone() for _ in range(R - 1)]
                              if d.value_cache is not None else [None] * (R - 1))
    odt = torch.float32 if d.problem_kwargs["out_dtype"] == "f32" else torch.float16
    out = torch.empty((p.rows, p.heads, p.v_head_size), dtype=odt, device=dev)
    lse = torch.empty((p.rows, p.heads), dtype=torch.float32, device=dev)

    def step(i):
        pkv.paged_decode_attention(prob, geo, d.query, keys[i % R], vals[i % R], d.block_table,
                                   d.seq_lens, d.candidates, d.num_candidates, d.k_scale,
                                   d.v_scale, d.softmax_scale, d.head_sink, out, lse, ws)

    def partial(i):
        pkv.paged_decode_partials(prob, geo, d.query, keys[i % R], vals[i % R], d.block_table,
                                  d.seq_lens, d.candidates, d.num_candidates, d.k_scale,
                                  d.v_scale, d.softmax_scale, ws)

    # warmup (eager, untimed)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    class Eager:
        def __init__(self, fn, n):
            self.fn, self.n = fn, n

        def replay(self):
            for i in range(self.n):
                self.fn(i)

    def capture(fn, n):
        if args.eager:
            return Eager(fn, n)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    K = args.steps
    g_step = capture(step, K)
    g_part = capture(partial, K)
    g_step.replay()  # untimed: first replay of the graph
    g_part.replay()
    torch.cuda.synchronize()

    # timed region: exactly K steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g_step.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / K

    # dominant kernel alone: K partial-only launches, same stream
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f0.record()
    g_part.replay()
    f1.record()
    torch.cuda.synchronize()
    ms_split = f0.elapsed_time(f1) / K

    value = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes / (ms_split * 1e-3) / 1e9
    # prefill shapes gather cache-resident rows many times over: there the
    # contractions bound the kernel (QK^T and PV, 2 (D + VD) flops per head
    # and attended token; the GQA group is padded to the 16-wide MFMA tile,
    # which is not counted)
    prefill = args.workload.startswith("P")
    flops = 0
    if prefill:
        from workloads import live_token_counts
        dims = p.head_size + p.v_head_size
        flops = int(live_token_counts(inp).sum()) * p.heads * 2 * dims
        tflops = flops / (ms_split * 1e-3) / 1e12
    kernel = "latent_kernel" if p.layout == "latent" else "split_kernel"
    traffic = read_traffic(kernel, args.workload)
    log(f"step {ms_step * 1e3:.2f} us ({value:.0f} GB/s), split kernel {ms_split * 1e3:.2f} us "
        f"({achieved:.0f} GB/s)")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": inp.name,
            "us_per_step": round(ms_step * 1e3, 3),
            "effective_kv_bytes_per_step": kv_bytes,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "cache_dtype": p.cache_dtype,
            "compute": "K/V codes converted to fp16 in registers; fp16 MFMA with fp32 "
                       "accumulation; fp32 softmax",
            "num_splits": geo.num_splits,
            "cold_cache_replicas": R,
            "timing": ("K eager launches" if args.eager else "one HIP-graph replay of K steps")
                      + ", HIP events on the launch stream",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": f"{kernel} (paged_decode_partials)",
            "kernel_us": round(ms_split * 1e3, 3),
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if prefill:
        line["roofline"] = {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": f"{kernel} (paged_decode_partials)",
            "kernel_us": round(ms_split * 1e3, 3),
            "algorithmic_flops_per_launch": flops,
            "gathered_kv_bytes_per_launch": kv_bytes,
        }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores")
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
