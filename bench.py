#!/usr/bin/env python3
"""Benchmark: one decode step = one paged_decode_attention call (split kernel +
combine) over one batch of synthetic input, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3] [--also C5]

Prints ONE JSON line.  The default workload is the continuous-batching FP16
step (16 rows of 512..8192 tokens, 32 query / 8 KV heads, head 128, ~290 MB of
K and V per step), the largest configuration; the latent FP8 step (32 rows x
4096 tokens) is timed the same way and reported in ``also``.  ``value`` is
the effective KV-cache bandwidth (bytes of K and V rows the step must read /
time per step) in GB/s; ``ms_per_step`` is the time per step.  Inputs are
resident in HBM before the timed region.  To measure HBM rather than the
256 MB Infinity Cache, step i reads replica i mod R of the caches (R x bytes
>= 1 GiB, whatever K is) and every timed round starts after an untimed
512 MiB read.  The K steps are replayed from one HIP graph and timed with
HIP events on the launch stream; the reported time is the median of
``--rounds`` (7) rounds after W eager warmup steps and one untimed replay,
the protocol of the DSA page's H200 measurements.

``roofline`` describes the dominant kernel (the split kernel): algorithmic KV
bytes per launch / its average duration (HIP events around a graph of K
partial-only launches on the same stream, same rounds), against the 8 TB/s
HBM peak.  ``traffic`` is filled from the committed rocprofv3 counter
summary (profiles/) when it was taken on the current kernel source, else
null.  ``cpu_baseline`` times the FP64 oracle on the host cores on a
bounded sample of the same workload.
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


def cpu_baseline(inp, budget_s: float = 15.0):
    """Time the FP64 oracle (as it stands) on the host cores on a bounded sample:
    the median of 3 runs with one thread per host CPU (whole steps of the
    workload if one step fits a quarter of the budget, else a subset of its
    rows), plus one single-thread run on a smaller subset of rows.  Returns
    the dict for the JSON line; `cores` is the number of threads the oracle
    ran with, `host_cpus` what the host reports."""
    import oracle
    from workloads import live_token_counts

    p = inp.problem
    cores = os.cpu_count() or 1
    counts = live_token_counts(inp)
    row_bytes = (p.head_size if p.layout == "latent" else p.head_size + p.v_head_size) * p.cache_itemsize

    def gbs(rows, dt, reps=1):
        sel = counts if rows is None else counts[rows]
        return int(sel.sum()) * p.kv_heads * row_bytes * reps / dt / 1e9

    # probe one row to size the sample
    t0 = time.perf_counter()
    oracle.paged_decode(inp, threads=cores, rows=[0])
    t_row = max(time.perf_counter() - t0, 1e-4)
    run_s = budget_s / 4
    rows_fit = max(1, int(run_s / t_row))
    if rows_fit >= p.rows:
        reps = max(1, int(run_s / (t_row * p.rows)))
        rows = None
        nrows = p.rows
        sample = f"{reps} full step(s) of the workload ({p.rows} rows) per run"
    else:
        reps = 1
        rows = list(range(min(p.rows, rows_fit)))
        nrows = len(rows)
        sample = f"{nrows} of {p.rows} rows of one step per run"
    used = min(cores, nrows * p.kv_heads)  # the oracle's threads take (row, KV head) units
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.paged_decode(inp, threads=cores, rows=rows)
        runs.append(time.perf_counter() - t0)
    dt = _median(runs)
    # single thread: as many rows as fit a quarter of the budget
    rows1 = list(range(max(1, min(p.rows, int(run_s / (t_row * used))))))
    t0 = time.perf_counter()
    oracle.paged_decode(inp, threads=1, rows=rows1)
    dt1 = time.perf_counter() - t0
    return {"value": round(gbs(rows, dt, reps), 4), "unit": "GB/s", "cores": used,
            "host_cpus": cores, "kind": "oracle",
            "single_thread_value": round(gbs(rows1, dt1), 4),
            "sample": f"{sample}; FP64 C oracle, {used} threads over (row, KV head) units "
                      f"(host reports {cores} CPUs); median of 3 runs "
                      f"({', '.join(f'{x:.2f}' for x in runs)} s), "
                      f"{dt / reps * 1e3 * p.rows / nrows:.1f} ms per full step; single "
                      f"thread on {len(rows1)} row(s): {dt1:.2f} s"}


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
    R = max(1, math.ceil(args.replica_bytes / max(algo, 1)))
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
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    rounds = []
    for _ in range(args.rounds):
        flush.max()  # untimed: a 512 MiB read evicts the Infinity Cache
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        replay()
        e1.record()
        torch.cuda.synchronize()
        rounds.append(e0.elapsed_time(e1) / K)
    ms = _median(rounds)
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
                   "timing": f"median of {args.rounds} rounds; each round "
                             + ("K eager launches" if args.eager else
                                "one HIP-graph replay of K calls")
                             + ", HIP events, after an untimed 512 MiB read"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "cache_write_kernel",
                     "kernel_us": round(ms * 1e3, 3), "algorithmic_bytes_per_launch": algo},
    }), flush=True)
    return 0


# ---- rocprofv3 summaries (profiles/) -----------------------------------------

PMC_SQ = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_LEVEL_WAVES SQ_ACTIVE_INST_LDS "
          "SQ_LDS_BANK_CONFLICT SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA")


def _pmc_commands(w: str, tag: str) -> list:
    """The rocprofv3 runs a counter summary is made from ($R = repository
    root); they run committed files only."""
    run = (f"python3 $R/bench.py --workload {w} --also= --rounds 3 --eager --steps 20 --warmup 2 "
           "--no-cpu-baseline")
    cmds = []
    for name, pmc in (("FETCH_SIZE", "FETCH_SIZE"), ("WRITE_SIZE", "WRITE_SIZE"), ("SQ", PMC_SQ)):
        cmds.append(f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 90 rocprofv3 --pmc {pmc} "
                    f"--output-format csv -d $R/gpurun_out/{tag}/pmc_{name}_{w} -o p -- {run}")
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds.append(f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 90 rocprofv3 --pmc {name} "
                    f"--output-format csv -d $R/gpurun_out/{tag}/pmc_{name}_copy -o p -- "
                    f"python3 $R/bench.py --copy-bytes 268435456")
    return cmds


def _read_counters(path: str) -> dict:
    """{kernel name: {counter: mean value per dispatch}} from a rocprofv3
    counter_collection.csv."""
    import csv
    import glob

    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {path}")
    sums, disp = {}, {}
    for f in files:
        for row in csv.DictReader(open(f)):
            k = row["Kernel_Name"]
            sums.setdefault(k, {}).setdefault(row["Counter_Name"], 0.0)
            sums[k][row["Counter_Name"]] += float(row["Counter_Value"])
            disp.setdefault(k, set()).add(row["Dispatch_Id"])
    return {k: {c: v / len(disp[k]) for c, v in cs.items()} | {"_dispatches": len(disp[k])}
            for k, cs in sums.items()}


def _dispatch_resources(path: str, kernel_name: str):
    """(grid size, workgroup size, VGPRs, LDS bytes) of the kernel's first
    dispatch in a counter_collection.csv, or None."""
    import csv
    import glob

    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Kernel_Name"] == kernel_name:
                return (int(row["Grid_Size"]), int(row["Workgroup_Size"]),
                        int(row["VGPR_Count"]) + int(row.get("Accum_VGPR_Count") or 0),
                        int(row["LDS_Block_Size"]))
    return None


def _attention_kernel(counters: dict, layout: str) -> str:
    """The attention kernel's short name among the profiled kernels."""
    names = ("latent_kernel",) if layout == "latent" else ("split_kvp_kernel", "split_kernel")
    for n in names:
        if any(f"pkv::{n}" in k for k in counters):
            return n
    raise KeyError(f"no attention kernel ({names}) among {list(counters)}")


def _pick(counters: dict, fragment: str):
    hits = [k for k in counters if fragment in k]
    return (hits[0], counters[hits[0]]) if hits else (None, {})


def summarize_counters(tag_dir: str, w: str) -> str:
    """The counter summary of the attention kernels of workload w from the
    rocprofv3 runs under tag_dir (see _pmc_commands)."""
    import workloads

    inp = workloads.workload(w)
    p = inp.problem
    fetch = _read_counters(os.path.join(tag_dir, f"pmc_FETCH_SIZE_{w}"))
    kernel = _attention_kernel(fetch, p.layout)
    write = _read_counters(os.path.join(tag_dir, f"pmc_WRITE_SIZE_{w}"))
    sq = _read_counters(os.path.join(tag_dir, f"pmc_SQ_{w}"))
    cf = _read_counters(os.path.join(tag_dir, "pmc_FETCH_SIZE_copy"))
    cw = _read_counters(os.path.join(tag_dir, "pmc_WRITE_SIZE_copy"))
    copy_kib = 268435456 / 1024
    _, cfv = _pick(cf, "copyBuffer")
    _, cwv = _pick(cw, "copyBuffer")
    fscale = copy_kib / cfv["FETCH_SIZE"]
    wscale = copy_kib / cwv["WRITE_SIZE"]
    kname, kf = _pick(fetch, f"pkv::{kernel}")
    _, kw = _pick(write, f"pkv::{kernel}")
    _, ks = _pick(sq, f"pkv::{kernel}")
    algo = inp.effective_kv_bytes()
    rd = kf["FETCH_SIZE"] * fscale * 1024
    wr = kw["WRITE_SIZE"] * wscale * 1024
    tag = os.path.basename(os.path.normpath(tag_dir))
    lines = [f"# HBM traffic and SQ counters of {kernel} on workload {w} ({inp.name}),",
             "# from rocprofv3 hardware counters, one run per counter set ($R = repository root).",
             "# runs:"]
    lines += [f"#   {c}" for c in _pmc_commands(w, tag)]
    lines += ["# summary: python3 $R/bench.py --summarize-counters $R/gpurun_out/" + tag
              + f" --workload {w}",
              "# scale = KiB the 256 MiB copy really reads (writes) / KiB the counter reports for it;",
              "# hbm bytes = counter KiB per dispatch x scale x 1024, averaged over the kernel's dispatches;",
              "# SQ counters: mean per dispatch, summed over the chip as rocprofv3 reports them.",
              f"kernel: {kname}",
              f"kernel_source_sha256_16: {kernel_source_hash()}",
              f"dispatches: {kf['_dispatches']}",
              f"fetch_size_kib_per_dispatch: {kf['FETCH_SIZE']:.1f}",
              f"write_size_kib_per_dispatch: {kw['WRITE_SIZE']:.1f}",
              f"copy_fetch_size_kib_per_dispatch: {cfv['FETCH_SIZE']:.1f}",
              f"copy_write_size_kib_per_dispatch: {cwv['WRITE_SIZE']:.1f}",
              f"fetch_scale: {fscale:.4f}",
              f"write_scale: {wscale:.4f}",
              f"hbm_read_bytes_per_launch: {rd:.0f}",
              f"hbm_write_bytes_per_launch: {wr:.0f}",
              f"hbm_bytes_per_launch: {rd + wr:.0f}",
              f"algorithmic_kv_bytes_per_launch: {algo}",
              f"read_over_algorithmic: {rd / algo:.4f}"]
    for c in PMC_SQ.split():
        if c in ks:
            lines.append(f"{c.lower()}_per_dispatch: {ks[c]:.4g}")
    if ks.get("SQ_ACTIVE_INST_LDS"):
        lines.append("lds_bank_conflict_cycles_per_lds_active_cycle: "
                     f"{ks['SQ_LDS_BANK_CONFLICT'] / ks['SQ_ACTIVE_INST_LDS']:.3f}")
    if ks.get("SQ_BUSY_CYCLES") and ks.get("SQ_LEVEL_WAVES"):
        lines.append("sq_level_waves_per_busy_cycle: "
                     f"{ks['SQ_LEVEL_WAVES'] / ks['SQ_BUSY_CYCLES']:.2f}")
    # the dispatch's resources as rocprofv3 records them (LDS in its
    # allocation granule; gfx950 has 160 KiB of LDS per CU)
    occ = _dispatch_resources(os.path.join(tag_dir, f"pmc_SQ_{w}"), kname)
    if occ:
        grid, wg, vgpr, lds = occ
        lines += [f"grid_ctas: {grid // wg}", f"threads_per_cta: {wg}",
                  f"lds_bytes_per_cta: {lds}",
                  f"lds_limit_ctas_per_cu: {(160 * 1024) // lds if lds else 'none'}",
                  f"rocprof_vgpr_count: {vgpr}"]
    cname, cfc = _pick(fetch, "pkv::combine")
    if cname:
        _, cwc = _pick(write, "pkv::combine")
        lines += [f"combine_kernel: {cname}",
                  f"combine_hbm_read_bytes_per_launch: {cfc['FETCH_SIZE'] * fscale * 1024:.0f}",
                  f"combine_hbm_write_bytes_per_launch: {cwc['WRITE_SIZE'] * wscale * 1024:.0f}"]
    return "\n".join(lines) + "\n"


def summarize_trace(tag_dir: str, w: str, bench_log: str = "") -> str:
    """The per-kernel duration statistics of a rocprofv3 --kernel-trace --stats
    run of bench.py on workload w."""
    import csv
    import glob

    files = glob.glob(os.path.join(tag_dir, f"kt_{w}", "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_stats.csv under {tag_dir}/kt_{w}")
    tag = os.path.basename(os.path.normpath(tag_dir))
    lines = [f"# rocprofv3 kernel-trace statistics of bench.py on workload {w}",
             "# command ($R = repository root):",
             f"#   cd /tmp && export TMPDIR=/tmp && timeout -k 10 300 rocprofv3 --kernel-trace --stats "
             f"--output-format csv -d $R/gpurun_out/{tag}/kt_{w} -o kt -- python3 $R/bench.py "
             f"--workload {w} --also= --no-cpu-baseline",
             "# summary: python3 $R/bench.py --summarize-trace $R/gpurun_out/" + tag + f" --workload {w}",
             f"kernel_source_sha256_16: {kernel_source_hash()}",
             f"{'kernel':<72} {'calls':>6} {'avg_ns':>10} {'min_ns':>8} {'max_ns':>8}"]
    for row in csv.DictReader(open(files[0])):
        name = row["Name"]
        short = name if len(name) <= 72 else name[:69] + "..."
        lines.append(f"{short:<72} {row['Calls']:>6} {float(row['AverageNs']):>10.1f} "
                     f"{float(row['MinNs']):>8.0f} {float(row['MaxNs']):>8.0f}")
    if bench_log and os.path.exists(bench_log):
        for l in open(bench_log):
            if "] step" in l or ": step " in l:
                lines.append("# bench.py's own line in the traced run: " + l.strip())
    return "\n".join(lines) + "\n"


def workloads_names():
    import workloads

    return list(workloads.WORKLOADS)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="C3", choices=sorted(workloads_names()),
                    help="C1..C5: the decode configurations; P<rows>: the dynamic-sparse "
                         "prefill shape (rows x 2048 gathered candidates, MFMA-bound); "
                         "X<ctx>b<batch><dtype>: the PagedAttention page's isolated decode "
                         "shapes (64q/8kv, head 64, block 256)")
    ap.add_argument("--replica-bytes", type=float, default=1.0 * (1 << 30),
                    help="cold-cache protocol: replicate the cache until this many bytes")
    ap.add_argument("--rounds", type=int, default=7,
                    help="timed rounds of K steps; the median round is reported")
    ap.add_argument("--also", default="C5",
                    help="comma-separated further workloads timed the same way and reported "
                         "in the line's 'also' list ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="split-count override (0 = automatic)")
    ap.add_argument("--min-chunk", type=int, default=0, help="geometry min_chunk (0 = default)")
    ap.add_argument("--waves", type=int, default=0, help="geometry target waves (0 = default)")
    ap.add_argument("--kv-heads-per-cta", type=int, default=0,
                    help="geometry: KV heads per CTA (0 = default, 1, 4 or 8)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step eagerly instead of from a HIP graph (for "
                         "per-dispatch hardware counters)")
    ap.add_argument("--op", default="decode", choices=["decode", "write"],
                    help="decode: the decode step (default); write: the quantise-on-write "
                         "cache writer (reshape_and_cache) on the workload's cache format")
    ap.add_argument("--write-tokens", type=int, default=16384,
                    help="new tokens per writer call (--op write)")
    ap.add_argument("--summarize-counters", default="",
                    help="print the counter summary (profiles/) of the workload's attention kernel "
                         "from the rocprofv3 runs under this directory, and exit")
    ap.add_argument("--summarize-trace", default="",
                    help="print the kernel-trace summary of the workload's rocprofv3 "
                         "--kernel-trace --stats run under this directory, and exit")
    ap.add_argument("--trace-log", default="", help="bench.py log of the traced run (--summarize-trace)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 4 plain device-to-device copies of this many bytes and exit "
                         "(calibrates the HBM byte counters)")
    args = ap.parse_args()

    if args.summarize_counters:
        sys.stdout.write(summarize_counters(args.summarize_counters, args.workload))
        return 0
    if args.summarize_trace:
        sys.stdout.write(summarize_trace(args.summarize_trace, args.workload, args.trace_log))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library "
              "has no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
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

    line = decode_line(args, dev)
    print(json.dumps(line), flush=True)
    return 0


def _median(xs):
    ys = sorted(xs)
    return ys[len(ys) // 2]


def measure_decode(args, dev, workload: str, with_partials: bool = True) -> dict:
    """Time the decode step (split kernel + combine) and the split kernel alone
    on one workload with the cold-cache protocol:
      * R = ceil(replica_bytes / cache bytes) device replicas of the caches
        (independent of --steps), step i reads replica i mod R;
      * K steps captured in one HIP graph, W eager warmup steps and one
        untimed replay before timing;
      * every timed round is preceded by an untimed read of a 512 MiB buffer
        (twice the 256 MB Infinity Cache), so no round starts with the cache
        holding the replicas it reads first;
      * ms per step = median over --rounds rounds of (HIP events around one
        replay on the launch stream) / K."""
    import torch

    import quantized_paged_kv_amd as pkv
    import workloads
    from workloads.device import to_device

    log(f"generating {workload}")
    inp = workloads.workload(workload)
    p = inp.problem
    kv_bytes = inp.effective_kv_bytes()
    d = to_device(inp, dev)
    prob = pkv.make_problem(**d.problem_kwargs)
    geo = pkv.split_geometry(prob, splits_override=args.splits, min_chunk=args.min_chunk,
                             waves=args.waves, kv_heads_per_cta=args.kv_heads_per_cta)
    ws = pkv.workspace_for(geo, dev)

    # cold-cache replicas of the caches (the block table, lengths, Q, scales are shared)
    cache_bytes = d.key_cache.numel() * d.key_cache.element_size()
    if d.value_cache is not None:
        cache_bytes += d.value_cache.numel() * d.value_cache.element_size()
    R = max(1, math.ceil(args.replica_bytes / max(cache_bytes, 1)))
    log(f"{workload}: kv bytes/step {kv_bytes}, cache bytes {cache_bytes}, replicas {R} "
        f"({R * cache_bytes} bytes), splits {geo.num_splits}")
    keys = [d.key_cache] + [d.key_cache.clone() for _ in range(R - 1)]
    vals = [d.value_cache] + ([d.value_cache.clone() for _ in range(R - 1)]
                              if d.value_cache is not None else [None] * (R - 1))
    odt = torch.float32 if d.problem_kwargs["out_dtype"] == "f32" else torch.float16
    qrows = p.rows * max(1, p.query_tokens)  # query rows: rows x tokens per row
    out = torch.empty((qrows, p.heads, p.v_head_size), dtype=odt, device=dev)
    lse = torch.empty((qrows, p.heads), dtype=torch.float32, device=dev)
    # a read of 512 MiB (twice the Infinity Cache) before every timed round
    # evicts the replicas and leaves clean lines (a write would leave dirty
    # lines whose write-back the first timed steps would pay for)
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)

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
    g_part = capture(partial, K) if with_partials else None
    g_step.replay()  # untimed: first replay of the graph
    if g_part is not None:
        g_part.replay()
    torch.cuda.synchronize()

    def timed_rounds(g):
        per_step = []
        for _ in range(args.rounds):
            flush.max()  # untimed: evict the Infinity Cache
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()  # exactly K steps
            e1.record()
            torch.cuda.synchronize()
            per_step.append(e0.elapsed_time(e1) / K)
        return _median(per_step), per_step

    ms_step, rounds_step = timed_rounds(g_step)
    ms_split, rounds_split = timed_rounds(g_part) if g_part is not None else (None, [])
    kernel = ("latent_kernel" if p.layout == "latent" else
              "split_kvp_kernel" if geo.kv_heads_per_cta > 1 else "split_kernel")
    res = {"inp": inp, "geo": geo, "kv_bytes": kv_bytes, "R": R, "cache_bytes": cache_bytes,
           "ms_step": ms_step, "rounds_step": rounds_step, "ms_split": ms_split,
           "rounds_split": rounds_split, "kernel": kernel}
    msg = f"{workload}: step {ms_step * 1e3:.2f} us ({kv_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s)"
    if ms_split is not None:
        msg += (f", split kernel {ms_split * 1e3:.2f} us "
                f"({kv_bytes / (ms_split * 1e-3) / 1e9:.0f} GB/s)")
    log(msg + f" [median of {args.rounds} rounds of {K} steps]")
    del keys, vals, flush
    torch.cuda.empty_cache()
    return res


def decode_line(args, dev) -> dict:
    m = measure_decode(args, dev, args.workload)
    inp, geo, p = m["inp"], m["geo"], m["inp"].problem
    kv_bytes, ms_step, ms_split = m["kv_bytes"], m["ms_step"], m["ms_split"]
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes / (ms_split * 1e-3) / 1e9
    kernel = m["kernel"]
    traffic = read_traffic(kernel, args.workload)
    K = args.steps
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
            "kv_heads_per_cta": geo.kv_heads_per_cta,
            "cold_cache_replicas": m["R"],
            "cold_cache_replica_bytes": m["R"] * m["cache_bytes"],
            "timing": (f"median of {args.rounds} rounds; each round "
                       + ("K eager launches" if args.eager else "one HIP-graph replay of K steps")
                       + ", HIP events on the launch stream, after an untimed 512 MiB read "
                         "that evicts the Infinity Cache"),
            "us_per_step_rounds": [round(x * 1e3, 3) for x in m["rounds_step"]],
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
            "kernel_us_rounds": [round(x * 1e3, 3) for x in m["rounds_split"]],
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if args.workload.startswith("P"):
        # prefill shapes gather cache-resident rows many times over (every row
        # of a sequence attends its own candidates): the bytes that must come
        # from HBM are the unique rows, the rest is served by the caches, and
        # the kernel waits on its chain of dependent loads (candidate, block
        # id, row); reported as gathered bytes per second with the MFMA
        # utilisation beside it (QK^T and PV, 2 (D + VD) flops per head and
        # attended token; the 12 -> 16 head padding and the residual tile are
        # not counted)
        from workloads import live_token_counts
        dims = p.head_size + p.v_head_size
        flops = int(live_token_counts(inp).sum()) * p.heads * 2 * dims
        tflops = flops / (ms_split * 1e-3) / 1e12
        line["roofline"]["bound"] = "latency"
        line["roofline"]["note"] = ("gathered KV bytes per second; the bound is the chain of "
                                    "dependent loads per gathered row, not HBM bandwidth")
        line["roofline"]["mfma_tflops"] = round(tflops, 2)
        line["roofline"]["mfma_frac_of_fp16_peak"] = round(tflops / MFMA_F16_PEAK_TFLOPS, 4)
    also = [w for w in args.also.split(",") if w and w != args.workload]
    if also:
        line["also"] = []
        for w in also:
            a = measure_decode(args, dev, w)
            v = a["kv_bytes"] / (a["ms_step"] * 1e-3) / 1e9
            kv = a["kv_bytes"] / (a["ms_split"] * 1e-3) / 1e9
            line["also"].append({
                "workload": a["inp"].name, "us_per_step": round(a["ms_step"] * 1e3, 3),
                "value": round(v, 2), "unit": "GB/s",
                "pct_of_hbm_peak": round(100.0 * v / HBM_PEAK_GBS, 2),
                "kernel": a["kernel"], "kernel_us": round(a["ms_split"] * 1e3, 3),
                "kernel_frac_of_hbm_peak": round(kv / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(a["kernel"], w),
                "num_splits": a["geo"].num_splits, "cold_cache_replicas": a["R"]})
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores")
        line["cpu_baseline"] = cpu_baseline(inp)
    return line


if __name__ == "__main__":
    sys.exit(main())
