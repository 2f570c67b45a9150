"""Helpers for the GPU tests: run the HIP library through its C ABI on a
``workloads.Inputs`` and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

# Spec tolerance on unit-variance V: max abs error and mean abs error.
MAX_ABS = 2e-3
MEAN_ABS = 2e-4
# log-sum-exp (natural-log units)
LSE_ABS = 2e-3


def announce(msg: str):
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(inp, out_dtype=None, geometry=None, partials_then_combine=False, **geo):
    """One decode step on cuda:0; returns (out float64, lse float64, geometry)."""
    import torch

    import quantized_paged_kv_amd as pkv
    from workloads.device import to_device

    d = to_device(inp, "cuda", out_dtype)
    prob = pkv.make_problem(**d.problem_kwargs)
    g = geometry if geometry is not None else pkv.split_geometry(prob, **geo)
    ws = pkv.workspace_for(g)
    p = inp.problem
    qrows = p.rows * max(1, p.query_tokens)  # query rows: rows x query tokens per row
    odt = torch.float32 if d.problem_kwargs["out_dtype"] == "f32" else torch.float16
    out = torch.full((qrows, p.heads, p.v_head_size), float("nan"), dtype=odt, device="cuda")
    lse = torch.full((qrows, p.heads), float("nan"), dtype=torch.float32, device="cuda")
    if partials_then_combine:
        pkv.paged_decode_partials(prob, g, d.query, d.key_cache, d.value_cache, d.block_table,
                                  d.seq_lens, d.candidates, d.num_candidates, d.k_scale,
                                  d.v_scale, d.softmax_scale, ws)
        pkv.split_combine(prob, g, ws, d.head_sink, out, lse)
    else:
        pkv.paged_decode_attention(prob, g, d.query, d.key_cache, d.value_cache, d.block_table,
                                   d.seq_lens, d.candidates, d.num_candidates, d.k_scale,
                                   d.v_scale, d.softmax_scale, d.head_sink, out, lse, ws)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), g


def assert_close_to_oracle(got, lse, ref, ref_lse, max_abs=MAX_ABS, mean_abs=MEAN_ABS, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if np.array_equal(got, got.astype(np.float16).astype(np.float64)):
        # An FP16 output cannot come closer to the exact result than rounding
        # it to FP16: where every output is one unit-variance value (a window
        # of one position, one-token rows) that rounding alone averages about
        # 2e-4, so the mean bound is at least 1.1 times its mean.
        floor = float(np.abs(ref.astype(np.float16).astype(np.float64) - ref).mean())
        mean_abs = max(mean_abs, 1.1 * floor)
    err = np.abs(got - ref)
    assert err.max() <= max_abs, f"{what}: max abs error {err.max():.3e} > {max_abs:.1e}"
    assert err.mean() <= mean_abs, f"{what}: mean abs error {err.mean():.3e} > {mean_abs:.1e}"
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    fin = ~empty
    if fin.any():
        # Folding the key scale into the query (Q' = fp16(Q * k_scale), as the
        # INT8 DSA page does) moves each logit by at most 2^-11 of
        # scale * sum_d |Q'_d K_d|, a few 1e-4 nats on unit-variance data; the
        # log-sum-exp moves by at most the largest logit shift.
        lerr = np.abs(lse[fin] - ref_lse[fin])
        tol = LSE_ABS + 1e-5 * np.abs(ref_lse[fin])
        assert np.all(lerr <= tol), f"{what}: lse error {lerr.max():.3e}"
    return float(err.max()), float(err.mean())
