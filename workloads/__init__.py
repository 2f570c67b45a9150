"""Seeded synthetic inputs for paged-KV decode attention.

This module only draws inputs: shapes, random values, their storage codes,
block tables, lengths and candidate lists.  It computes no attention.  Both
the FP64 oracle (tests) and the GPU library (tests, bench) consume the arrays
it returns, so a parity test compares the two sides on byte-identical inputs.

Storage codes.  Caches are stored as codes the decode path reads:
  * ``f16``: IEEE binary16 values, stored as ``numpy.float16``;
  * ``i8``:  signed bytes, value = code * scale (symmetric, no zero point);
  * ``fp8``: OCP float8 e4m3fn bit patterns in ``numpy.uint8``,
             value = decode(code) * scale.
Quantised codes for the synthetic caches are drawn the way the workloads
describe them (``x ~ N(0, 1)``, ``s = max|x| / 127`` and ``code = rint(x / s)``
for INT8; ``s = max|x| / 448`` and a round-to-nearest-even cast for FP8).
That is how the synthetic cache contents are produced, not part of the
decode; both sides only ever see the resulting codes and scales.

Layout (one reading of the PagedAttention page, which does not fix it):
  key_cache   [num_pool_blocks, block_size, kv_heads, head_size]
  value_cache [num_pool_blocks, block_size, kv_heads, v_head_size]  (absent
              for the latent layout, where V is the first v_head_size
              channels of the K row)
  block_table [rows, max_blocks_per_row] int32, seq_lens [rows] int32,
  candidates  [rows, max_candidates] int32 (gathered rows only),
  k_scale / v_scale  [1] (per tensor) or [kv_heads, dim] (per channel) fp32,
  head_sink   [heads] fp32 (scaled-logit units) or None.

Pool blocks that no block table references are filled with poison (NaN for
FP16 and FP8 caches, 127 for INT8) so that a read outside the live range
shows up in the output.

Named workloads (draw order fixed: Q, K, V, scales, lengths, table
permutation, sink, candidates; the seed defaults to the workload number):
  C1  tiny FP16 decode: 1 row, 4 q / 1 kv head, head 64, context 256, block 16
  C2  INT8 per-tensor: 1 row, 24 q / 2 kv heads, head 256, context 4096
  C3  continuous batching FP16: 16 rows, lengths U{512..8192}, 32 q / 8 kv,
      head 128, block 16, shuffled table, per-head sink ~ N(0, 1)
  C4  INT8 per-channel dynamic-sparse: 8 rows of one sequence (context
      32768), 24 q / 2 kv, head 256, 2048 sorted candidates per row,
      per-channel scales ~ U(0.005, 0.05), codes clip(rint(N(0, 40^2)))
  C5  absorbed-MLA latent FP8 e4m3fn: 32 rows, context 4096, 16 q heads over
      one latent head of 576 channels, V = first 512, block 64
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

CACHE_DTYPES = ("f16", "i8", "fp8")
QUANTS = ("none", "tensor", "channel")
LAYOUTS = ("separate", "latent")


@dataclass(frozen=True)
class Problem:
    """Static shape and type description of one decode step."""

    rows: int
    heads: int
    kv_heads: int
    head_size: int
    v_head_size: int
    block_size: int
    max_blocks_per_row: int
    num_pool_blocks: int
    max_candidates: int = 0  # 0 = dense rows, > 0 = gathered candidate lists
    cache_dtype: str = "f16"
    k_quant: str = "none"
    v_quant: str = "none"
    layout: str = "separate"
    out_dtype: str = "f16"
    sliding_window: int = 0  # > 0: attend to the last sliding_window positions only
    softcap: float = 0.0     # > 0: logits x -> softcap * tanh(x / softcap)
    query_tokens: int = 1    # query tokens per row (several: causal within the row)

    @property
    def group(self) -> int:
        return self.heads // self.kv_heads

    @property
    def capacity(self) -> int:
        return self.max_blocks_per_row * self.block_size

    @property
    def cache_itemsize(self) -> int:
        return 2 if self.cache_dtype == "f16" else 1


@dataclass
class Inputs:
    problem: Problem
    query: np.ndarray  # float16 [rows, heads, head_size]
    key_cache: np.ndarray
    value_cache: Optional[np.ndarray]
    block_table: np.ndarray  # int32 [rows, max_blocks_per_row]
    seq_lens: np.ndarray  # int32 [rows]
    softmax_scale: float
    k_scale: Optional[np.ndarray] = None  # float32
    v_scale: Optional[np.ndarray] = None
    head_sink: Optional[np.ndarray] = None  # float32 [heads]
    candidates: Optional[np.ndarray] = None  # int32 [rows, max_candidates]
    num_candidates: Optional[np.ndarray] = None  # int32 [rows]
    name: str = ""
    meta: dict = field(default_factory=dict)

    def effective_kv_bytes(self) -> int:
        """Bytes of K and V rows the step must read: sum over rows and KV heads
        of |T_r| * (head_size + v_head_size) * itemsize; a latent row counts
        once.  |T_r| is the number of live tokens (dense) or valid candidates
        (gathered) of row r."""
        p = self.problem
        n = live_token_counts(self)
        if p.layout == "latent":
            row = p.head_size * p.cache_itemsize
        else:
            row = (p.head_size + p.v_head_size) * p.cache_itemsize
        return int(n.sum()) * p.kv_heads * row


def live_token_counts(inp: Inputs) -> np.ndarray:
    """Number of attended entries per row (list length after dropping invalid
    candidates; clamped context length for dense rows)."""
    p = inp.problem
    lens = np.clip(inp.seq_lens.astype(np.int64), 0, p.capacity)
    lo = np.maximum(lens - p.sliding_window, 0) if p.sliding_window > 0 else np.zeros_like(lens)
    if p.max_candidates == 0:
        return lens - lo
    out = np.zeros(p.rows, dtype=np.int64)
    for r in range(p.rows):
        nc = int(np.clip(inp.num_candidates[r], 0, p.max_candidates))
        c = inp.candidates[r, :nc].astype(np.int64)
        out[r] = int(((c >= lo[r]) & (c < lens[r])).sum())
    return out


# ----------------------------------------------------------------------------
# storage-code helpers (input generation only)
# ----------------------------------------------------------------------------

def quantize_i8_per_tensor(x: np.ndarray):
    s = np.float32(np.abs(x).max() / 127.0)
    codes = np.clip(np.rint(x / s), -127, 127).astype(np.int8)
    return codes, np.array([s], dtype=np.float32)


def quantize_i8_per_channel(x: np.ndarray, scale: np.ndarray):
    """x [..., kv_heads, dim]; scale [kv_heads, dim] (given)."""
    codes = np.clip(np.rint(x / scale), -127, 127).astype(np.int8)
    return codes


def fp8_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even cast to OCP e4m3fn, returned as bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def quantize_fp8_per_tensor(x: np.ndarray):
    s = np.float32(np.abs(x).max() / 448.0)
    return fp8_e4m3fn_codes(x / s), np.array([s], dtype=np.float32)


def poison_value(cache_dtype: str):
    if cache_dtype == "f16":
        return np.float16(np.nan)
    if cache_dtype == "fp8":
        return np.uint8(0x7F)  # e4m3fn NaN
    return np.int8(127)


def code_dtype(cache_dtype: str):
    return {"f16": np.float16, "i8": np.int8, "fp8": np.uint8}[cache_dtype]


# ----------------------------------------------------------------------------
# generic generator
# ----------------------------------------------------------------------------

def make_inputs(
    problem: Problem,
    seed: int,
    seq_lens=None,
    *,
    softmax_scale: Optional[float] = None,
    q_std: float = 1.0,
    with_sink: bool = False,
    candidates=None,
    num_candidates=None,
    per_channel_scale_range=(0.005, 0.05),
    code_std: Optional[float] = None,
    shared_table: bool = False,
    poison_blocks: Optional[int] = None,
    name: str = "",
) -> Inputs:
    """Draw one decode step.

    ``seq_lens``: int, sequence or None (= capacity for every row).
    ``candidates``: None (dense), or an int32 [rows, max_candidates] array.
    ``code_std``: draw INT8 codes directly as clip(rint(N(0, code_std^2)))
    (per-channel scales then drawn from ``per_channel_scale_range``) instead of
    quantising N(0, 1) values.
    ``shared_table``: all rows share one block table (rows are query tokens of
    one sequence).
    """
    p = problem
    rng = np.random.default_rng(seed)
    R, H, KVH, D, VD, B = p.rows, p.heads, p.kv_heads, p.head_size, p.v_head_size, p.block_size
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(D)
    if seq_lens is None:
        lens = np.full(R, p.capacity, dtype=np.int64)
    elif np.isscalar(seq_lens):
        lens = np.full(R, int(seq_lens), dtype=np.int64)
    else:
        lens = np.asarray(seq_lens, dtype=np.int64)
    # blocks each row needs (clamped to capacity); rows that share a table
    # need the longest row's blocks once.
    need = np.minimum((np.clip(lens, 0, None) + B - 1) // B, p.max_blocks_per_row)
    used = int(need.max()) if shared_table else int(need.sum())
    extra = poison_blocks if poison_blocks is not None else max(4, used // 16)
    pool = max(p.num_pool_blocks, used + extra)
    p = replace(p, num_pool_blocks=pool)

    # Q ([rows, T, heads, D] flattened to [rows * T, heads, D] with T query
    # tokens per row)
    T = max(1, p.query_tokens)
    query = (rng.standard_normal((R * T, H, D), dtype=np.float32) * q_std).astype(np.float16)

    # K, V (values or codes)
    kshape = (pool, B, KVH, D)
    vshape = (pool, B, KVH, VD)
    k_scale = v_scale = None
    if p.cache_dtype == "f16":
        key = rng.standard_normal(kshape, dtype=np.float32).astype(np.float16)
        val = None if p.layout == "latent" else rng.standard_normal(vshape, dtype=np.float32).astype(np.float16)
        if p.k_quant != "none" or p.v_quant != "none":
            raise ValueError("FP16 caches are generated unquantised")
    elif p.cache_dtype == "i8":
        if code_std is not None:
            key = np.clip(np.rint(rng.standard_normal(kshape, dtype=np.float32) * code_std), -127, 127).astype(np.int8)
            val = None
            if p.layout != "latent":
                val = np.clip(np.rint(rng.standard_normal(vshape, dtype=np.float32) * code_std), -127, 127).astype(np.int8)
            lo, hi = per_channel_scale_range
            k_scale = (rng.uniform(lo, hi, size=(KVH, D)).astype(np.float32)
                       if p.k_quant == "channel" else np.array([rng.uniform(lo, hi)], dtype=np.float32))
            if p.layout != "latent":
                v_scale = (rng.uniform(lo, hi, size=(KVH, VD)).astype(np.float32)
                           if p.v_quant == "channel" else np.array([rng.uniform(lo, hi)], dtype=np.float32))
        else:
            kx = rng.standard_normal(kshape, dtype=np.float32)
            vx = None if p.layout == "latent" else rng.standard_normal(vshape, dtype=np.float32)
            if p.k_quant == "tensor":
                key, k_scale = quantize_i8_per_tensor(kx)
            else:
                k_scale = (np.abs(kx).max(axis=(0, 1)) / 127.0).astype(np.float32)
                key = quantize_i8_per_channel(kx, k_scale)
            val = None
            if vx is not None:
                if p.v_quant == "tensor":
                    val, v_scale = quantize_i8_per_tensor(vx)
                else:
                    v_scale = (np.abs(vx).max(axis=(0, 1)) / 127.0).astype(np.float32)
                    val = quantize_i8_per_channel(vx, v_scale)
    elif p.cache_dtype == "fp8":
        kx = rng.standard_normal(kshape, dtype=np.float32)
        vx = None if p.layout == "latent" else rng.standard_normal(vshape, dtype=np.float32)
        if p.k_quant == "tensor":
            key, k_scale = quantize_fp8_per_tensor(kx)
        else:
            k_scale = (np.abs(kx).max(axis=(0, 1)) / 448.0).astype(np.float32)
            key = fp8_e4m3fn_codes(kx / k_scale)
        val = None
        if vx is not None:
            if p.v_quant == "tensor":
                val, v_scale = quantize_fp8_per_tensor(vx)
            else:
                v_scale = (np.abs(vx).max(axis=(0, 1)) / 448.0).astype(np.float32)
                val = fp8_e4m3fn_codes(vx / v_scale)
    else:
        raise ValueError(p.cache_dtype)

    # block tables: one random permutation of the pool; rows take consecutive
    # runs of it; the leftover blocks are poisoned.
    perm = rng.permutation(pool).astype(np.int32)
    table = np.full((R, p.max_blocks_per_row), -1, dtype=np.int32)
    if shared_table:
        n0 = int(need.max())
        row_tab = perm[:n0]
        for r in range(R):
            table[r, :n0] = row_tab
        taken = n0
    else:
        taken = 0
        for r in range(R):
            n = int(need[r])
            table[r, :n] = perm[taken:taken + n]
            taken += n
    unused = perm[taken:]
    pv = poison_value(p.cache_dtype)
    key[unused] = pv
    if val is not None:
        val[unused] = pv
    # entries past a row's live blocks point at a poisoned block, not -1, so a
    # read past the live range would return poison instead of faulting
    fill = int(unused[0]) if len(unused) else 0
    table[table < 0] = fill

    sink = rng.standard_normal(H).astype(np.float32) if with_sink else None

    cand = ncand = None
    if candidates is not None:
        cand = np.ascontiguousarray(candidates, dtype=np.int32)
        ncand = (np.full(R, cand.shape[1], dtype=np.int32) if num_candidates is None
                 else np.asarray(num_candidates, dtype=np.int32))

    return Inputs(problem=p, query=query, key_cache=key, value_cache=val, block_table=table,
                  seq_lens=lens.astype(np.int32), softmax_scale=float(softmax_scale),
                  k_scale=k_scale, v_scale=v_scale, head_sink=sink, candidates=cand,
                  num_candidates=ncand, name=name)


def expand_query_tokens(inp: Inputs) -> Inputs:
    """The same step with one query token per row: row r's T tokens become
    rows r * T + j, each with the row's block-table row and the length its
    token attends, max(0, len - (T - 1 - j)) with len clamped to capacity.
    Pure rearrangement of the inputs (no attention arithmetic)."""
    p = inp.problem
    T = max(1, p.query_tokens)
    if T == 1:
        return inp
    lens = np.clip(inp.seq_lens.astype(np.int64), 0, p.capacity)
    j = np.arange(T)
    tok_lens = np.maximum(0, lens[:, None] - (T - 1 - j)[None, :]).reshape(-1)
    return Inputs(problem=replace(p, rows=p.rows * T, query_tokens=1), query=inp.query,
                  key_cache=inp.key_cache, value_cache=inp.value_cache,
                  block_table=np.repeat(inp.block_table, T, axis=0),
                  seq_lens=tok_lens.astype(np.int32), softmax_scale=inp.softmax_scale,
                  k_scale=inp.k_scale, v_scale=inp.v_scale, head_sink=inp.head_sink,
                  name=(inp.name + ", as separate rows") if inp.name else "", meta=dict(inp.meta))


def sorted_subsets(rng: np.random.Generator, rows: int, universe: int, k: int) -> np.ndarray:
    """Per row, a sorted random subset of [0, universe) of size k."""
    out = np.empty((rows, k), dtype=np.int32)
    for r in range(rows):
        out[r] = np.sort(rng.choice(universe, size=k, replace=False)).astype(np.int32)
    return out


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

def c1(seed: int = 1) -> Inputs:
    p = Problem(rows=1, heads=4, kv_heads=1, head_size=64, v_head_size=64, block_size=16,
                max_blocks_per_row=16, num_pool_blocks=64, cache_dtype="f16")
    return make_inputs(p, seed, 256, softmax_scale=1.0 / 8.0, poison_blocks=48,
                       name="C1 tiny FP16 decode: 1 row, 4q/1kv, head 64, context 256, block 16")


def c2(seed: int = 2, batch: int = 1) -> Inputs:
    """C2; with ``batch`` > 1 the same shape for that many rows (each row its
    own context of 4096 tokens and shuffled blocks), the batch sweep that
    shows where the step stops being latency bound."""
    p = Problem(rows=batch, heads=24, kv_heads=2, head_size=256, v_head_size=256, block_size=16,
                max_blocks_per_row=256, num_pool_blocks=0, cache_dtype="i8",
                k_quant="tensor", v_quant="tensor")
    rows = "1 row" if batch == 1 else f"{batch} rows"
    return make_inputs(p, seed, 4096, softmax_scale=0.0625,
                       name=f"C2 INT8 per-tensor decode: {rows}, 24q/2kv, head 256, context 4096, block 16")


def c3(seed: int = 3) -> Inputs:
    rng = np.random.default_rng(seed + 1000)
    lens = rng.integers(512, 8192, size=16, endpoint=True)
    p = Problem(rows=16, heads=32, kv_heads=8, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=512, num_pool_blocks=0, cache_dtype="f16")
    return make_inputs(p, seed, lens, softmax_scale=1.0 / np.sqrt(128.0), with_sink=True,
                       name="C3 continuous batching FP16: 16 rows, lengths U[512,8192], 32q/8kv, head 128, block 16, head sink")


def c3_tokens(T: int, seed: int = 3) -> Inputs:
    """C3 with T query tokens per sequence (a speculative / multi-token decode
    step): the same 16 sequences, lengths (now counting the T new tokens),
    heads and cache; token j of a sequence attends len - T + 1 + j positions."""
    rng = np.random.default_rng(seed + 1000)
    lens = rng.integers(512, 8192, size=16, endpoint=True)
    p = Problem(rows=16, heads=32, kv_heads=8, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=512, num_pool_blocks=0, cache_dtype="f16", query_tokens=T)
    return make_inputs(p, seed, lens, softmax_scale=1.0 / np.sqrt(128.0), with_sink=True,
                       name=f"C3 with {T} query tokens per sequence: 16 sequences, lengths "
                            f"U[512,8192], 32q/8kv, head 128, block 16, head sink")


def c4(seed: int = 4, rows: int = 8) -> Inputs:
    rng = np.random.default_rng(seed + 1000)
    ctx, k = 32768, 2048
    cand = sorted_subsets(rng, rows, ctx, k)
    p = Problem(rows=rows, heads=24, kv_heads=2, head_size=256, v_head_size=256, block_size=16,
                max_blocks_per_row=ctx // 16, num_pool_blocks=0, max_candidates=k,
                cache_dtype="i8", k_quant="channel", v_quant="channel")
    return make_inputs(p, seed, ctx, softmax_scale=0.0625, q_std=1.4, candidates=cand,
                       code_std=40.0, shared_table=True,
                       name=f"C4 INT8 per-channel dynamic-sparse: {rows} row{'s' if rows > 1 else ''}, 24q/2kv, "
                            "head 256, context 32768, 2048 candidates")


def c5(seed: int = 5) -> Inputs:
    p = Problem(rows=32, heads=16, kv_heads=1, head_size=576, v_head_size=512, block_size=64,
                max_blocks_per_row=64, num_pool_blocks=0, cache_dtype="fp8", k_quant="tensor",
                v_quant="tensor", layout="latent")
    return make_inputs(p, seed, 4096, softmax_scale=1.0 / 24.0,
                       name="C5 absorbed-MLA latent FP8 e4m3fn: 32 rows, context 4096, 16q/1 latent head, 576/512, block 64")


def dsa_prefill(rows: int, ctx: int = 8192, seed: int = 6) -> Inputs:
    """The dynamic-sparse prefill shape: ``rows`` query rows of one sequence
    of ``ctx`` tokens, each attending its own 2048 sorted random candidates,
    with C4's head shapes, distributions and scales (24q/2kv, head 256, INT8
    per-channel, codes clip(rint(N(0, 40^2))), Q ~ N(0, 1.4^2), scale 1/16).
    Every row is evaluated whole (one split), so the work is the MFMA
    contractions over gathered, cache-resident rows."""
    rng = np.random.default_rng(seed + 1000)
    k = 2048
    cand = sorted_subsets(rng, rows, ctx, k)
    p = Problem(rows=rows, heads=24, kv_heads=2, head_size=256, v_head_size=256, block_size=16,
                max_blocks_per_row=ctx // 16, num_pool_blocks=0, max_candidates=k,
                cache_dtype="i8", k_quant="channel", v_quant="channel")
    return make_inputs(p, seed, ctx, softmax_scale=0.0625, q_std=1.4, candidates=cand,
                       code_std=40.0, shared_table=True,
                       name=f"DSA prefill INT8 per-channel: {rows} rows, 24q/2kv, head 256, "
                            f"context {ctx}, 2048 candidates per row")


def paged_quantized(ctx: int, batch: int, cache_dtype: str, seed: int = 7) -> Inputs:
    """The PagedAttention page's isolated paged-decode shape: ``batch`` rows
    of ``ctx`` tokens, 64 query / 8 KV heads, head size 64, block 256, INT8
    or FP8 per-tensor cache from N(0, 1) values (s = max|x| / 127 or / 448),
    Q ~ N(0, 1), scale 1/8, shuffled blocks."""
    p = Problem(rows=batch, heads=64, kv_heads=8, head_size=64, v_head_size=64, block_size=256,
                max_blocks_per_row=ctx // 256, num_pool_blocks=0, cache_dtype=cache_dtype,
                k_quant="tensor", v_quant="tensor")
    return make_inputs(p, seed, ctx, softmax_scale=0.125,
                       name=f"paged {cache_dtype} per-tensor decode: {batch} rows x {ctx} tokens, "
                            f"64q/8kv, head 64, block 256")


WORKLOADS = {"C1": c1, "C2": c2, "C3": c3, "C4": c4, "C5": c5,
             **{f"C2b{b}": (lambda seed=2, b=b: c2(seed, b)) for b in (8, 32, 64)},
             **{f"X{c}b{b}{d}": (lambda seed=7, c=c, b=b, d=d: paged_quantized(c, b, d, seed))
                for c, b in ((1024, 32), (4096, 8), (4096, 32), (16384, 8), (16384, 32))
                for d in ("i8", "fp8")},
             "C4r1": lambda seed=4: c4(seed, rows=1),
             "C3t4": lambda seed=3: c3_tokens(4, seed),
             "C3t4rows": lambda seed=3: expand_query_tokens(c3_tokens(4, seed)),
             "C3t8": lambda seed=3: c3_tokens(8, seed),
             "C3t8rows": lambda seed=3: expand_query_tokens(c3_tokens(8, seed)),
             "P128": lambda seed=6: dsa_prefill(128, seed=seed),
             "P2048": lambda seed=6: dsa_prefill(2048, seed=seed),
             "P8192": lambda seed=6: dsa_prefill(8192, seed=seed)}


def workload(name: str, seed: Optional[int] = None) -> Inputs:
    f = WORKLOADS[name]
    return f() if seed is None else f(seed)


# ----------------------------------------------------------------------------
# new rows for the quantise-on-write cache writer
# ----------------------------------------------------------------------------

@dataclass
class NewTokens:
    """Fresh K/V rows, their slots and the scales to quantise them with."""
    key: np.ndarray                      # float16 [T, kv_heads, head_size]
    value: Optional[np.ndarray]          # float16 [T, kv_heads, v_head_size] or None
    slot_mapping: np.ndarray             # int64 [T]
    k_scale: Optional[np.ndarray]        # float32 [1] or [kv_heads, head_size]
    v_scale: Optional[np.ndarray]


def _writer_scale(rng, quant, kv_heads, dim, code_max, x_std):
    """Scales that put about 4 standard deviations at the top code, so a few
    values saturate; per channel they vary by a factor of 4."""
    if quant == "none":
        return None
    base = 4.0 * x_std / code_max
    if quant == "tensor":
        return np.array([base * rng.uniform(0.7, 1.4)], dtype=np.float32)
    return (base * rng.uniform(0.5, 2.0, size=(kv_heads, dim))).astype(np.float32)


def new_tokens(problem: Problem, num_tokens: int, seed: int, *, x_std: float = 1.0,
               skip_fraction: float = 0.1, slots=None) -> NewTokens:
    """Draw ``num_tokens`` new rows ~ N(0, x_std^2) as float16 (a tenth of
    them ten times larger, to reach saturation), per-tensor or per-channel
    scales, and a slot mapping: distinct random slots of the pool, with
    ``skip_fraction`` of the tokens given -1 or a slot past the pool (the
    writer skips those).  ``slots`` replaces the drawn mapping."""
    p = problem
    rng = np.random.default_rng(seed)
    T, KVH = int(num_tokens), p.kv_heads
    latent = p.layout == "latent"

    def rows(dim):
        x = rng.standard_normal((T, KVH, dim), dtype=np.float32) * x_std
        big = rng.random((T, KVH, dim)) < 0.1
        return np.where(big, x * 10.0, x).astype(np.float16)

    key = rows(p.head_size)
    value = None if latent else rows(p.v_head_size)
    code_max = {"f16": 1.0, "i8": 127.0, "fp8": 448.0}[p.cache_dtype]
    k_scale = _writer_scale(rng, p.k_quant, KVH, p.head_size, code_max, x_std)
    v_scale = None if latent else _writer_scale(rng, p.v_quant, KVH, p.v_head_size, code_max, x_std)
    n_slots = p.num_pool_blocks * p.block_size
    if slots is None:
        if T > n_slots:
            raise ValueError("more new tokens than pool slots")
        slot_mapping = rng.choice(n_slots, size=T, replace=False).astype(np.int64)
        skip = rng.random(T) < skip_fraction
        past = rng.integers(n_slots, 2 * n_slots, size=T)
        slot_mapping = np.where(skip, np.where(rng.random(T) < 0.5, -1, past), slot_mapping)
    else:
        slot_mapping = np.asarray(slots, dtype=np.int64)
    return NewTokens(key=key, value=value, slot_mapping=slot_mapping.astype(np.int64),
                     k_scale=k_scale, v_scale=v_scale)


def every_fp16_value() -> np.ndarray:
    """All binary16 values except NaN (both zeros and both infinities
    included), in bit-pattern order."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[~np.isnan(v)]
