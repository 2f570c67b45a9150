"""Quantise-on-write reference for the paged KV cache -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module; the GPU library never calls it.

Source: ONNX Runtime PR #29912 (PagedAttention), "Summary of Changes": the
``slot_mapping`` input gives each new token's cache slot explicitly, and
ReshapeAndCache quantises the new K/V rows on write with ``k_scale`` /
``v_scale`` at PER_TENSOR or PER_CHANNEL granularity, the inverse of the
dequantisation every read path applies.

What it computes (plain numpy, one token and element at a time in meaning):
  for token t with slot = slot_mapping[t] inside [0, num_pool_blocks *
  block_size), KV head g and channel d:
      v    = float32(x[t, g, d]) / float32(scale[g, d])      (IEEE division)
      code = INT8: clip(round-half-even(v), -128, 127)
             FP8 e4m3fn: the finite e4m3fn value nearest to v, ties to the
                 even code (so |v| beyond 448 saturates to 448)
             FP16: v rounded to binary16 (round-half-even)
  written to cache[slot // block_size, slot % block_size, g, d]; tokens with
  a slot outside the pool are skipped.  LATENT caches hold one row per token
  (no value cache).  scale = 1 without quantisation.

Readings (the page does not spell them out): the quotient is formed in FP32
(the precision of the scales), ties round to even, INT8 codes use the full
[-128, 127] range, FP8 saturates instead of producing NaN.
"""
from __future__ import annotations

import numpy as np


def _fp8_table():
    """The 127 finite non-negative e4m3fn values with their codes, from the
    bit-field definition (bias 7; exponent 0 is subnormal; S.1111.111 is
    NaN)."""
    codes = np.arange(0, 127, dtype=np.int64)  # 0x7F is NaN
    e = codes >> 3
    m = codes & 7
    vals = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    return codes, vals


_FP8_CODES, _FP8_VALS = _fp8_table()


def fp8_e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3fn code to each float (ties to the even code).

    The finite values are sorted by code, so the two candidates of |v| are
    the table entries around its insertion point."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v).reshape(-1)
    hi = np.clip(np.searchsorted(_FP8_VALS, a), 1, len(_FP8_VALS) - 1)
    lo = hi - 1
    d_lo = a - _FP8_VALS[lo]
    d_hi = _FP8_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_FP8_CODES[hi] % 2 == 0))
    out = np.where(pick_hi, _FP8_CODES[hi], _FP8_CODES[lo]).astype(np.uint8)
    out[a >= _FP8_VALS[-1]] = _FP8_CODES[-1]  # beyond the largest finite value
    sign = np.signbit(v).reshape(-1).astype(np.uint8) << 7  # the sign survives rounding to zero
    return (out | sign).reshape(v.shape)


def int8_encode(v: np.ndarray) -> np.ndarray:
    return np.clip(np.rint(np.asarray(v, dtype=np.float32)), -128, 127).astype(np.int8)


def quantize(x_f16: np.ndarray, scale: np.ndarray, cache_dtype: str) -> np.ndarray:
    """Codes of x (float16, [..., dim]) under scale (broadcast over x)."""
    v = x_f16.astype(np.float32) / np.asarray(scale, dtype=np.float32)
    if cache_dtype == "i8":
        return int8_encode(v)
    if cache_dtype == "fp8":
        return fp8_e4m3fn_encode(v)
    return v.astype(np.float16)


def _scale_for(scale, quant, kv_heads, dim):
    if quant == "none" or scale is None:
        return np.ones((kv_heads, dim), dtype=np.float32)
    s = np.asarray(scale, dtype=np.float32)
    if quant == "tensor":
        return np.full((kv_heads, dim), s.reshape(-1)[0], dtype=np.float32)
    return s.reshape(kv_heads, dim)


def reshape_and_cache(problem, key, value, slot_mapping, k_scale, v_scale, key_cache, value_cache):
    """Write the new tokens into copies of the caches and return them.

    key: float16 [T, kv_heads, head_size]; value: float16 [T, kv_heads,
    v_head_size] or None (latent); slot_mapping: int64 [T]; caches in the
    storage layout of workloads (codes)."""
    p = problem
    kc = key_cache.copy()
    vc = None if value_cache is None else value_cache.copy()
    ks = _scale_for(k_scale, p.k_quant, p.kv_heads, p.head_size)
    vs = _scale_for(v_scale, p.v_quant, p.kv_heads, p.v_head_size)
    n_slots = kc.shape[0] * p.block_size
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0 or slot >= n_slots:
            continue
        b, o = divmod(slot, p.block_size)
        for g in range(p.kv_heads):
            kc[b, o, g] = quantize(key[t, g], ks[g], p.cache_dtype)
            if vc is not None:
                vc[b, o, g] = quantize(value[t, g], vs[g], p.cache_dtype)
    return kc, vc
