"""Copy a ``workloads.Inputs`` to device tensors (torch) for the GPU library.

Pure data movement: byte-identical copies of the arrays the oracle reads.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class DeviceInputs:
    problem_kwargs: dict
    query: "object"
    key_cache: "object"
    value_cache: Optional[object]
    block_table: "object"
    seq_lens: "object"
    candidates: Optional[object]
    num_candidates: Optional[object]
    k_scale: Optional[object]
    v_scale: Optional[object]
    head_sink: Optional[object]
    softmax_scale: float


def problem_kwargs(p, out_dtype: Optional[str] = None) -> dict:
    return dict(num_rows=p.rows, num_heads=p.heads, num_kv_heads=p.kv_heads,
                head_size=p.head_size, v_head_size=p.v_head_size, block_size=p.block_size,
                max_blocks_per_row=p.max_blocks_per_row, num_pool_blocks=p.num_pool_blocks,
                max_candidates=p.max_candidates, cache_dtype=p.cache_dtype,
                out_dtype=out_dtype or p.out_dtype, k_quant=p.k_quant,
                v_quant="none" if p.layout == "latent" else p.v_quant, layout=p.layout,
                sliding_window=p.sliding_window, softcap=p.softcap,
                query_tokens=p.query_tokens)


def _t(a, device):
    import torch

    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.float16)
    return torch.from_numpy(a).to(device)


def to_device(inp, device="cuda", out_dtype: Optional[str] = None) -> DeviceInputs:
    p = inp.problem
    return DeviceInputs(
        problem_kwargs=problem_kwargs(p, out_dtype),
        query=_t(inp.query, device),
        key_cache=_t(inp.key_cache, device),
        value_cache=None if p.layout == "latent" else _t(inp.value_cache, device),
        block_table=_t(inp.block_table.astype(np.int32), device),
        seq_lens=_t(inp.seq_lens.astype(np.int32), device),
        candidates=None if p.max_candidates == 0 else _t(inp.candidates.astype(np.int32), device),
        num_candidates=None if p.max_candidates == 0 else _t(inp.num_candidates.astype(np.int32), device),
        k_scale=_t(inp.k_scale, device),
        v_scale=None if p.layout == "latent" else _t(inp.v_scale, device),
        head_sink=_t(inp.head_sink, device),
        softmax_scale=inp.softmax_scale,
    )
