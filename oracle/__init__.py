"""FP64 CPU oracle for paged-KV decode attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links
or calls it, and it imports nothing of the GPU library.

The arithmetic lives in ``pkv_oracle.c`` (plain C, FP64, plain loops); this
module only marshals numpy arrays into it.  ``build()`` compiles the C file
with gcc into ``liboracle.so`` next to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_CODE = {"f16": 0, "i8": 1, "fp8": 2}
QUANT_CODE = {"none": 0, "tensor": 1, "channel": 2}


def build(verbose: bool = False) -> str:
    """Compile the oracle (gcc -O2, no fast-math) into oracle/liboracle.so."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", _SRC, "-o",
           _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_fp8e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_fp8e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_code.restype = ctypes.c_double
    lib.oracle_decode_code.argtypes = [ctypes.c_int, ctypes.c_uint32]
    lib.oracle_dequant.restype = ctypes.c_double
    lib.oracle_dequant.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_float]
    lib.oracle_paged_decode.restype = ctypes.c_int
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_paged_decode.argtypes = ([I] * 13 + [P] * 9 + [ctypes.c_double, P, ctypes.c_double]
                                        + [I, I, I, P, I, P, P])
    _lib = lib
    return lib


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(bits)


def fp8e4m3_to_f64(bits: int) -> float:
    return _load().oracle_fp8e4m3_to_f64(bits)


def dequant(cache_dtype: str, code: int, scale: float) -> float:
    return _load().oracle_dequant(DTYPE_CODE[cache_dtype], code & 0xFFFFFFFF, scale)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def paged_decode(inp, chunk: int = 0, threads: int | None = None, rows=None):
    """Evaluate one decode step in FP64.

    ``inp``: a ``workloads.Inputs``.  ``chunk`` > 0 evaluates the split variant
    (partials over consecutive chunks of each row's token list, merged in
    FP64).  ``rows``: optional list of rows to evaluate (the others are left
    as NaN).  Returns ``(out [rows, heads, v_head_size], lse [rows, heads])``
    as float64 arrays.
    """
    lib = _load()
    p = inp.problem
    if threads is None:
        threads = os.cpu_count() or 1
    q = np.ascontiguousarray(inp.query).view(np.uint16)
    kc = np.ascontiguousarray(inp.key_cache)
    vc = None if p.layout == "latent" else np.ascontiguousarray(inp.value_cache)
    bt = np.ascontiguousarray(inp.block_table, dtype=np.int32)
    sl = np.ascontiguousarray(inp.seq_lens, dtype=np.int32)
    cand = None if p.max_candidates == 0 else np.ascontiguousarray(inp.candidates, dtype=np.int32)
    ncand = None if p.max_candidates == 0 else np.ascontiguousarray(inp.num_candidates, dtype=np.int32)
    ks = None if inp.k_scale is None else np.ascontiguousarray(inp.k_scale, dtype=np.float32)
    vs = None if inp.v_scale is None else np.ascontiguousarray(inp.v_scale, dtype=np.float32)
    sink = None if inp.head_sink is None else np.ascontiguousarray(inp.head_sink, dtype=np.float32)
    out = np.full((p.rows, p.heads, p.v_head_size), np.nan, dtype=np.float64)
    lse = np.full((p.rows, p.heads), np.nan, dtype=np.float64)
    sub = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    rc = lib.oracle_paged_decode(
        p.rows, p.heads, p.kv_heads, p.head_size, p.v_head_size, p.block_size,
        p.max_blocks_per_row, p.num_pool_blocks, p.max_candidates, DTYPE_CODE[p.cache_dtype],
        QUANT_CODE[p.k_quant], QUANT_CODE[p.v_quant], 1 if p.layout == "latent" else 0,
        _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(sl), _ptr(cand), _ptr(ncand), _ptr(ks),
        _ptr(vs), float(inp.softmax_scale), _ptr(sink), float(p.softcap), int(p.sliding_window),
        int(chunk), int(threads), _ptr(sub),
        0 if sub is None else len(sub), _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"oracle_paged_decode failed with code {rc}")
    return out, lse
