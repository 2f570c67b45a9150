"""Python binding of libpkv (split-KV paged decode attention for MI355X).

Argument marshalling only: every step of the decode runs in the HIP kernels of
``libpkv.so`` (built in-tree by ``python -m quantized_paged_kv_amd.build``).
PyTorch provides device memory and the stream.  If the library is missing the
import of any entry point raises; there is no fallback.

Entry points (same names as the C ABI in include/pkv.h):
  split_geometry(problem, ...)                -> Geometry
  paged_decode_attention(problem, geometry, ...)
  paged_decode_attention_noalloc(problem, geometry, ...)
  paged_decode_partials(problem, geometry, ...)
  split_combine(problem, geometry, ...)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

DTYPES = {"f16": 0, "i8": 1, "fp8": 2, "f32": 3}
QUANTS = {"none": 0, "tensor": 1, "channel": 2}
LAYOUTS = {"separate": 0, "latent": 1}
STATUS = {0: "PKV_OK", 1: "PKV_EINVAL", 2: "PKV_EUNSUPPORTED", 3: "PKV_EALIGN",
          4: "PKV_EWORKSPACE", 5: "PKV_EHIP"}


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_rows", "num_heads", "num_kv_heads", "head_size", "v_head_size", "block_size",
        "max_blocks_per_row", "num_pool_blocks", "max_candidates", "cache_dtype", "out_dtype",
        "k_quant", "v_quant", "layout", "sliding_window")] + [("softcap", ctypes.c_float),
                                                              ("query_tokens", ctypes.c_int32)]


class GeometryOpts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_cus", "ctas_per_cu", "splits_override", "min_chunk", "max_splits", "waves",
        "balance", "kv_heads_per_cta")]


class Geometry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_splits", "min_chunk", "threads", "head_blocks", "grid_x", "grid_y", "grid_z",
        "target_ctas", "kv_heads_per_cta")] + [("workspace_bytes", ctypes.c_uint64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None

SYMBOLS = ("split_geometry", "paged_decode_attention", "paged_decode_partials", "split_combine",
           "paged_decode_attention_noalloc", "reshape_and_cache", "pkv_status_string",
           "pkv_last_error")

# bytes of partials the allocation-free entry point holds per device
NOALLOC_WORKSPACE_BYTES = 64 << 20


def load():
    """Load libpkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m quantized_paged_kv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.split_geometry.restype = ctypes.c_int
    lib.split_geometry.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(GeometryOpts),
                                   ctypes.POINTER(Geometry)]
    lib.paged_decode_attention.restype = ctypes.c_int
    lib.paged_decode_attention.argtypes = ([ctypes.POINTER(Problem), ctypes.POINTER(Geometry)]
                                           + [P] * 9 + [ctypes.c_float] + [P] * 4
                                           + [ctypes.c_size_t, P])
    lib.paged_decode_partials.restype = ctypes.c_int
    lib.paged_decode_partials.argtypes = ([ctypes.POINTER(Problem), ctypes.POINTER(Geometry)]
                                          + [P] * 9 + [ctypes.c_float, P, ctypes.c_size_t, P])
    lib.paged_decode_attention_noalloc.restype = ctypes.c_int
    lib.paged_decode_attention_noalloc.argtypes = ([ctypes.POINTER(Problem),
                                                    ctypes.POINTER(Geometry)]
                                                   + [P] * 9 + [ctypes.c_float] + [P] * 4)
    lib.split_combine.restype = ctypes.c_int
    lib.split_combine.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Geometry), P,
                                  ctypes.c_size_t, P, P, P, P]
    lib.reshape_and_cache.restype = ctypes.c_int
    lib.reshape_and_cache.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32] + [P] * 8
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise PkvError(status, load().pkv_last_error().decode())


def make_problem(num_rows, num_heads, num_kv_heads, head_size, v_head_size, block_size,
                 max_blocks_per_row, num_pool_blocks, max_candidates=0, cache_dtype="f16",
                 out_dtype="f16", k_quant="none", v_quant="none", layout="separate",
                 sliding_window=0, softcap=0.0, query_tokens=1) -> Problem:
    def code(table, v):
        return table[v] if isinstance(v, str) else int(v)

    return Problem(int(num_rows), int(num_heads), int(num_kv_heads), int(head_size),
                   int(v_head_size), int(block_size), int(max_blocks_per_row),
                   int(num_pool_blocks), int(max_candidates), code(DTYPES, cache_dtype),
                   code(DTYPES, out_dtype), code(QUANTS, k_quant), code(QUANTS, v_quant),
                   code(LAYOUTS, layout), int(sliding_window), float(softcap),
                   int(query_tokens))


def split_geometry(problem: Problem, num_cus=0, ctas_per_cu=0, splits_override=0, min_chunk=0,
                   max_splits=0, waves=0, balance=0, kv_heads_per_cta=0) -> Geometry:
    opts = GeometryOpts(int(num_cus), int(ctas_per_cu), int(splits_override), int(min_chunk),
                        int(max_splits), int(waves), int(balance), int(kv_heads_per_cta))
    g = Geometry()
    _check(load().split_geometry(ctypes.byref(problem), ctypes.byref(opts), ctypes.byref(g)))
    return g


_ITEMSIZE = {0: 2, 1: 1, 2: 1, 3: 4}  # pkv_dtype -> bytes


def _require(t, nbytes, name):
    """A tensor argument must be device memory holding at least nbytes (the
    C ABI takes raw pointers and cannot check their extent).  Integers are
    raw device addresses and are passed through unchecked."""
    if t is None or isinstance(t, int):
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes; the problem needs {nbytes}")


def _check_extents(p: Problem, query=None, key_cache=None, value_cache=None, block_table=None,
                   seq_lens=None, candidates=None, num_candidates=None, k_scale=None,
                   v_scale=None, head_sink=None, out=None, lse_out=None):
    """Sizes every tensor argument must have for `p` (see include/pkv.h)."""
    qrows = p.num_rows * max(1, p.query_tokens)
    cb = _ITEMSIZE.get(p.cache_dtype, 1)
    slots = p.num_pool_blocks * p.block_size * p.num_kv_heads
    _require(query, qrows * p.num_heads * p.head_size * 2, "query")
    _require(key_cache, slots * p.head_size * cb, "key_cache")
    _require(value_cache, slots * p.v_head_size * cb, "value_cache")
    _require(block_table, p.num_rows * p.max_blocks_per_row * 4, "block_table")
    _require(seq_lens, p.num_rows * 4, "seq_lens")
    _require(candidates, p.num_rows * p.max_candidates * 4, "candidates")
    _require(num_candidates, p.num_rows * 4, "num_candidates")
    _require(k_scale, 4 * (p.num_kv_heads * p.head_size if p.k_quant == 2 else 1), "k_scale")
    _require(v_scale, 4 * (p.num_kv_heads * p.v_head_size if p.v_quant == 2 else 1), "v_scale")
    _require(head_sink, 4 * p.num_heads, "head_sink")
    _require(out, qrows * p.num_heads * p.v_head_size * _ITEMSIZE.get(p.out_dtype, 2), "out")
    _require(lse_out, qrows * p.num_heads * 4, "lse_out")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def paged_decode_attention(problem: Problem, geometry: Geometry, query, key_cache, value_cache,
                           block_table, seq_lens, candidates, num_candidates, k_scale, v_scale,
                           softmax_scale: float, head_sink, out, lse_out, workspace,
                           workspace_bytes=None, stream=None):
    """One decode step (split kernel + combine) on `stream` (default: torch's
    current stream).  Tensors are passed by device pointer; None = NULL."""
    _check_extents(problem, query, key_cache, value_cache, block_table, seq_lens, candidates,
                   num_candidates, k_scale, v_scale, head_sink, out, lse_out)
    _require(workspace, int(geometry.workspace_bytes), "workspace")
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().paged_decode_attention(
        ctypes.byref(problem), ctypes.byref(geometry), _ptr(query), _ptr(key_cache),
        _ptr(value_cache), _ptr(block_table), _ptr(seq_lens), _ptr(candidates),
        _ptr(num_candidates), _ptr(k_scale), _ptr(v_scale), float(softmax_scale),
        _ptr(head_sink), _ptr(out), _ptr(lse_out), _ptr(workspace), int(wb), _stream(stream)))


def paged_decode_attention_noalloc(problem: Problem, geometry: Geometry, query, key_cache,
                                   value_cache, block_table, seq_lens, candidates,
                                   num_candidates, k_scale, v_scale, softmax_scale: float,
                                   head_sink, out, lse_out, stream=None):
    """paged_decode_attention without a workspace argument: the partials go
    to the library's per-device array (NOALLOC_WORKSPACE_BYTES); calls that
    overlap on one GPU race."""
    _check_extents(problem, query, key_cache, value_cache, block_table, seq_lens, candidates,
                   num_candidates, k_scale, v_scale, head_sink, out, lse_out)
    _check(load().paged_decode_attention_noalloc(
        ctypes.byref(problem), ctypes.byref(geometry), _ptr(query), _ptr(key_cache),
        _ptr(value_cache), _ptr(block_table), _ptr(seq_lens), _ptr(candidates),
        _ptr(num_candidates), _ptr(k_scale), _ptr(v_scale), float(softmax_scale),
        _ptr(head_sink), _ptr(out), _ptr(lse_out), _stream(stream)))


def paged_decode_partials(problem: Problem, geometry: Geometry, query, key_cache, value_cache,
                          block_table, seq_lens, candidates, num_candidates, k_scale, v_scale,
                          softmax_scale: float, workspace, workspace_bytes=None, stream=None):
    """The split kernel alone: per-split partials into `workspace`."""
    _check_extents(problem, query, key_cache, value_cache, block_table, seq_lens, candidates,
                   num_candidates, k_scale, v_scale)
    _require(workspace, int(geometry.workspace_bytes), "workspace")
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().paged_decode_partials(
        ctypes.byref(problem), ctypes.byref(geometry), _ptr(query), _ptr(key_cache),
        _ptr(value_cache), _ptr(block_table), _ptr(seq_lens), _ptr(candidates),
        _ptr(num_candidates), _ptr(k_scale), _ptr(v_scale), float(softmax_scale),
        _ptr(workspace), int(wb), _stream(stream)))


def split_combine(problem: Problem, geometry: Geometry, workspace, head_sink, out, lse_out,
                  workspace_bytes=None, stream=None):
    """Merge the partials in `workspace` into `out` (and `lse_out`)."""
    _check_extents(problem, head_sink=head_sink, out=out, lse_out=lse_out)
    _require(workspace, int(geometry.workspace_bytes), "workspace")
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check(load().split_combine(ctypes.byref(problem), ctypes.byref(geometry), _ptr(workspace),
                                int(wb), _ptr(head_sink), _ptr(out), _ptr(lse_out),
                                _stream(stream)))


def reshape_and_cache(problem: Problem, key, value, slot_mapping, k_scale, v_scale, key_cache,
                      value_cache, num_tokens=None, stream=None):
    """Quantise the new rows `key` / `value` ([T, kv_heads, dim] float16) into
    the caches at the slots `slot_mapping` (int64 [T]) names; slots outside
    the pool are skipped.  LATENT: `value` and `value_cache` are None."""
    t = int(key.shape[0]) if num_tokens is None else int(num_tokens)
    cb = _ITEMSIZE.get(problem.cache_dtype, 1)
    slots = problem.num_pool_blocks * problem.block_size * problem.num_kv_heads
    kvh = problem.num_kv_heads
    _require(key, t * kvh * problem.head_size * 2, "key")
    _require(value, t * kvh * problem.v_head_size * 2, "value")
    _require(slot_mapping, t * 8, "slot_mapping")
    _require(k_scale, 4 * (kvh * problem.head_size if problem.k_quant == 2 else 1), "k_scale")
    _require(v_scale, 4 * (kvh * problem.v_head_size if problem.v_quant == 2 else 1), "v_scale")
    _require(key_cache, slots * problem.head_size * cb, "key_cache")
    _require(value_cache, slots * problem.v_head_size * cb, "value_cache")
    _check(load().reshape_and_cache(ctypes.byref(problem), t, _ptr(key), _ptr(value),
                                    _ptr(slot_mapping), _ptr(k_scale), _ptr(v_scale),
                                    _ptr(key_cache), _ptr(value_cache), _stream(stream)))


def workspace_for(geometry: Geometry, device="cuda"):
    """A workspace tensor of the size the geometry needs (16-byte aligned)."""
    import torch

    n = max(16, int(geometry.workspace_bytes))
    return torch.empty((n + 15) // 16 * 4, dtype=torch.float32, device=device)
