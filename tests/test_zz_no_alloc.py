"""paged_decode_attention_noalloc (the entry point for callers that cannot
allocate: its partials live in the library's per-device array) against
paged_decode_attention with a caller workspace and the same geometry: the
same kernels, so the outputs must be bitwise equal.  Two calls in a row, the
second on a smaller problem (the array keeps the first call's partials),
then the first problem again; each checked against the oracle as well."""
import numpy as np
import pytest

import oracle
import workloads
from workloads import Problem
from tests.gpu_util import announce, assert_close_to_oracle

pytestmark = pytest.mark.gpu


def _problem(rows, lens_hi, seed, cache="f16", kvh=8, heads=32, D=128):
    quant = "none" if cache == "f16" else "tensor"
    p = Problem(rows=rows, heads=heads, kv_heads=kvh, head_size=D, v_head_size=D, block_size=16,
                max_blocks_per_row=64, num_pool_blocks=0, cache_dtype=cache, k_quant=quant,
                v_quant=quant)
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, lens_hi, size=rows, endpoint=True)
    lens[0] = lens_hi
    return workloads.make_inputs(p, seed, lens, with_sink=True, softmax_scale=1 / np.sqrt(D))


def _both(inp):
    import torch

    import quantized_paged_kv_amd as pkv
    from workloads.device import to_device

    d = to_device(inp, "cuda")
    prob = pkv.make_problem(**d.problem_kwargs)
    g = pkv.split_geometry(prob)
    assert 0 < g.workspace_bytes <= pkv.NOALLOC_WORKSPACE_BYTES
    p = inp.problem
    outs = []
    for noalloc in (False, True):
        out = torch.full((p.rows, p.heads, p.v_head_size), float("nan"), dtype=torch.float16,
                         device="cuda")
        lse = torch.full((p.rows, p.heads), float("nan"), dtype=torch.float32, device="cuda")
        args = (prob, g, d.query, d.key_cache, d.value_cache, d.block_table, d.seq_lens,
                d.candidates, d.num_candidates, d.k_scale, d.v_scale, d.softmax_scale,
                d.head_sink, out, lse)
        if noalloc:
            pkv.paged_decode_attention_noalloc(*args)
        else:
            ws = pkv.workspace_for(g)
            pkv.paged_decode_attention(*args, ws)
        torch.cuda.synchronize()
        outs.append((out.double().cpu().numpy(), lse.double().cpu().numpy()))
    return outs, g


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    big = _problem(24, 1024, 41)
    small = _problem(5, 300, 42, cache="i8", kvh=2, heads=24, D=256)
    for name, inp in (("first call, 24 rows", big), ("second call, 5 rows (smaller)", small),
                      ("third call, 24 rows again", big)):
        announce(f"noalloc {name}")
        ((a, la), (b, lb)), g = _both(inp)
        assert g.num_splits > 1  # the partials really go through the array
        assert np.array_equal(a, b, equal_nan=False) and np.array_equal(la, lb)
        ref, ref_lse = oracle.paged_decode(inp)
        assert_close_to_oracle(b, lb, ref, ref_lse, what=f"noalloc {name}")
