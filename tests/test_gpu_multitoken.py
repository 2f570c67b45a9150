"""Several query tokens per row (the multi-token decode of speculative and
chunked steps; the DSA page's decode tests sweep 1, 3 and 8 query rows of
one sequence).  The T tokens of a row share its block-table row and attend
causally (token j: len - T + 1 + j positions); the kernels put the (token,
head) pairs of a KV head into the 16-wide MFMA columns, so a KV tile is read
once for all of them.  The oracle evaluates the same step as T * rows
separate rows (workloads.expand_query_tokens); the tolerance is the usual
one."""
import numpy as np
import pytest

import oracle
import workloads
from workloads import Problem
from tests.gpu_util import announce, assert_close_to_oracle, run_gpu

pytestmark = pytest.mark.gpu


def _mt(cache, D, heads, kvh, T, seed=50, rows=6, B=16, mbpr=12):
    quant = "none" if cache == "f16" else ("channel" if seed % 2 else "tensor")
    cap = mbpr * B
    lens = [0, 1, T, cap - 3, cap + 40, 77][:rows]
    p = Problem(rows=rows, heads=heads, kv_heads=kvh, head_size=D, v_head_size=D, block_size=B,
                max_blocks_per_row=mbpr, num_pool_blocks=0, cache_dtype=cache, k_quant=quant,
                v_quant=quant, query_tokens=T)
    return workloads.make_inputs(p, seed + T, lens, with_sink=True, softmax_scale=1.0 / np.sqrt(D))


CASES = [("f16", 128, 32, 8, T) for T in (1, 2, 3, 4, 8)] + [
    ("i8", 256, 24, 2, 3), ("fp8", 64, 64, 8, 2), ("i8", 128, 8, 4, 8), ("fp8", 128, 16, 4, 4),
    ("fp8", 64, 24, 4, 3), ("i8", 128, 40, 4, 3), ("f16", 64, 16, 4, 7)]


def _kpc_allowed(D, heads, kvh, T, kpc):
    vgroup = T * heads // kvh
    return kpc == 1 or (kvh % kpc == 0 and (vgroup <= 16 or (kpc == 4 and vgroup <= 32 and D <= 128)))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_multitoken_rows_against_the_oracle(case):
    cache, D, heads, kvh, T = case
    inp = _mt(cache, D, heads, kvh, T, seed=51 + (1 if cache == "i8" else 0))
    ref, ref_lse = oracle.paged_decode(workloads.expand_query_tokens(inp))
    vgroup = T * heads // kvh
    for S in (1, 5):
        for kpc in [k for k in (1, 4, 8) if _kpc_allowed(D, heads, kvh, T, k)]:
            announce(f"multi-token {case} S={S} kv_heads_per_cta={kpc}")
            got, lse, g = run_gpu(inp, splits_override=S, min_chunk=16, kv_heads_per_cta=kpc)
            assert g.head_blocks == -(-vgroup // 16)
            assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{case} S={S} kpc={kpc}")
            # a token with nothing to attend (len - T + 1 + j <= 0) is empty
            empty = np.isneginf(ref_lse)
            assert np.all(got[empty] == 0)


@pytest.mark.parametrize("name", ["C3t4", "C3t8"])
def test_multitoken_continuous_batching_full_size(name):
    """C3's 16 sequences with 4 (one MFMA tile of (token, head) pairs per KV
    head) or 8 query tokens (two tiles, both taken by each wave) each, in the
    four-KV-head kernel of the default geometry, against the oracle on all
    their query rows."""
    inp = workloads.workload(name)
    ref, ref_lse = oracle.paged_decode(workloads.expand_query_tokens(inp))
    announce(f"{name} default geometry")
    got, lse, g = run_gpu(inp)
    assert g.kv_heads_per_cta == 4
    mx, mn = assert_close_to_oracle(got, lse, ref, ref_lse, what=name)
    announce(f"{name}: S={g.num_splits} kv_heads_per_cta={g.kv_heads_per_cta} "
             f"head_blocks={g.head_blocks} max_abs={mx:.2e} mean_abs={mn:.2e}")


@pytest.mark.parametrize("T", [3, 8])
def test_multitoken_fp32_path(T):
    """A CTA over budget (large queries: the FP32 path) with several tokens
    per row evaluates each (token, head) pair with its own length (with 8
    tokens: both head blocks of each wave)."""
    inp = _mt("i8", 128, 32, 8, T, seed=13)
    inp.query[...] = (inp.query.astype(np.float32) * 200.0).astype(np.float16)
    ref, ref_lse = oracle.paged_decode(workloads.expand_query_tokens(inp))
    for kpc in (1, 4):
        announce(f"multi-token FP32 path T={T} kv_heads_per_cta={kpc}")
        got, lse, _ = run_gpu(inp, splits_override=2, min_chunk=16, out_dtype="f32",
                              kv_heads_per_cta=kpc)
        scale = np.abs(ref).max()
        assert np.abs(got - ref).max() <= 1e-4 * scale
        fin = np.isfinite(ref_lse)
        np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("T,kpc", [(3, 4), (8, 1), (8, 4)])
def test_multitoken_with_softcap(T, kpc):
    """The soft cap (the kernels' EXT instantiation) with several tokens per
    row: the cap applies to every (token, head) pair's scaled logits."""
    from dataclasses import replace
    inp = _mt("fp8", 128, 32, 8, T, seed=61)
    inp = workloads.Inputs(**{**inp.__dict__, "problem": replace(inp.problem, softcap=2.5)})
    inp.query[...] = (inp.query.astype(np.float32) * 3.0).astype(np.float16)  # so the cap binds
    ref, ref_lse = oracle.paged_decode(workloads.expand_query_tokens(inp))
    uncapped, _ = oracle.paged_decode(workloads.expand_query_tokens(
        workloads.Inputs(**{**inp.__dict__, "problem": replace(inp.problem, softcap=0.0)})))
    assert np.abs(ref - uncapped).max() > 1e-2  # the cap changes the result
    for S in (1, 4):
        announce(f"multi-token softcap T={T} S={S} kv_heads_per_cta={kpc}")
        got, lse, _ = run_gpu(inp, splits_override=S, min_chunk=16, kv_heads_per_cta=kpc)
        assert_close_to_oracle(got, lse, ref, ref_lse, what=f"softcap T={T} S={S}")


@pytest.mark.parametrize("T,W", [(3, 1), (3, 17), (8, 5), (8, 40), (4, 100)])
@pytest.mark.parametrize("kpc,balance", [(1, 2), (4, 1), (4, 2)])
def test_multitoken_with_sliding_window(T, W, kpc, balance):
    """A sliding window with several tokens per row: token j attends the last
    W of its own len - T + 1 + j positions, so the tokens' windows start at
    different positions; the row's range starts at the first token's window
    start and each (token, head) slot masks the positions before its own.
    Windows shorter than T, inside one tile and across several tiles, with
    one or four KV heads per CTA, both decompositions and split counts."""
    from dataclasses import replace
    inp = _mt("f16" if W % 2 else "i8", 128, 32, 8, T, seed=71 + W)
    inp = workloads.Inputs(**{**inp.__dict__, "problem": replace(inp.problem, sliding_window=W)})
    ref, ref_lse = oracle.paged_decode(workloads.expand_query_tokens(inp))
    full, _ = oracle.paged_decode(workloads.expand_query_tokens(
        workloads.Inputs(**{**inp.__dict__, "problem": replace(inp.problem, sliding_window=0)})))
    assert np.abs(ref - full).max() > 1e-2  # the window changes the result
    for geo in (dict(balance=balance), dict(splits_override=3, min_chunk=16, balance=balance)):
        announce(f"multi-token window T={T} W={W} kv_heads_per_cta={kpc} {geo}")
        got, lse, g = run_gpu(inp, kv_heads_per_cta=kpc, **geo)
        assert (g.target_ctas > 0) == (balance == 1)
        assert_close_to_oracle(got, lse, ref, ref_lse, what=f"window T={T} W={W} kpc={kpc} {geo}")


@pytest.mark.parametrize("T,W", [(3, 20), (8, 40)])
def test_multitoken_with_sliding_window_fp32_path(T, W):
    """The FP32 path (large queries) with several tokens per row and a
    window: each (token, head) pair keeps its own window."""
    from dataclasses import replace
    inp = _mt("i8", 128, 32, 8, T, seed=13)
    inp = workloads.Inputs(**{**inp.__dict__, "problem": replace(inp.problem, sliding_window=W)})
    inp.query[...] = (inp.query.astype(np.float32) * 200.0).astype(np.float16)
    ref, ref_lse = oracle.paged_decode(workloads.expand_query_tokens(inp))
    for kpc in (1, 4):
        announce(f"multi-token window FP32 path T={T} W={W} kv_heads_per_cta={kpc}")
        got, lse, _ = run_gpu(inp, splits_override=2, min_chunk=16, out_dtype="f32",
                              kv_heads_per_cta=kpc)
        scale = np.abs(ref).max()
        assert np.abs(got - ref).max() <= 1e-4 * scale
        fin = np.isfinite(ref_lse)
        np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-5, atol=1e-4)
