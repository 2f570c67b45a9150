"""GPU parity of the sliding window and the logit soft cap (ONNX Runtime PR
#29912, "Summary of Changes": the paged decode kernel supports both).

The oracle attends positions [len - W, len) and caps each scaled logit as
c tanh(x / c).  The kernels number a windowed row's positions from the
window start rounded down to 16 and mask the few positions before it; these
tests cover windows that start inside a tile, on a tile boundary, and before
the row, every kernel family, both decompositions, and that blocks wholly
before the window are never read."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, assert_close_to_oracle, run_gpu
from tests.test_gpu_parity import _small
from workloads import Inputs

pytestmark = pytest.mark.gpu

FAMILIES = [
    ("f16", 128, 128, "separate", False),
    ("i8", 256, 256, "separate", False),
    ("fp8", 64, 64, "separate", False),
    ("fp8", 576, 512, "latent", False),
    ("i8", 128, 128, "separate", True),
    ("f16", 576, 512, "latent", True),
]


def _with(inp, window=0, softcap=0.0):
    return Inputs(**{**inp.__dict__,
                     "problem": replace(inp.problem, sliding_window=window, softcap=softcap)})


@pytest.mark.parametrize("fam", FAMILIES, ids=lambda v: "-".join(map(str, v)))
@pytest.mark.parametrize("W", [1, 16, 20, 100, 500])
def test_sliding_window(fam, W):
    # row lengths 0, 1, 17, 187, 192 (capacity): windows start inside a
    # tile (W = 20, 100), on a tile boundary (W = 16 at 192), or before the
    # row (W = 500)
    inp = _with(_small(*fam, seed=11), window=W)
    ref, ref_lse = oracle.paged_decode(inp)
    for geo in (dict(splits_override=1, min_chunk=16), dict(splits_override=5, min_chunk=16),
                dict(balance=1)):
        announce(f"window {W} {fam} {geo}")
        got, lse, g = run_gpu(inp, **geo)
        assert_close_to_oracle(got, lse, ref, ref_lse, what=f"W={W} {fam} {geo}")


@pytest.mark.parametrize("fam", FAMILIES, ids=lambda v: "-".join(map(str, v)))
@pytest.mark.parametrize("cap,W", [(1.5, 0), (30.0, 0), (2.0, 20)])
def test_softcap(fam, cap, W):
    inp = _with(_small(*fam, seed=12), window=W, softcap=cap)
    ref, ref_lse = oracle.paged_decode(inp)
    for geo in (dict(splits_override=3, min_chunk=16), dict(balance=1)):
        announce(f"softcap {cap} window {W} {fam} {geo}")
        got, lse, _ = run_gpu(inp, **geo)
        assert_close_to_oracle(got, lse, ref, ref_lse, what=f"cap={cap} W={W} {fam} {geo}")


def test_softcap_bounds_a_huge_logit():
    """Queries scaled so that raw logits reach thousands of nats: the cap
    keeps them in (-c, c), so lse < c + log(len)."""
    inp = _small("f16", 128, 128, "separate", False, seed=13, sink=False)
    inp.query[...] = (inp.query.astype(np.float32) * 200.0).astype(np.float16)
    inp = _with(inp, softcap=20.0)
    ref, ref_lse = oracle.paged_decode(inp)
    announce("softcap 20 with logits in the thousands")
    got, lse, _ = run_gpu(inp, splits_override=4, min_chunk=16)
    assert_close_to_oracle(got, lse, ref, ref_lse, what="huge logits, cap 20")
    fin = np.isfinite(ref_lse)
    assert np.all(lse[fin] < 20.0 + np.log(200.0))


@pytest.mark.parametrize("cache", ["f16", "fp8"])
def test_window_never_reads_blocks_before_it(cache):
    """Blocks that lie wholly before a row's window are filled with NaN: the
    result stays finite and equal to the oracle's (which never reads them)."""
    lay, D, VD = ("latent", 576, 512) if cache == "fp8" else ("separate", 128, 128)
    inp = _small(cache, D, VD, lay, False, seed=14)
    W = 40
    ref, ref_lse = oracle.paged_decode(_with(inp, window=W))
    B = inp.problem.block_size
    kc = inp.key_cache.copy()
    vc = None if inp.value_cache is None else inp.value_cache.copy()
    nan = workloads.poison_value(cache)
    for r in range(inp.problem.rows):
        n = min(int(inp.seq_lens[r]), inp.problem.capacity)
        first = max(0, n - W) // B  # the block holding the window start
        for b in range(first):
            blk = inp.block_table[r, b]
            kc[blk] = nan
            if vc is not None:
                vc[blk] = nan
    bad = _with(Inputs(**{**inp.__dict__, "key_cache": kc, "value_cache": vc}), window=W)
    for geo in (dict(splits_override=4, min_chunk=16), dict(balance=1)):
        announce(f"window {W} over poisoned blocks {cache} {geo}")
        got, lse, _ = run_gpu(bad, **geo)
        assert_close_to_oracle(got, lse, ref, ref_lse, what=f"poisoned before window {geo}")


def test_continuous_batching_workload_with_window_and_cap():
    """The 16-row continuous-batching workload (lengths 512..8192) with a
    1000-token window and a soft cap of 30, default geometry."""
    inp = _with(workloads.workload("C3"), window=1000, softcap=30.0)
    ref, ref_lse = oracle.paged_decode(inp)
    announce("C3 window 1000 softcap 30")
    got, lse, g = run_gpu(inp)
    mx, mn = assert_close_to_oracle(got, lse, ref, ref_lse, what="C3 window+cap")
    announce(f"C3 window: S={g.num_splits} max_abs={mx:.2e} mean_abs={mn:.2e}")


@pytest.mark.parametrize("cache,D", [("f16", 128), ("i8", 64)], ids=lambda v: str(v))
@pytest.mark.parametrize("heads,kvh", [(32, 8), (80, 4)])
@pytest.mark.parametrize("W,cap", [(20, 0.0), (100, 2.0), (0, 30.0)])
def test_window_and_cap_with_four_kv_heads_per_cta(cache, D, heads, kvh, W, cap):
    """The window and the cap in the four-KV-head kernel, with one head block
    per wave (group 4) and two (group 20), both decompositions."""
    inp = _with(_small(cache, D, D, "separate", False, seed=13, heads=heads, kvh=kvh),
                window=W, softcap=cap)
    ref, ref_lse = oracle.paged_decode(inp)
    for geo in (dict(splits_override=3, min_chunk=16), dict(balance=1)):
        announce(f"four KV heads per CTA, {cache} D={D} {heads}q/{kvh}kv window {W} cap {cap} {geo}")
        got, lse, g = run_gpu(inp, kv_heads_per_cta=4, **geo)
        assert g.kv_heads_per_cta == 4
        assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{cache} {heads}q W={W} cap={cap} {geo}")
