"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle on the
same seeded inputs.  Tolerance (unit-variance V): max abs error <= 2e-3 and
mean abs error <= 2e-4; bitwise equality where the result must not depend on
the run (repeat, graph replay, physical block placement, a row with one
active split against S = 1)."""
import numpy as np
import pytest

import oracle
import workloads
from workloads import Inputs, Problem
from tests.gpu_util import announce, assert_close_to_oracle, run_gpu

pytestmark = pytest.mark.gpu

_cache = {}


def named(name):
    if name not in _cache:
        inp = workloads.workload(name)
        _cache[name] = (inp, oracle.paged_decode(inp))
    return _cache[name]


# ---------------------------------------------------------------------------
# the five workloads at full size, default geometry (the bench configuration)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5", "C2b8", "C4r1"])
def test_workload_parity(name):
    inp, (ref, ref_lse) = named(name)
    announce(f"{name} default geometry")
    got, lse, g = run_gpu(inp)
    mx, mn = assert_close_to_oracle(got, lse, ref, ref_lse, what=name)
    announce(f"{name}: S={g.num_splits} max_abs={mx:.2e} mean_abs={mn:.2e}")


@pytest.mark.parametrize("S", [1, 2, 4, 7, 16])
def test_c1_split_counts(S):
    inp, (ref, ref_lse) = named("C1")
    announce(f"C1 S={S}")
    got, lse, g = run_gpu(inp, splits_override=S, min_chunk=16)
    assert g.num_splits == S
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"C1 S={S}")


@pytest.mark.parametrize("name", ["C2", "C4", "C5"])
@pytest.mark.parametrize("S", [1, 3, 64])
def test_split_overrides(name, S):
    inp, (ref, ref_lse) = named(name)
    announce(f"{name} S={S}")
    got, lse, _ = run_gpu(inp, splits_override=S, min_chunk=16)
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{name} S={S}")


# paged_decode_attention and partials + split_combine give bit-identical
# results, for every form of the merge: a wave per pair for up to 8 splits
# (C5) or 16 splits with many pairs, and a CTA per pair (C2: 64 splits, C3:
# 48, C4 at 24, C1 at 16).
@pytest.mark.parametrize("name,S", [("C3", 0), ("C5", 0), ("C2", 0), ("C4", 24), ("C1", 16)])
def test_partials_then_combine_equals_one_call(name, S):
    inp, (ref, ref_lse) = named(name)
    announce(f"{name} S={S} partials + combine vs paged_decode_attention")
    geo = dict(splits_override=S, min_chunk=16) if S else {}
    a, la, g = run_gpu(inp, **geo)
    b, lb, _ = run_gpu(inp, partials_then_combine=True, **geo)
    assert g.num_splits > 1
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    assert_close_to_oracle(a, la, ref, ref_lse, what=name)


# ---------------------------------------------------------------------------
# every compiled variant on small ragged problems
# ---------------------------------------------------------------------------

VARIANTS = []
for cache in ("f16", "i8", "fp8"):
    for D, VD, lay in ((64, 64, "separate"), (128, 128, "separate"), (256, 256, "separate"),
                       (576, 512, "latent")):
        for gathered in (False, True):
            VARIANTS.append((cache, D, VD, lay, gathered))


def _small(cache, D, VD, lay, gathered, seed=7, rows=5, heads=None, kvh=None, B=16,
           quant=None, sink=True):
    rng = np.random.default_rng(seed)
    if lay == "latent":
        heads, kvh = heads or 16, kvh or 1
    else:
        heads, kvh = heads or 12, kvh or 2
    mbpr = 12
    cap = mbpr * B
    lens = [0, 1, 17, cap - 5, cap + 40][:rows]
    if quant is None:
        quant = "none" if cache == "f16" else ("channel" if seed % 2 else "tensor")
    p = Problem(rows=rows, heads=heads, kv_heads=kvh, head_size=D, v_head_size=VD, block_size=B,
                max_blocks_per_row=mbpr, num_pool_blocks=0,
                max_candidates=70 if gathered else 0, cache_dtype=cache, k_quant=quant,
                v_quant=quant, layout=lay)
    cand = None
    if gathered:
        cand = rng.integers(-3, cap + 3, size=(rows, 70)).astype(np.int32)
        cand[2, :5] = [3, 3, 3, 16, 15]
    return workloads.make_inputs(p, seed, lens, candidates=cand, with_sink=sink,
                                 softmax_scale=1.0 / np.sqrt(D),
                                 num_candidates=None if not gathered else [70, 9, 70, 0, 33])


@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: "-".join(map(str, v)))
def test_every_variant(v):
    inp = _small(*v)
    ref, ref_lse = oracle.paged_decode(inp)
    for S in (1, 5):
        announce(f"variant {v} S={S}")
        got, lse, _ = run_gpu(inp, splits_override=S, min_chunk=16)
        assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{v} S={S}")


@pytest.mark.parametrize("cache", ["f16", "i8", "fp8"])
def test_per_channel_and_fp32_output(cache):
    inp = _small(cache, 128, 128, "separate", False, seed=3,
                 quant="none" if cache == "f16" else "channel")
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"{cache} fp32 output")
    got, lse, _ = run_gpu(inp, out_dtype="f32", splits_override=3, min_chunk=16)
    assert_close_to_oracle(got, lse, ref, ref_lse, max_abs=1e-3, mean_abs=1e-4, what=cache)


def test_more_than_16_heads_per_kv_head():
    inp = _small("f16", 128, 128, "separate", False, heads=40, kvh=2)
    ref, ref_lse = oracle.paged_decode(inp)
    announce("group 20 (two head blocks)")
    got, lse, g = run_gpu(inp, splits_override=2, min_chunk=16)
    assert g.head_blocks == 2
    assert_close_to_oracle(got, lse, ref, ref_lse, what="group 20")


@pytest.mark.parametrize("B", [32, 64, 256])
def test_block_sizes(B):
    inp = _small("i8", 128, 128, "separate", False, B=B, seed=4)
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"block size {B}")
    got, lse, _ = run_gpu(inp, splits_override=4, min_chunk=16)
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"B={B}")


# ---------------------------------------------------------------------------
# edge cases and bitwise properties
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lens", [[0, 0], [1, 15], [16, 17], [255, 256], [256, 999]])
def test_edge_lengths(lens):
    p = Problem(rows=2, heads=4, kv_heads=1, head_size=64, v_head_size=64, block_size=16,
                max_blocks_per_row=16, num_pool_blocks=0, cache_dtype="f16")
    inp = workloads.make_inputs(p, 21, lens, with_sink=True, softmax_scale=0.125)
    ref, ref_lse = oracle.paged_decode(inp)
    for S in (1, 4):
        announce(f"lens {lens} S={S}")
        got, lse, _ = run_gpu(inp, splits_override=S, min_chunk=16)
        assert_close_to_oracle(got, lse, ref, ref_lse, what=f"lens {lens} S={S}")
        if lens[0] == 0:
            assert np.all(got[0] == 0) and np.all(np.isneginf(lse[0]))



@pytest.mark.parametrize("kind", ["kvp", "per_head", "gathered", "latent", "multitoken"])
@pytest.mark.parametrize("balance", [1, 2])
def test_out_of_range_lengths_are_clamped(kind, balance):
    """Row lengths (and candidate counts) anywhere in int32 -- negative, zero,
    past the capacity, INT32_MIN and INT32_MAX -- act as their clamp to
    [0, capacity] ([0, max_candidates]), in both decompositions, as the
    oracle reads them."""
    import dataclasses

    cap, rows, nc = 256, 8, 40
    kw = dict(rows=rows, max_blocks_per_row=cap // 16, block_size=16, num_pool_blocks=0)
    if kind == "latent":
        p = Problem(heads=16, kv_heads=1, head_size=576, v_head_size=512, cache_dtype="fp8",
                    k_quant="tensor", v_quant="tensor", layout="latent",
                    **dict(kw, block_size=64, max_blocks_per_row=cap // 64))
    elif kind == "kvp":
        p = Problem(heads=32, kv_heads=8, head_size=128, v_head_size=128, cache_dtype="f16", **kw)
    elif kind == "multitoken":
        p = Problem(heads=32, kv_heads=8, head_size=64, v_head_size=64, cache_dtype="i8",
                    k_quant="tensor", v_quant="tensor", query_tokens=3, **kw)
    else:
        p = Problem(heads=12, kv_heads=2, head_size=256, v_head_size=256, cache_dtype="i8",
                    k_quant="channel", v_quant="channel",
                    max_candidates=nc if kind == "gathered" else 0, **kw)
    rng = np.random.default_rng(91)
    cand = ncand = None
    if kind == "gathered":
        cand = rng.integers(-2, cap + 2, size=(rows, nc)).astype(np.int32)
        ncand = np.full(rows, nc)
    inp = workloads.make_inputs(p, 91, cap, with_sink=True, candidates=cand,
                                num_candidates=ncand, softmax_scale=1.0 / np.sqrt(p.head_size))
    i32 = np.iinfo(np.int32)
    lens = np.array([-5, i32.max, i32.min, 3, cap, cap + 1, 0, 17], dtype=np.int32)
    inp = dataclasses.replace(inp, seq_lens=lens)
    if kind == "gathered":
        inp = dataclasses.replace(inp, num_candidates=np.array(
            [-1, i32.max, nc, i32.min, 5, 0, nc + 7, 3], dtype=np.int32))
    ref_inp = workloads.expand_query_tokens(inp) if p.query_tokens > 1 else inp
    ref, ref_lse = oracle.paged_decode(ref_inp)
    announce(f"out-of-range lengths: {kind} balance={balance}")
    got, lse, g = run_gpu(inp, balance=balance)
    assert (g.target_ctas > 0) == (balance == 1)
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"clamped lengths {kind} balance={balance}")

def test_repeat_is_bitwise_identical():
    inp, _ = named("C3")
    announce("C3 repeat")
    a, la, _ = run_gpu(inp)
    b, lb, _ = run_gpu(inp)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_block_table_permutation_is_bitwise_invariant():
    inp = _small("i8", 256, 256, "separate", False, seed=5)
    announce("block-table permutation")
    a, la, _ = run_gpu(inp, splits_override=3, min_chunk=16)
    pool = inp.problem.num_pool_blocks
    perm = np.random.default_rng(1).permutation(pool)
    k2 = np.empty_like(inp.key_cache)
    v2 = np.empty_like(inp.value_cache)
    k2[perm] = inp.key_cache
    v2[perm] = inp.value_cache
    moved = Inputs(**{**inp.__dict__, "key_cache": k2, "value_cache": v2,
                      "block_table": perm[inp.block_table].astype(np.int32)})
    b, lb, _ = run_gpu(moved, splits_override=3, min_chunk=16)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_one_active_split_equals_single_split():
    # every row shorter than min_chunk: one active split whatever S is
    p = Problem(rows=3, heads=8, kv_heads=2, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=8, num_pool_blocks=0, cache_dtype="f16")
    inp = workloads.make_inputs(p, 8, [5, 60, 64], with_sink=True)
    announce("one active split vs S=1")
    a, la, _ = run_gpu(inp, splits_override=1, min_chunk=64)
    b, lb, _ = run_gpu(inp, splits_override=8, min_chunk=64)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_invalid_block_id_masks_its_tokens():
    p = Problem(rows=2, heads=4, kv_heads=1, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=6, num_pool_blocks=0, cache_dtype="f16")
    inp = workloads.make_inputs(p, 9, [90, 90])
    bad = inp.block_table.copy()
    bad[0, 2] = -7
    bad[1, 4] = inp.problem.num_pool_blocks + 3
    masked = Inputs(**{**inp.__dict__, "block_table": bad})
    # expected: the same rows with the tokens of those blocks left out
    keep0 = [t for t in range(90) if t // 16 != 2]
    keep1 = [t for t in range(90) if t // 16 != 4]
    n = max(len(keep0), len(keep1))
    cand = np.full((2, n), -1, dtype=np.int32)
    cand[0, :len(keep0)] = keep0
    cand[1, :len(keep1)] = keep1
    pg = Problem(**{**p.__dict__, "num_pool_blocks": inp.problem.num_pool_blocks, "max_candidates": n})
    ref_inp = Inputs(**{**inp.__dict__, "problem": pg, "candidates": cand,
                        "num_candidates": np.array([n, n], dtype=np.int32)})
    ref, ref_lse = oracle.paged_decode(ref_inp)
    announce("invalid block ids")
    got, lse, _ = run_gpu(masked, splits_override=2, min_chunk=16)
    assert_close_to_oracle(got, lse, ref, ref_lse, what="invalid block ids")


def test_hip_graph_replay_matches_eager_with_new_lengths():
    import torch

    import quantized_paged_kv_amd as pkv
    from workloads.device import to_device

    p = Problem(rows=5, heads=12, kv_heads=2, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=12, num_pool_blocks=0, cache_dtype="fp8", k_quant="tensor",
                v_quant="tensor")
    # every row owns all its blocks, so any replay length up to capacity is valid
    inp = workloads.make_inputs(p, 6, 12 * 16, with_sink=True, softmax_scale=1 / np.sqrt(128))
    d = to_device(inp, "cuda")
    prob = pkv.make_problem(**d.problem_kwargs)
    g = pkv.split_geometry(prob, splits_override=4, min_chunk=16)
    ws = pkv.workspace_for(g)
    p = inp.problem
    out = torch.zeros((p.rows, p.heads, p.v_head_size), dtype=torch.float16, device="cuda")
    lse = torch.zeros((p.rows, p.heads), dtype=torch.float32, device="cuda")

    def step():
        pkv.paged_decode_attention(prob, g, d.query, d.key_cache, d.value_cache, d.block_table,
                                   d.seq_lens, None, None, d.k_scale, d.v_scale,
                                   d.softmax_scale, d.head_sink, out, lse, ws)

    announce("graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    lens_list = [[1, 2, 3, 4, 5], [0, 100, 191, 7, 64], [192, 192, 0, 999, 33]]
    for lens in lens_list:
        d.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        announce(f"graph replay lens={lens}")
        graph.replay()
        torch.cuda.synchronize()
        o_graph, l_graph = out.clone(), lse.clone()
        for _ in range(3):  # further replays (each reuses the workspace counters)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(o_graph, out) and torch.equal(l_graph, lse)
        step()  # eager
        torch.cuda.synchronize()
        assert torch.equal(o_graph, out) and torch.equal(l_graph, lse)
        # and the replay is right, not just repeatable
        ref_inp = Inputs(**{**inp.__dict__, "seq_lens": np.array(lens, dtype=np.int32)})
        ref, ref_lse = oracle.paged_decode(workloads.expand_query_tokens(ref_inp))
        assert_close_to_oracle(o_graph.double().cpu().numpy(), l_graph.double().cpu().numpy(),
                               ref, ref_lse, what=f"replay {lens}")


def _replay_with_lengths(inp, lens_list, what, **geo):
    """Capture one decode step in a HIP graph, then for each length vector:
    write it to the device, replay four times (bitwise equal to each other
    and to an eager call) and compare with the oracle at those lengths."""
    import torch

    import quantized_paged_kv_amd as pkv
    from workloads.device import to_device

    d = to_device(inp, "cuda")
    prob = pkv.make_problem(**d.problem_kwargs)
    g = pkv.split_geometry(prob, **geo)
    ws = pkv.workspace_for(g)
    p = inp.problem
    qrows = p.rows * max(1, p.query_tokens)
    out = torch.zeros((qrows, p.heads, p.v_head_size), dtype=torch.float16, device="cuda")
    lse = torch.zeros((qrows, p.heads), dtype=torch.float32, device="cuda")

    def step():
        pkv.paged_decode_attention(prob, g, d.query, d.key_cache, d.value_cache, d.block_table,
                                   d.seq_lens, d.candidates, d.num_candidates, d.k_scale,
                                   d.v_scale, d.softmax_scale, d.head_sink, out, lse, ws)

    announce(f"{what}: graph capture (S={g.num_splits}, target_ctas={g.target_ctas}, "
             f"kv_heads_per_cta={g.kv_heads_per_cta})")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for lens in lens_list:
        d.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        announce(f"{what}: graph replay lens={list(lens)}")
        graph.replay()
        torch.cuda.synchronize()
        o_graph, l_graph = out.clone(), lse.clone()
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(o_graph, out) and torch.equal(l_graph, lse)
        step()  # eager
        torch.cuda.synchronize()
        assert torch.equal(o_graph, out) and torch.equal(l_graph, lse)
        ref_inp = Inputs(**{**inp.__dict__, "seq_lens": np.array(lens, dtype=np.int32)})
        ref, ref_lse = oracle.paged_decode(workloads.expand_query_tokens(ref_inp))
        assert_close_to_oracle(o_graph.double().cpu().numpy(), l_graph.double().cpu().numpy(),
                               ref, ref_lse, what=f"{what} replay {list(lens)}")
    return g


def _replay_lens(rows, cap, seed):
    """Length vectors for replays: random, rows going to 0 and to the full
    capacity, and lengths around tile and block edges (and past capacity,
    which is clamped)."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, 15, 16, 17, 63, 64, 65, cap - 1, cap, cap + 9, 2, 31, 33, 100, cap // 2]
    return [rng.integers(1, cap, size=rows, endpoint=True),
            np.where(np.arange(rows) % 2 == 0, 0, cap),
            np.array([edges[i % len(edges)] for i in range(rows)]),
            np.full(rows, cap), np.zeros(rows, dtype=np.int64)]


@pytest.mark.parametrize("kpc", [0, 8])
def test_graph_replay_continuous_batching_shape(kpc):
    """C3's shape at a smaller capacity: 16 rows (the live-balanced
    decomposition, asked for, every CTA reading all lengths), 32 query / 8 KV heads,
    head 128, FP16 with a head sink: several KV heads per CTA."""
    cap = 512
    p = Problem(rows=16, heads=32, kv_heads=8, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=cap // 16, num_pool_blocks=0, cache_dtype="f16")
    inp = workloads.make_inputs(p, 31, cap, with_sink=True, softmax_scale=1 / np.sqrt(128))
    # (balance asked for: at this capacity the automatic geometry would take
    # the static decomposition, the chunk floor cutting full rows the same way)
    geo = {"kv_heads_per_cta": kpc, "balance": 1} if kpc else {"balance": 1}
    g = _replay_with_lengths(inp, _replay_lens(16, cap, 31), f"C3 shape kpc={kpc}", **geo)
    assert g.target_ctas > 0 and g.kv_heads_per_cta == (kpc or 4) and g.num_splits > 1


@pytest.mark.parametrize("rows,kpc", [(63, 0), (64, 4), (65, 0), (65, 4), (200, 4), (1024, 4)])
def test_live_balanced_row_counts(rows, kpc):
    """The live-balanced decomposition reads one length per lane up to 64
    rows and 64-row groups beyond: row counts on both sides of 64 and up to
    its limit of 1024, lengths from 0 to the capacity, against the oracle on
    every row (per-KV-head kernel and four KV heads per CTA)."""
    cap = 128
    rng = np.random.default_rng(rows)
    lens = rng.integers(0, cap, size=rows, endpoint=True)
    lens[:3] = [0, cap, 1]
    p = Problem(rows=rows, heads=8, kv_heads=4, head_size=64, v_head_size=64, block_size=16,
                max_blocks_per_row=cap // 16, num_pool_blocks=0, cache_dtype="f16")
    inp = workloads.make_inputs(p, 40 + rows, lens, with_sink=True, softmax_scale=0.125)
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"live-balanced, {rows} rows, kv_heads_per_cta={kpc or 1}")
    got, lse, g = run_gpu(inp, balance=1, min_chunk=16, kv_heads_per_cta=kpc or 1)
    assert g.target_ctas > 0 and g.num_splits > 1
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{rows} rows")


@pytest.mark.parametrize("cache,heads,kvh,D,VD,lay", [
    ("f16", 64, 8, 64, 64, "separate"), ("f16", 32, 8, 128, 128, "separate"),
    ("i8", 24, 2, 256, 256, "separate"), ("fp8", 16, 1, 576, 512, "latent")])
@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
def test_combine_many_live_balanced_splits(cache, heads, kvh, D, VD, lay, out_dtype):
    """The combine with more splits than it reads speculatively (rows of up
    to 64 live-balanced splits; 512-2048 pairs: the CTA-per-pair combine,
    whose slots past 16 are read only when their weight is nonzero, and from
    1024 pairs at 128 or more channels the wave-per-pair one), for every
    value-head size, against
    the oracle; paged_decode_attention equals partials + split_combine."""
    cap = 1024
    rows = 32
    rng = np.random.default_rng(D + heads)
    lens = rng.integers(0, cap, size=rows, endpoint=True)
    lens[:4] = [cap, 0, 1, cap - 17]
    quant = "none" if cache == "f16" else "tensor"
    p = Problem(rows=rows, heads=heads, kv_heads=kvh, head_size=D, v_head_size=VD, block_size=16,
                max_blocks_per_row=cap // 16, num_pool_blocks=0, cache_dtype=cache,
                k_quant=quant, v_quant=quant, layout=lay)
    inp = workloads.make_inputs(p, 50 + D, lens, with_sink=True, softmax_scale=1.0 / np.sqrt(D))
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"combine, {cache} {VD} channels, {out_dtype} output, up to 64 live-balanced splits")
    geo = dict(num_cus=256, ctas_per_cu=8, balance=1, splits_override=64, min_chunk=16)
    got, lse, g = run_gpu(inp, out_dtype=out_dtype, **geo)
    assert g.target_ctas > 0 and g.num_splits == 64
    tol = dict(max_abs=1e-3, mean_abs=1e-4) if out_dtype == "f32" else {}
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{VD} channels {out_dtype}", **tol)
    b, lb, _ = run_gpu(inp, out_dtype=out_dtype, geometry=g, partials_then_combine=True)
    assert np.array_equal(got, b) and np.array_equal(lse, lb)


@pytest.mark.parametrize("cache,heads,kvh,D,VD,lay,rows,S,balance", [
    ("i8", 24, 2, 256, 256, "separate", 48, 64, 1),     # 1152 pairs, 16-split batches
    ("fp8", 16, 1, 576, 512, "latent", 64, 40, 1),      # two waves per pair
    ("f16", 32, 8, 128, 128, "separate", 16, 16, 1),    # 512 pairs, S <= 16: all speculative
    ("f16", 64, 8, 64, 64, "separate", 16, 12, 1),
    ("f16", 32, 8, 128, 128, "separate", 32, 48, 2)])   # static decomposition
@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
def test_combine_wave_per_pair(cache, heads, kvh, D, VD, lay, rows, S, balance, out_dtype):
    """The wave-per-pair combine (at most 16 splits from 512 pairs, any
    split count from 1024): rows with no position, one position, one split
    and all S splits, with the loads past the speculated splits taken in
    batches up to the last split with a weight; against the oracle, and
    paged_decode_attention equals partials + split_combine."""
    cap = 1024
    rng = np.random.default_rng(rows + S + D)
    lens = rng.integers(0, cap, size=rows, endpoint=True)
    lens[:5] = [cap, 0, 1, 16, cap - 17]
    quant = "none" if cache == "f16" else "tensor"
    p = Problem(rows=rows, heads=heads, kv_heads=kvh, head_size=D, v_head_size=VD, block_size=16,
                max_blocks_per_row=cap // 16, num_pool_blocks=0, cache_dtype=cache,
                k_quant=quant, v_quant=quant, layout=lay)
    inp = workloads.make_inputs(p, 70 + D, lens, with_sink=True, softmax_scale=1.0 / np.sqrt(D))
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"wave combine, {cache} {VD} channels, {rows * heads} pairs, S={S}, {out_dtype}")
    geo = dict(num_cus=256, ctas_per_cu=8, balance=balance, splits_override=S, min_chunk=16,
               kv_heads_per_cta=1)
    got, lse, g = run_gpu(inp, out_dtype=out_dtype, **geo)
    assert g.num_splits == S and (g.target_ctas > 0) == (balance == 1)
    tol = dict(max_abs=1e-3, mean_abs=1e-4) if out_dtype == "f32" else {}
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{VD} channels S={S} {out_dtype}", **tol)
    b, lb, _ = run_gpu(inp, out_dtype=out_dtype, geometry=g, partials_then_combine=True)
    assert np.array_equal(got, b) and np.array_equal(lse, lb)


@pytest.mark.parametrize("T", [4, 8])
def test_graph_replay_multitoken_shape(T):
    """C3's shape with T query tokens per row (four: the four-KV-head kernel,
    one (token, head) tile per KV head; eight: two head blocks), replayed
    with changing lengths, including rows shorter than T."""
    cap = 256
    p = Problem(rows=16, heads=32, kv_heads=8, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=cap // 16, num_pool_blocks=0, cache_dtype="f16",
                query_tokens=T)
    inp = workloads.make_inputs(p, 33, cap, with_sink=True, softmax_scale=1 / np.sqrt(128))
    g = _replay_with_lengths(inp, _replay_lens(16, cap, 33), f"C3 shape, {T} tokens per row",
                             balance=1, min_chunk=16)
    assert g.target_ctas > 0 and g.head_blocks == T // 4 and g.num_splits > 1


def test_graph_replay_latent_shape():
    """C5's shape at a smaller capacity: 16 rows of the latent FP8 layout
    (16 query heads over one 576-channel head, V = first 512 channels, block
    64): the live-balanced decomposition on the latent kernel's
    direct-to-LDS ring."""
    cap = 1024
    p = Problem(rows=16, heads=16, kv_heads=1, head_size=576, v_head_size=512, block_size=64,
                max_blocks_per_row=cap // 64, num_pool_blocks=0, cache_dtype="fp8",
                k_quant="tensor", v_quant="tensor", layout="latent")
    inp = workloads.make_inputs(p, 32, cap, with_sink=True, softmax_scale=1 / 24)
    # (asked for: the automatic geometry takes the static decomposition here,
    # since the chunk floor would cut even full rows the same way)
    g = _replay_with_lengths(inp, _replay_lens(16, cap, 32), "C5 shape", balance=1)
    assert g.target_ctas > 0 and g.num_splits > 1
    gs = _replay_with_lengths(inp, _replay_lens(16, cap, 32), "C5 shape, automatic geometry")
    assert gs.target_ctas == 0 and gs.num_splits > 1



@pytest.mark.parametrize("balance,latent", [(1, False), (2, False), (1, True)])
def test_graph_replay_gathered_rows(balance, latent):
    """Gathered rows under graph replay: between replays the candidate lists,
    their live counts and the row lengths change (random lists with invalid
    entries, empty lists, full sorted lists, lengths cutting lists short).
    Each replay is bitwise the eager call's and meets the oracle, in the
    live-balanced decomposition (every CTA sums the live candidate counts)
    and the static one, on the per-head and the latent kernels."""
    import torch

    import quantized_paged_kv_amd as pkv
    from workloads.device import to_device

    rows, cap, nc = 16, 1024, 300
    if latent:
        p = Problem(rows=rows, heads=16, kv_heads=1, head_size=576, v_head_size=512,
                    block_size=64, max_blocks_per_row=cap // 64, num_pool_blocks=0,
                    max_candidates=nc, cache_dtype="f16", layout="latent")
    else:
        p = Problem(rows=rows, heads=24, kv_heads=2, head_size=256, v_head_size=256,
                    block_size=16, max_blocks_per_row=cap // 16, num_pool_blocks=0,
                    max_candidates=nc, cache_dtype="i8", k_quant="channel", v_quant="channel")
    rng = np.random.default_rng(77)
    cand0 = rng.integers(-3, cap + 3, size=(rows, nc)).astype(np.int32)
    inp = workloads.make_inputs(p, 77, cap, with_sink=True, candidates=cand0,
                                num_candidates=np.full(rows, nc),
                                softmax_scale=1.0 / np.sqrt(p.head_size))
    d = to_device(inp, "cuda")
    prob = pkv.make_problem(**d.problem_kwargs)
    g = pkv.split_geometry(prob, balance=balance)
    assert (g.target_ctas > 0) == (balance == 1)
    ws = pkv.workspace_for(g)
    out = torch.zeros((rows, p.heads, p.v_head_size), dtype=torch.float16, device="cuda")
    lse = torch.zeros((rows, p.heads), dtype=torch.float32, device="cuda")

    def step():
        pkv.paged_decode_attention(prob, g, d.query, d.key_cache, d.value_cache, d.block_table,
                                   d.seq_lens, d.candidates, d.num_candidates, d.k_scale,
                                   d.v_scale, d.softmax_scale, d.head_sink, out, lse, ws)

    what = f"gathered replay balance={balance} latent={latent}"
    announce(f"{what}: graph capture (S={g.num_splits}, target_ctas={g.target_ctas})")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    sorted_full = np.sort(np.stack([rng.permutation(cap)[:nc] for _ in range(rows)]), axis=1)
    steps = [
        (rng.integers(-3, cap + 3, size=(rows, nc)), rng.integers(0, nc + 1, size=rows),
         np.full(rows, cap)),
        (cand0, np.zeros(rows, dtype=np.int64), np.full(rows, cap)),
        (sorted_full, np.full(rows, nc), np.full(rows, cap)),
        (sorted_full, np.full(rows, nc), rng.integers(0, cap + 1, size=rows)),
        (sorted_full, np.where(np.arange(rows) % 2 == 0, 0, nc), np.full(rows, cap)),
    ]
    for i, (cand, ncand, lens) in enumerate(steps):
        d.candidates.copy_(torch.from_numpy(np.ascontiguousarray(cand, dtype=np.int32)))
        d.num_candidates.copy_(torch.from_numpy(np.asarray(ncand, dtype=np.int32)))
        d.seq_lens.copy_(torch.from_numpy(np.asarray(lens, dtype=np.int32)))
        announce(f"{what}: replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        o_graph, l_graph = out.clone(), lse.clone()
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(o_graph, out) and torch.equal(l_graph, lse)
        step()
        torch.cuda.synchronize()
        assert torch.equal(o_graph, out) and torch.equal(l_graph, lse)
        ref_inp = Inputs(**{**inp.__dict__, "candidates": np.asarray(cand, dtype=np.int32),
                            "num_candidates": np.asarray(ncand, dtype=np.int32),
                            "seq_lens": np.asarray(lens, dtype=np.int32)})
        ref, ref_lse = oracle.paged_decode(ref_inp)
        assert_close_to_oracle(o_graph.double().cpu().numpy(), l_graph.double().cpu().numpy(),
                               ref, ref_lse, what=f"{what} replay {i}")


# ---------------------------------------------------------------------------
# the pages' worked examples (FP32 output)
# ---------------------------------------------------------------------------

from tests.test_oracle_pins import _golden_rows  # noqa: E402

# The large-value-scale rows reach the FP32 path through the tail-depth
# check; signed cancellation is handled by the high + residual FP16
# probability tiles; the others stay on the fast path.


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_worked_examples_on_gpu(row):
    name = row[0]
    (_, q0, q1, ka0, ka1, kb0, kb1, va, vb, vscale, sscale, expected, *_rest) = row
    D = 256
    p = Problem(rows=1, heads=1, kv_heads=1, head_size=D, v_head_size=D, block_size=16,
                max_blocks_per_row=1, num_pool_blocks=1, max_candidates=2, cache_dtype="i8",
                k_quant="tensor", v_quant="tensor", out_dtype="f32")
    q = np.zeros((1, 1, D), dtype=np.float16)
    q[0, 0, 0], q[0, 0, 1] = np.float16(float(q0)), np.float16(float(q1))
    k = np.zeros((1, 16, 1, D), dtype=np.int8)
    v = np.zeros((1, 16, 1, D), dtype=np.int8)
    k[0, 3, 0, :2] = [int(ka0), int(ka1)]
    k[0, 11, 0, :2] = [int(kb0), int(kb1)]
    v[0, 3, 0, 0], v[0, 11, 0, 0] = int(va), int(vb)
    inp = Inputs(problem=p, query=q, key_cache=k, value_cache=v,
                 block_table=np.zeros((1, 1), dtype=np.int32), seq_lens=np.array([16], np.int32),
                 softmax_scale=float(sscale), k_scale=np.array([1.0], np.float32),
                 v_scale=np.array([float(vscale)], np.float32),
                 candidates=np.array([[3, 11]], np.int32), num_candidates=np.array([2], np.int32))
    # Accuracy bound of the FP32 arithmetic on these rows: every probability
    # enters the PV products with a relative error of at most about 2^-22
    # (FP16 high + residual tiles) plus the FP32 exponential's, so the output
    # error is at most 2^-21 of the magnitude of the summed terms,
    # sum_t (p_t / l) |V_t| -- 2^-21 |O| (5e-7 relative) where nothing cancels,
    # and 2^-21 * 4064 for the signed cancellation, whose exact result 0.496 is
    # what remains of +-4064 (a single FP16 tile gives 0 there).
    x = np.array([float(q0) * float(ka0) + float(q1) * float(ka1),
                  float(q0) * float(kb0) + float(q1) * float(kb1)]) * float(sscale)
    w = np.exp(x - x.max())
    w /= w.sum()
    mag = float(np.sum(w * np.abs(np.array([float(va), float(vb)]) * float(vscale))))
    tol = 2.0 ** -21 * mag
    for S in (1, 3):
        announce(f"worked example {name} S={S}")
        got, lse, _ = run_gpu(inp, splits_override=S, min_chunk=16)
        assert abs(got[0, 0, 0] - float(expected)) <= tol, (got[0, 0, 0], float(expected), tol)
        assert np.all(got[0, 0, 1:] == 0)
        ref, ref_lse = oracle.paged_decode(inp)
        assert abs(lse[0, 0] - ref_lse[0, 0]) <= 2.0 ** -21 * max(1.0, abs(ref_lse[0, 0]))


# ---------------------------------------------------------------------------
# robust numerics: the folding bound and the tail-depth check send a CTA to
# the FP32 path, whose result is exact to FP32 rounding
# ---------------------------------------------------------------------------

def test_folding_rounding_case_takes_the_fp32_path():
    from tests.test_oracle_pins import folding_case
    inp, expected = folding_case()
    ref, _ = oracle.paged_decode(inp)
    assert ref[0, 0, 0] == pytest.approx(expected, rel=1e-12)
    announce("folding rounding case")
    got, _, _ = run_gpu(inp, splits_override=1, out_dtype="f32")
    # the folded FP16 query would give 0.5 here
    assert got[0, 0, 0] == pytest.approx(expected, rel=1e-6)
    assert np.all(got[0, 0, 1:] == 0)


def _near_exact(got, ref, lse, ref_lse, rel):
    scale = np.abs(ref).max()
    assert np.abs(got - ref).max() <= rel * scale, (np.abs(got - ref).max(), scale)
    assert np.allclose(lse, ref_lse, rtol=0, atol=1e-5 * (1 + np.abs(ref_lse).max()))


@pytest.mark.parametrize("gathered", [False, True])
def test_large_value_scale_with_deep_tail_is_exact(gathered):
    # value scale 2^20 and queries spread wide enough that probabilities fall
    # below the FP16 tile's range: the tail-depth check must fire.  No sink:
    # a row without a deep tail (one token) stays on the fast path, whose lse
    # carries the folding error that a sink would pass on to the output.
    inp = _small("i8", 256, 256, "separate", gathered, seed=11, quant="tensor", sink=False)
    inp.query[...] = (inp.query.astype(np.float32) * 6.0).astype(np.float16)
    inp.v_scale = (inp.v_scale * 2.0 ** 20).astype(np.float32)
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"large value scale, deep tail, gathered={gathered}")
    got, lse, _ = run_gpu(inp, splits_override=3, min_chunk=16, out_dtype="f32")
    # splits without a deep tail keep the fast path's accuracy (about 1e-3
    # of the value magnitude); the worked examples pin the exact tail cases
    _near_exact(got, ref, lse, ref_lse, 1e-3)


@pytest.mark.parametrize("cache,D,VD,lay,quant", [
    ("i8", 128, 128, "separate", "channel"), ("fp8", 128, 128, "separate", "channel"),
    ("fp8", 576, 512, "latent", "tensor"), ("i8", 576, 512, "latent", "channel")])
def test_folding_over_budget_is_exact(cache, D, VD, lay, quant):
    # large queries: the FP16 rounding of Q k_scale moves the logits by well
    # over 0.125 nats, so every CTA takes the FP32 path
    inp = _small(cache, D, VD, lay, lay == "separate", seed=13, quant=quant)
    inp.query[...] = (inp.query.astype(np.float32) * 200.0).astype(np.float16)
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"folding over budget, {cache} {lay}")
    got, lse, _ = run_gpu(inp, splits_override=2, min_chunk=16, out_dtype="f32")
    _near_exact(got, ref, lse, ref_lse, 1e-4)


# ---------------------------------------------------------------------------
# one split per row: the split kernel writes the output itself
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("v", [("i8", 256, 256, "separate", False), ("f16", 128, 128, "separate", True),
                               ("fp8", 576, 512, "latent", False), ("i8", 576, 512, "latent", True)],
                         ids=lambda v: "-".join(map(str, v)))
@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
def test_single_split_direct_output_equals_partials_and_combine(v, out_dtype):
    """With S = 1 paged_decode_attention skips the combine launch; its output
    and lse are bitwise those of paged_decode_partials + split_combine (rows
    include an empty one; the head sink is on)."""
    inp = _small(*v, seed=9)
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"direct output {v} {out_dtype}")
    a, la, g = run_gpu(inp, out_dtype=out_dtype, splits_override=1, min_chunk=16)
    assert g.num_splits == 1
    b, lb, _ = run_gpu(inp, out_dtype=out_dtype, geometry=g, partials_then_combine=True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    assert_close_to_oracle(a, la, ref, ref_lse, what=f"direct {v}")


def test_single_split_direct_output_on_the_fp32_path():
    """A CTA that takes the FP32 path (folding over budget) with S = 1 also
    writes the final output directly, bitwise as the combine would."""
    inp = _small("i8", 256, 256, "separate", False, seed=10, quant="channel")
    # Q k_scale products that FP16 cannot hold exactly, and large: the
    # folding bound is far over budget for every head
    inp.k_scale[...] = np.float32(1.0 / 3.0)
    inp.query[...] = (inp.query.astype(np.float32) * 1000.0).astype(np.float16)
    ref, ref_lse = oracle.paged_decode(inp)
    announce("direct output, FP32 path")
    a, la, g = run_gpu(inp, splits_override=1, min_chunk=16)
    b, lb, _ = run_gpu(inp, geometry=g, partials_then_combine=True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(la[fin], ref_lse[fin], rtol=1e-5, atol=1e-3)


def test_prefill_shape_sampled_rows():
    """The dynamic-sparse prefill shape (128 rows x 2048 gathered candidates,
    INT8 per-channel, one split per row by default geometry) against the
    oracle on a sample of rows."""
    inp = workloads.workload("P128")
    rows = list(range(0, 128, 9))
    ref, ref_lse = oracle.paged_decode(inp, rows=rows)
    announce("P128 prefill shape")
    got, lse, g = run_gpu(inp)
    assert_close_to_oracle(got[rows], lse[rows], ref[rows], ref_lse[rows], what="P128")
    announce(f"P128: S={g.num_splits}")


def test_prefill_whole_step_2048_rows():
    """The dynamic-sparse prefill shape with 2048 rows (each its own 2048
    sorted candidates of an 8192-token sequence, INT8 per channel; the DSA
    page's prefill table) at the default geometry, every row against the
    oracle."""
    inp = workloads.workload("P2048")
    announce("P2048 prefill shape: the oracle on all 2048 rows (host cores, ~30 s)")
    ref, ref_lse = oracle.paged_decode(inp)
    announce("P2048 prefill shape, whole step")
    got, lse, g = run_gpu(inp)
    mx, mn = assert_close_to_oracle(got, lse, ref, ref_lse, what="P2048")
    announce(f"P2048: S={g.num_splits} max_abs={mx:.2e} mean_abs={mn:.2e}")


@pytest.mark.parametrize("name", ["X4096b8i8", "X1024b32fp8"])
@pytest.mark.parametrize("S", [0, 12, 16])
def test_paged_page_shapes(name, S):
    """The PagedAttention page's isolated decode shapes (64q/8kv, head 64,
    block 256, INT8 / FP8 per tensor): default geometry, and 12 or 16 splits,
    which with 512+ (row, head) pairs take the wave-per-pair combine."""
    inp, (ref, ref_lse) = named(name)
    announce(f"{name} S={S}")
    geo = {} if S == 0 else dict(splits_override=S, min_chunk=16)
    got, lse, g = run_gpu(inp, **geo)
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{name} S={g.num_splits}")


# ---------------------------------------------------------------------------
# long rows: a wave walks more than 64 tiles, so the per-wave window of
# block ids (64 tiles per vector register) is refilled mid-row; and more rows
# than the live-balanced decomposition takes (static mode), and exactly its
# limit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cache,lay", [("fp8", "separate"), ("i8", "separate"),
                                       ("fp8", "latent"), ("f16", "latent")])
@pytest.mark.parametrize("S", [1, 3])
def test_long_rows_refill_block_windows(cache, lay, S):
    if lay == "separate":
        heads, kvh, D, VD, ctx = 4, 1, 64, 64, 65536
    else:
        heads, kvh, D, VD, ctx = 16, 1, 576, 512, 16384
    quant = "none" if cache == "f16" else "tensor"
    p = Problem(rows=2, heads=heads, kv_heads=kvh, head_size=D, v_head_size=VD, block_size=16,
                max_blocks_per_row=ctx // 16, num_pool_blocks=0, cache_dtype=cache,
                k_quant=quant, v_quant=quant, layout=lay)
    inp = workloads.make_inputs(p, 11, [ctx, ctx - 37], with_sink=True,
                                softmax_scale=1.0 / np.sqrt(D))
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"long rows {cache} {lay} ctx {ctx} S={S}")
    got, lse, g = run_gpu(inp, splits_override=S, min_chunk=16)
    assert g.num_splits == S
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"long {cache} {lay} S={S}")


@pytest.mark.parametrize("rows,balance", [(1100, 0), (1024, 1), (1024, 2)])
def test_many_rows(rows, balance):
    rng = np.random.default_rng(rows)
    lens = rng.integers(0, 97, size=rows)
    lens[:3] = [0, 96, 1]
    p = Problem(rows=rows, heads=8, kv_heads=2, head_size=64, v_head_size=64, block_size=16,
                max_blocks_per_row=6, num_pool_blocks=0, cache_dtype="f16")
    inp = workloads.make_inputs(p, 12, lens, with_sink=True, softmax_scale=0.125)
    ref, ref_lse = oracle.paged_decode(inp)
    announce(f"{rows} rows balance={balance}")
    got, lse, g = run_gpu(inp, balance=balance)
    assert (g.target_ctas > 0) == (balance == 1)
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{rows} rows balance={balance}")


# ---------------------------------------------------------------------------
# four KV heads per CTA (chosen automatically with a multiple of four KV
# heads, at most 16 query heads per KV head and head size <= 128): against
# the oracle, next to one KV head per CTA
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cache,D", [(c, D) for c in ("f16", "i8", "fp8") for D in (64, 128, 256)],
                         ids=lambda v: str(v))
@pytest.mark.parametrize("heads,kvh", [(32, 8), (64, 8), (12, 4)])
def test_four_kv_heads_per_cta(cache, D, heads, kvh):
    inp = _small(cache, D, D, "separate", False, seed=21, heads=heads, kvh=kvh)
    ref, ref_lse = oracle.paged_decode(inp)
    for S in (1, 5):
        for kpc in [k for k in (1, 4, 8) if kvh % k == 0]:
            announce(f"{cache} D={D} {heads}q/{kvh}kv S={S} kv_heads_per_cta={kpc}")
            got, lse, g = run_gpu(inp, splits_override=S, min_chunk=16, kv_heads_per_cta=kpc)
            assert g.kv_heads_per_cta == kpc
            assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{cache} D={D} S={S} kpc={kpc}")


@pytest.mark.parametrize("cache,D", [("f16", 128), ("i8", 64), ("fp8", 128)], ids=lambda v: str(v))
@pytest.mark.parametrize("heads", [72, 128])
def test_four_kv_heads_per_cta_two_head_blocks(cache, D, heads):
    """17-32 query heads per KV head (group 18, a ragged second block, and
    32): each wave takes both 16-slot head blocks of its KV head."""
    inp = _small(cache, D, D, "separate", False, seed=23, heads=heads, kvh=4)
    ref, ref_lse = oracle.paged_decode(inp)
    for S in (1, 5):
        for kpc in (1, 4):
            announce(f"{cache} D={D} {heads}q/4kv S={S} kv_heads_per_cta={kpc}")
            got, lse, g = run_gpu(inp, splits_override=S, min_chunk=16, kv_heads_per_cta=kpc)
            assert g.kv_heads_per_cta == kpc and g.head_blocks == 2
            assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{cache} D={D} {heads}q S={S} kpc={kpc}")


def test_four_kv_heads_per_cta_is_the_default_where_allowed():
    import quantized_paged_kv_amd as pkv
    from workloads.device import problem_kwargs

    for name, expect in (("C3", 4), ("X4096b8i8", 4), ("C3t8", 4), ("C2", 1), ("C4", 1), ("C5", 1)):
        inp, _ = named(name)
        g = pkv.split_geometry(pkv.make_problem(**problem_kwargs(inp.problem)))
        assert g.kv_heads_per_cta == expect, name


@pytest.mark.parametrize("heads,kvh", [(32, 8), (80, 4)])
@pytest.mark.parametrize("case", ["fold", "tail"])
def test_four_kv_heads_per_cta_fp32_path(case, heads, kvh):
    # every CTA takes the FP32 path: folding over budget (large queries), or
    # a deep tail with a large value scale (group 20: two head blocks per wave)
    if case == "fold":
        inp = _small("i8", 128, 128, "separate", False, seed=13, quant="channel", heads=heads, kvh=kvh)
        inp.query[...] = (inp.query.astype(np.float32) * 200.0).astype(np.float16)
        rel = 1e-4
    else:
        inp = _small("i8", 128, 128, "separate", False, seed=11, quant="tensor", heads=heads, kvh=kvh,
                     sink=False)
        inp.query[...] = (inp.query.astype(np.float32) * 6.0).astype(np.float16)
        inp.v_scale = (inp.v_scale * 2.0 ** 20).astype(np.float32)
        rel = 1e-3
    ref, ref_lse = oracle.paged_decode(inp)
    for S in (1, 2):
        announce(f"four KV heads per CTA, FP32 path ({case}), S={S}")
        got, lse, g = run_gpu(inp, splits_override=S, min_chunk=16, out_dtype="f32",
                              kv_heads_per_cta=4)
        _near_exact(got, ref, lse, ref_lse, rel)
