"""GPU parity of the quantise-on-write cache writer (``reshape_and_cache``)
against the oracle (ONNX Runtime PR #29912, "Summary of Changes":
ReshapeAndCache writes each new token at the slot its slot_mapping entry
names, quantised with k_scale / v_scale).

Codes are integer decisions taken from the same FP32 quotient on both sides,
so every comparison here is bit-exact on whole caches (skipped slots must
keep their previous bytes)."""
import numpy as np
import pytest

import workloads
from oracle import cache_write
from tests.gpu_util import announce
from workloads import Problem

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch

    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
    return torch.from_numpy(a).cuda()


def _bytes(t):
    return t.cpu().contiguous().view(-1).view(__import__("torch").uint8).numpy()


def _old_cache(rng, shape, cache_dtype):
    """Prior cache contents: random bytes (finite for FP16 caches)."""
    if cache_dtype == "f16":
        return rng.standard_normal(shape).astype(np.float16)
    return rng.integers(0, 256, size=shape, dtype=np.uint8).view(workloads.code_dtype(cache_dtype))


def _run_writer(p, nt, kc, vc, num_tokens=None):
    import torch

    import quantized_paged_kv_amd as pkv
    from workloads.device import problem_kwargs

    prob = pkv.make_problem(**problem_kwargs(p))
    dk, dv = _dev(kc), _dev(vc)
    pkv.reshape_and_cache(prob, _dev(nt.key), _dev(nt.value), _dev(nt.slot_mapping),
                          _dev(nt.k_scale), _dev(nt.v_scale), dk, dv, num_tokens=num_tokens)
    torch.cuda.synchronize()
    return dk, dv


def _check(p, nt, seed=0):
    rng = np.random.default_rng(seed + 1000)
    B, pool, KVH = p.block_size, p.num_pool_blocks, p.kv_heads
    kc = _old_cache(rng, (pool, B, KVH, p.head_size), p.cache_dtype)
    vc = None if p.layout == "latent" else _old_cache(rng, (pool, B, KVH, p.v_head_size),
                                                      p.cache_dtype)
    ref_k, ref_v = cache_write.reshape_and_cache(p, nt.key, nt.value, nt.slot_mapping,
                                                 nt.k_scale, nt.v_scale, kc, vc)
    dk, dv = _run_writer(p, nt, kc, vc)
    got_k = _bytes(dk).reshape(ref_k.view(np.uint8).shape)
    bad = np.nonzero(got_k != ref_k.view(np.uint8))
    assert bad[0].size == 0, f"key cache differs at {len(bad[0])} bytes, first {tuple(b[0] for b in bad)}"
    if vc is not None:
        got_v = _bytes(dv).reshape(ref_v.view(np.uint8).shape)
        assert np.array_equal(got_v, ref_v.view(np.uint8)), "value cache differs"


CASES = [
    ("f16", "none", "none"), ("f16", "tensor", "channel"),
    ("i8", "tensor", "tensor"), ("i8", "channel", "channel"), ("i8", "channel", "tensor"),
    ("fp8", "tensor", "tensor"), ("fp8", "channel", "channel"), ("fp8", "tensor", "channel"),
]


@pytest.mark.parametrize("cache,kq,vq", CASES, ids=lambda x: str(x))
def test_separate_caches_bitwise(cache, kq, vq):
    # 700 tokens x 8 KV heads x (16 + 16) chunks: 700 CTAs' worth of threads
    # with a ragged last CTA, a tenth of the tokens skipped
    p = Problem(rows=1, heads=32, kv_heads=8, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=64, num_pool_blocks=64, cache_dtype=cache, k_quant=kq,
                v_quant=vq)
    announce(f"writer separate {cache} k={kq} v={vq}")
    _check(p, workloads.new_tokens(p, 700, seed=11))


@pytest.mark.parametrize("cache,kq", [("f16", "none"), ("i8", "tensor"), ("i8", "channel"),
                                      ("fp8", "tensor"), ("fp8", "channel")])
def test_latent_cache_bitwise(cache, kq):
    # one 576-channel latent row per token, block 64
    p = Problem(rows=1, heads=16, kv_heads=1, head_size=576, v_head_size=512, block_size=64,
                max_blocks_per_row=16, num_pool_blocks=16, cache_dtype=cache, k_quant=kq,
                v_quant="none", layout="latent")
    announce(f"writer latent {cache} k={kq}")
    _check(p, workloads.new_tokens(p, 333, seed=12))


@pytest.mark.parametrize("cache", ["f16", "i8", "fp8"])
@pytest.mark.parametrize("scale", [1.0, 0.125, 0.0371, 3.0, 1.0 / 448.0, -0.37, 2.0 ** 110,
                                   1e-39])
def test_every_fp16_input_bitwise(cache, scale):
    """Every non-NaN binary16 value (ties, saturation, subnormals, signed
    zeros, infinities) through the writer with a per-tensor scale; 2^110
    gives FP32 quotients below the normal range, 1e-39 is a subnormal scale
    (quotients overflow)."""
    vals = workloads.every_fp16_value()
    D = 64
    T = -(-len(vals) // D)
    x = np.zeros(T * D, dtype=np.float16)
    x[:len(vals)] = vals
    key = x.reshape(T, 1, D)
    value = x[::-1].copy().reshape(T, 1, D)
    B = 16
    quant = "none" if cache == "f16" and scale == 1.0 else "tensor"
    p = Problem(rows=1, heads=1, kv_heads=1, head_size=D, v_head_size=D, block_size=B,
                max_blocks_per_row=1, num_pool_blocks=-(-T // B), cache_dtype=cache,
                k_quant=quant, v_quant=quant)
    s = None if quant == "none" else np.array([scale], np.float32)
    vs = None if quant == "none" else np.array([scale * 0.75], np.float32)
    nt = workloads.NewTokens(key=key, value=value, slot_mapping=np.arange(T, dtype=np.int64),
                             k_scale=s, v_scale=vs)
    announce(f"writer every fp16 {cache} scale={scale}")
    _check(p, nt)


def test_zero_tokens_and_all_skipped_leave_the_cache():
    p = Problem(rows=1, heads=8, kv_heads=2, head_size=64, v_head_size=64, block_size=16,
                max_blocks_per_row=4, num_pool_blocks=4, cache_dtype="i8", k_quant="channel",
                v_quant="tensor")
    announce("writer zero tokens / all skipped")
    nt = workloads.new_tokens(p, 5, seed=3, slots=[-1, 64, 1 << 40, -(1 << 40), 65])
    _check(p, nt)
    rng = np.random.default_rng(4)
    kc = _old_cache(rng, (4, 16, 2, 64), "i8")
    vc = _old_cache(rng, (4, 16, 2, 64), "i8")
    dk, dv = _run_writer(p, nt, kc, vc, num_tokens=0)
    assert np.array_equal(_bytes(dk), kc.view(np.uint8).reshape(-1))
    assert np.array_equal(_bytes(dv), vc.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("cache,quant", [("i8", "channel"), ("fp8", "tensor")])
def test_append_then_decode_matches_oracle(cache, quant):
    """One decode step as a server runs it: each row's newest token is
    written through the writer at its slot (block_table[r][t / B] * B + t % B),
    then the step attends over the updated cache.  The oracle does the same
    with its own writer and decode."""
    import torch

    import oracle
    import quantized_paged_kv_amd as pkv
    from tests.gpu_util import assert_close_to_oracle
    from workloads.device import problem_kwargs, to_device

    p = Problem(rows=6, heads=16, kv_heads=2, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=64, num_pool_blocks=1, cache_dtype=cache, k_quant=quant,
                v_quant=quant)
    lens = np.array([1, 17, 300, 511, 64, 1000])
    inp = workloads.make_inputs(p, seed=21, seq_lens=lens)
    p = inp.problem
    B = p.block_size
    pos = lens - 1
    slots = np.array([int(inp.block_table[r, pos[r] // B]) * B + pos[r] % B
                      for r in range(p.rows)], dtype=np.int64)
    nt = workloads.new_tokens(p, p.rows, seed=22, slots=slots)
    # the scales of the cache already in place
    nt.k_scale, nt.v_scale = inp.k_scale, inp.v_scale
    announce(f"writer append+decode {cache} {quant}")

    ref_k, ref_v = cache_write.reshape_and_cache(p, nt.key, nt.value, nt.slot_mapping,
                                                 nt.k_scale, nt.v_scale, inp.key_cache,
                                                 inp.value_cache)
    import dataclasses

    ref_inp = dataclasses.replace(inp, key_cache=ref_k, value_cache=ref_v)
    ref, ref_lse = oracle.paged_decode(ref_inp)

    d = to_device(inp, "cuda")
    prob = pkv.make_problem(**problem_kwargs(p))
    pkv.reshape_and_cache(prob, _dev(nt.key), _dev(nt.value), _dev(nt.slot_mapping),
                          d.k_scale, d.v_scale, d.key_cache, d.value_cache)
    g = pkv.split_geometry(prob)
    ws = pkv.workspace_for(g)
    out = torch.empty((p.rows, p.heads, p.v_head_size), dtype=torch.float16, device="cuda")
    lse = torch.empty((p.rows, p.heads), dtype=torch.float32, device="cuda")
    pkv.paged_decode_attention(prob, g, d.query, d.key_cache, d.value_cache, d.block_table,
                               d.seq_lens, d.candidates, d.num_candidates, d.k_scale, d.v_scale,
                               d.softmax_scale, d.head_sink, out, lse, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(d.key_cache), ref_k.view(np.uint8).reshape(-1))
    assert np.array_equal(_bytes(d.value_cache), ref_v.view(np.uint8).reshape(-1))
    assert_close_to_oracle(out.double().cpu().numpy(), lse.double().cpu().numpy(), ref, ref_lse,
                           what="append+decode")


@pytest.mark.parametrize("cache,quant", [("i8", "channel"), ("fp8", "tensor")])
def test_graph_replay_write_then_decode(cache, quant):
    """A serving loop's step captured once in a HIP graph -- the writer puts
    each row's newest token at its slot, then the decode attends over the
    updated cache -- and replayed for four consecutive steps with new tokens,
    new slots and lengths grown by one.  After every replay the caches are
    bit-exact the oracle writer's (applied step after step) and the output
    meets the oracle's decode of them at the usual tolerance.

    The new rows are drawn at a tenth of unit deviation (their tenfold
    outliers at unit deviation), so the cache stays the unit-variance data
    the tolerance is stated for: rows at the default deviation saturate at
    the cache's top code, and keys of that size scale up the logit shift
    that folding the key scale into the FP16 query allows (2^-11 of
    scale * sum_d |Q'_d K_d|), which a row of two to five tokens passes on
    to its output almost undamped."""
    import dataclasses

    import torch

    import oracle
    import quantized_paged_kv_amd as pkv
    from tests.gpu_util import assert_close_to_oracle
    from workloads.device import problem_kwargs, to_device

    p = Problem(rows=6, heads=16, kv_heads=2, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=64, num_pool_blocks=1, cache_dtype=cache, k_quant=quant,
                v_quant=quant)
    # the next four positions of every row stay in the last block the row
    # already owns, so the new tokens' slots are the row's own
    lens = np.array([1, 17, 300, 507, 33, 1000])
    inp = workloads.make_inputs(p, seed=23, seq_lens=lens)
    p = inp.problem
    B, KVH, D = p.block_size, p.kv_heads, p.head_size
    d = to_device(inp, "cuda")
    prob = pkv.make_problem(**problem_kwargs(p))
    g = pkv.split_geometry(prob)
    ws = pkv.workspace_for(g)
    out = torch.empty((p.rows, p.heads, p.v_head_size), dtype=torch.float16, device="cuda")
    lse = torch.empty((p.rows, p.heads), dtype=torch.float32, device="cuda")
    dkey = torch.zeros((p.rows, KVH, D), dtype=torch.float16, device="cuda")
    dval = torch.zeros((p.rows, KVH, D), dtype=torch.float16, device="cuda")
    dslots = torch.full((p.rows,), -1, dtype=torch.int64, device="cuda")

    def step():
        pkv.reshape_and_cache(prob, dkey, dval, dslots, d.k_scale, d.v_scale, d.key_cache,
                              d.value_cache)
        pkv.paged_decode_attention(prob, g, d.query, d.key_cache, d.value_cache, d.block_table,
                                   d.seq_lens, d.candidates, d.num_candidates, d.k_scale,
                                   d.v_scale, d.softmax_scale, d.head_sink, out, lse, ws)

    announce(f"graph write+decode {cache} {quant}: capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up: every slot is -1, so the writer skips all rows
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    ref_k, ref_v = inp.key_cache.copy(), inp.value_cache.copy()
    cur = lens.copy()
    for it in range(4):
        cur = cur + 1  # the new token's position is cur - 1
        pos = cur - 1
        slots = np.array([int(inp.block_table[r, pos[r] // B]) * B + pos[r] % B
                          for r in range(p.rows)], dtype=np.int64)
        assert np.all(pos // B < -(-lens // B)) and len(set(slots.tolist())) == p.rows
        nt = workloads.new_tokens(p, p.rows, seed=30 + it, x_std=0.1, slots=slots)
        dkey.copy_(_dev(nt.key))
        dval.copy_(_dev(nt.value))
        dslots.copy_(_dev(slots))
        d.seq_lens.copy_(_dev(cur.astype(np.int32)))
        announce(f"graph write+decode {cache} {quant}: replay {it}")
        graph.replay()
        torch.cuda.synchronize()
        ref_k, ref_v = cache_write.reshape_and_cache(p, nt.key, nt.value, slots, inp.k_scale,
                                                     inp.v_scale, ref_k, ref_v)
        assert np.array_equal(_bytes(d.key_cache), ref_k.view(np.uint8).reshape(-1))
        assert np.array_equal(_bytes(d.value_cache), ref_v.view(np.uint8).reshape(-1))
        ref_inp = dataclasses.replace(inp, key_cache=ref_k, value_cache=ref_v,
                                      seq_lens=cur.astype(np.int32))
        ref, ref_lse = oracle.paged_decode(ref_inp)
        assert_close_to_oracle(out.double().cpu().numpy(), lse.double().cpu().numpy(), ref,
                               ref_lse, what=f"write+decode replay {it}")
