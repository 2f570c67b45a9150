"""Pins for the FP64 oracle: each check ties it to something other than itself.

* exact decoding: library conversions (numpy float16, torch float8_e4m3fn) and
  exact rational arithmetic (fractions.Fraction);
* brute force: an independent pure-Python softmax attention (math.fsum, the
  caches decoded with numpy / torch) on tiny inputs of every storage type,
  quantisation, layout and row kind;
* a special case that reduces to a library routine (torch softmax in float64);
* invariants and closed forms (rows sum to one, a single token, equal keys,
  split = monolithic, head-sink closed form = an extra zero-value logit,
  block-table permutation leaves every bit unchanged, empty rows);
* the worked numerical examples printed on the pages (tests/golden).
"""
import math
import os
from dataclasses import replace
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Inputs, Problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# exact decoding
# ---------------------------------------------------------------------------

def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(ref[~both_nan], got[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(got))


def test_fp8_e4m3fn_decode_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8e4m3_to_f64(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    # OCP e4m3fn anchor points: largest finite 448, smallest normal 2^-6,
    # smallest subnormal 2^-9, one, minus one, NaN only at S.1111.111
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x38] == 1.0 and got[0xB8] == -1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and int(np.isnan(got).sum()) == 2


@pytest.mark.parametrize("scale", [1.0, 0.0625, 0.0347, 3.0e-3, 2.0 ** -135, 2.0 ** 60, 1.7e38])
def test_int8_dequant_exact(scale):
    s32 = float(np.float32(scale))
    for code in range(256):
        signed = code - 256 if code >= 128 else code
        exact = Fraction(signed) * Fraction(s32)
        assert Fraction(oracle.dequant("i8", code, s32)) == exact


def test_fp8_dequant_exact():
    for s in (1.0, 0.0101, 2.0 ** -20):
        s32 = float(np.float32(s))
        for code in range(256):
            v = oracle.fp8e4m3_to_f64(code)
            if math.isnan(v):
                continue
            assert Fraction(oracle.dequant("fp8", code, s32)) == Fraction(v) * Fraction(s32)


# ---------------------------------------------------------------------------
# independent brute force (pure Python, fsum)
# ---------------------------------------------------------------------------

def _decode_cache(codes, cache_dtype):
    if cache_dtype == "f16":
        return codes.astype(np.float64)
    if cache_dtype == "i8":
        return codes.astype(np.int8).astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _scale(scale, quant, g, dim):
    if quant == "none":
        return np.ones(dim)
    if quant == "tensor":
        return np.full(dim, float(scale[0]))
    return np.asarray(scale, dtype=np.float64).reshape(-1, dim)[g]


def brute_force(inp: Inputs):
    p = inp.problem
    K = _decode_cache(inp.key_cache, p.cache_dtype)
    V = None if p.layout == "latent" else _decode_cache(inp.value_cache, p.cache_dtype)
    q = inp.query.astype(np.float64)
    group = p.heads // p.kv_heads
    out = np.zeros((p.rows, p.heads, p.v_head_size))
    lse = np.zeros((p.rows, p.heads))
    for r in range(p.rows):
        n = min(max(int(inp.seq_lens[r]), 0), p.max_blocks_per_row * p.block_size)
        if p.max_candidates:
            nc = min(max(int(inp.num_candidates[r]), 0), p.max_candidates)
            toks = [int(c) for c in inp.candidates[r, :nc] if 0 <= c < n]
        else:
            toks = list(range(n))
        for h in range(p.heads):
            g = h // group
            ks = _scale(inp.k_scale, p.k_quant, g, p.head_size)
            if p.layout == "latent":
                vs = ks[: p.v_head_size]
            else:
                vs = _scale(inp.v_scale, p.v_quant, g, p.v_head_size)
            krows, vrows, xs = [], [], []
            for t in toks:
                blk = int(inp.block_table[r, t // p.block_size])
                off = t % p.block_size
                k = K[blk, off, g, :] * ks
                if p.layout == "latent":
                    v = K[blk, off, g, : p.v_head_size] * vs
                else:
                    v = V[blk, off, g, :] * vs
                xs.append(inp.softmax_scale * math.fsum(q[r, h, d] * k[d] for d in range(p.head_size)))
                vrows.append(v)
            if not toks:
                out[r, h] = 0.0
                lse[r, h] = -math.inf
                continue
            m = max(xs)
            w = [math.exp(x - m) for x in xs]
            L = math.fsum(w)
            for c in range(p.v_head_size):
                out[r, h, c] = math.fsum(w[i] * vrows[i][c] for i in range(len(toks))) / L
            lse[r, h] = m + math.log(L)
            if inp.head_sink is not None:
                out[r, h] *= 1.0 / (1.0 + math.exp(float(inp.head_sink[h]) - lse[r, h]))
    return out, lse


TINY_CASES = [
    # cache, kq, vq, layout, gathered, sink, heads, kvh, D, VD, B
    ("f16", "none", "none", "separate", False, False, 4, 1, 8, 8, 4),
    ("f16", "none", "none", "separate", False, True, 6, 2, 8, 4, 2),
    ("i8", "tensor", "tensor", "separate", False, False, 4, 2, 8, 8, 4),
    ("i8", "channel", "channel", "separate", True, True, 6, 3, 4, 8, 2),
    ("i8", "channel", "tensor", "separate", True, False, 2, 2, 8, 8, 1),
    ("fp8", "tensor", "tensor", "separate", False, True, 4, 2, 8, 8, 4),
    ("fp8", "channel", "channel", "separate", True, False, 4, 1, 8, 4, 2),
    ("fp8", "tensor", "tensor", "latent", False, False, 4, 1, 8, 4, 4),
    ("i8", "channel", "channel", "latent", True, True, 3, 1, 8, 6, 2),
    ("f16", "none", "none", "latent", False, True, 2, 1, 8, 4, 8),
]


def _tiny(case, seed):
    cache, kq, vq, layout, gathered, sink, H, KVH, D, VD, B = case
    rng = np.random.default_rng(seed)
    rows, mbpr = 3, 3
    lens = rng.integers(0, mbpr * B + 3, size=rows)  # includes 0 and > capacity
    lens[0] = max(lens[0], 1)
    p = Problem(rows=rows, heads=H, kv_heads=KVH, head_size=D, v_head_size=VD, block_size=B,
                max_blocks_per_row=mbpr, num_pool_blocks=0,
                max_candidates=6 if gathered else 0, cache_dtype=cache, k_quant=kq,
                v_quant=vq, layout=layout)
    cand = None
    if gathered:
        # invalid entries (negative, beyond the length), duplicates, unsorted
        cand = rng.integers(-2, mbpr * B + 2, size=(rows, 6)).astype(np.int32)
        cand[0, :2] = [1, 1]
    inp = workloads.make_inputs(p, seed, lens, candidates=cand, with_sink=sink,
                                num_candidates=None if not gathered else np.array([6, 4, 0][:rows]),
                                softmax_scale=0.37)
    return inp


@pytest.mark.parametrize("case", TINY_CASES)
@pytest.mark.parametrize("seed", [11, 12])
def test_brute_force_tiny(case, seed):
    inp = _tiny(case, seed)
    o, l = oracle.paged_decode(inp, threads=2)
    bo, bl = brute_force(inp)
    assert np.array_equal(np.isinf(l), np.isinf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(l[fin], bl[fin], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-14)


def test_dense_case_equals_torch_softmax():
    """Group 1, identity block table, one block per row: the definition
    reduces to softmax(q k^T * scale) v, evaluated by torch in float64."""
    T, D = 37, 16
    p = Problem(rows=2, heads=3, kv_heads=3, head_size=D, v_head_size=D, block_size=T,
                max_blocks_per_row=1, num_pool_blocks=2, cache_dtype="f16")
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 3, D)).astype(np.float16)
    k = rng.standard_normal((2, T, 3, D)).astype(np.float16)
    v = rng.standard_normal((2, T, 3, D)).astype(np.float16)
    inp = Inputs(problem=p, query=q, key_cache=k, value_cache=v,
                 block_table=np.array([[0], [1]], dtype=np.int32),
                 seq_lens=np.array([T, T], dtype=np.int32), softmax_scale=0.29)
    o, l = oracle.paged_decode(inp)
    for r in range(2):
        for h in range(3):
            qq = torch.from_numpy(q[r, h].astype(np.float64))
            kk = torch.from_numpy(k[r, :, h].astype(np.float64))
            vv = torch.from_numpy(v[r, :, h].astype(np.float64))
            ref = torch.softmax(kk @ qq * 0.29, dim=0) @ vv
            np.testing.assert_allclose(o[r, h], ref.numpy(), rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(l[r, h], torch.logsumexp(kk @ qq * 0.29, 0).item(), rtol=1e-14)


# ---------------------------------------------------------------------------
# invariants and closed forms
# ---------------------------------------------------------------------------

def _small(cache="f16", seed=3, lens=(45, 1, 64, 17), sink=False, **kw):
    kq = vq = "none" if cache == "f16" else "tensor"
    p = Problem(rows=len(lens), heads=4, kv_heads=2, head_size=16, v_head_size=16, block_size=16,
                max_blocks_per_row=4, num_pool_blocks=0, cache_dtype=cache, k_quant=kq,
                v_quant=vq, **kw)
    return workloads.make_inputs(p, seed, list(lens), with_sink=sink, softmax_scale=0.25)


def test_rows_sum_to_one():
    inp = _small()
    inp.value_cache[...] = np.float16(1.0)
    o, _ = oracle.paged_decode(inp)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-15)


def test_single_token_returns_its_value_exactly():
    inp = _small(lens=(1, 1, 1, 1))
    o, l = oracle.paged_decode(inp)
    B = inp.problem.block_size
    for r in range(4):
        blk = inp.block_table[r, 0]
        for h in range(4):
            v = inp.value_cache[blk, 0, h // 2].astype(np.float64)
            assert np.array_equal(o[r, h], v)


def test_equal_keys_give_the_mean_value():
    inp = _small(lens=(45, 7, 64, 17))
    inp.key_cache[...] = inp.key_cache[inp.block_table[0, 0], 0]
    o, _ = oracle.paged_decode(inp)
    for r in range(4):
        n = int(inp.seq_lens[r])
        for h in range(4):
            vals = []
            for t in range(n):
                blk = inp.block_table[r, t // 16]
                vals.append(inp.value_cache[blk, t % 16, h // 2].astype(np.float64))
            np.testing.assert_allclose(o[r, h], np.mean(vals, axis=0), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("chunk", [1, 7, 16, 64, 4096])
@pytest.mark.parametrize("cache", ["f16", "i8"])
def test_split_equals_monolithic(chunk, cache):
    inp = _small(cache=cache, sink=True, lens=(45, 1, 64, 0))
    o0, l0 = oracle.paged_decode(inp)
    o1, l1 = oracle.paged_decode(inp, chunk=chunk)
    np.testing.assert_allclose(o1, o0, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1[np.isfinite(l0)], l0[np.isfinite(l0)], rtol=1e-13)
    assert np.array_equal(np.isinf(l0), np.isinf(l1))


def test_head_sink_equals_extra_zero_value_logit():
    inp = _small(sink=True)
    o, l = oracle.paged_decode(inp)
    base = replace(inp.problem)
    plain = Inputs(**{**inp.__dict__, "head_sink": None, "problem": base})
    o0, l0 = oracle.paged_decode(plain)
    for r in range(4):
        for h in range(4):
            s = float(inp.head_sink[h])
            # softmax over the row's logits plus one extra logit s with value 0
            denom = math.exp(l0[r, h]) + math.exp(s)
            expect = o0[r, h] * math.exp(l0[r, h]) / denom
            np.testing.assert_allclose(o[r, h], expect, rtol=1e-14, atol=1e-16)
            assert l[r, h] == l0[r, h]  # lse is reported before the sink


def test_block_table_permutation_is_bitwise_invariant():
    inp = _small(cache="i8", sink=True)
    o0, l0 = oracle.paged_decode(inp)
    pool = inp.problem.num_pool_blocks
    perm = np.random.default_rng(9).permutation(pool)  # new id of each old block
    k2 = np.empty_like(inp.key_cache)
    v2 = np.empty_like(inp.value_cache)
    k2[perm] = inp.key_cache
    v2[perm] = inp.value_cache
    moved = Inputs(**{**inp.__dict__, "key_cache": k2, "value_cache": v2,
                      "block_table": perm[inp.block_table].astype(np.int32)})
    o1, l1 = oracle.paged_decode(moved)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_empty_and_clamped_rows():
    inp = _small(lens=(0, 64, 1000, -5))
    o, l = oracle.paged_decode(inp)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    assert np.all(o[3] == 0) and np.all(np.isneginf(l[3]))
    # a length beyond the capacity is clamped to it (64 tokens here)
    inp2 = Inputs(**{**inp.__dict__, "seq_lens": np.array([0, 64, 64, -5], dtype=np.int32)})
    o2, l2 = oracle.paged_decode(inp2)
    assert np.array_equal(o2[2], o[2]) and np.array_equal(l2[2], l[2])


def test_all_candidates_invalid_gives_empty_row():
    p = Problem(rows=1, heads=2, kv_heads=1, head_size=8, v_head_size=8, block_size=4,
                max_blocks_per_row=2, num_pool_blocks=0, max_candidates=3, cache_dtype="f16")
    inp = workloads.make_inputs(p, 1, 5, candidates=np.array([[-1, 5, 9]], dtype=np.int32))
    o, l = oracle.paged_decode(inp)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_bad_block_id_is_an_error():
    inp = _small()
    inp.block_table[1, 0] = inp.problem.num_pool_blocks
    with pytest.raises(RuntimeError):
        oracle.paged_decode(inp)


# ---------------------------------------------------------------------------
# the pages' worked examples
# ---------------------------------------------------------------------------

def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_worked_examples(row):
    (name, q0, q1, ka0, ka1, kb0, kb1, va, vb, vscale, sscale, expected, rtol,
     printed, printed_tol) = row
    D = 256
    p = Problem(rows=1, heads=1, kv_heads=1, head_size=D, v_head_size=D, block_size=16,
                max_blocks_per_row=1, num_pool_blocks=1, max_candidates=2, cache_dtype="i8",
                k_quant="tensor", v_quant="tensor", out_dtype="f32")
    q = np.zeros((1, 1, D), dtype=np.float16)
    q[0, 0, 0], q[0, 0, 1] = np.float16(float(q0)), np.float16(float(q1))
    assert float(q[0, 0, 0]) == float(q0) and float(q[0, 0, 1]) == float(q1)
    k = np.zeros((1, 16, 1, D), dtype=np.int8)
    v = np.zeros((1, 16, 1, D), dtype=np.int8)
    # candidate a at token 3, candidate b at token 11 (same 16-token block)
    k[0, 3, 0, :2] = [int(ka0), int(ka1)]
    k[0, 11, 0, :2] = [int(kb0), int(kb1)]
    v[0, 3, 0, 0], v[0, 11, 0, 0] = int(va), int(vb)
    vs = np.float32(float(vscale))
    assert float(vs) == float(vscale)
    inp = Inputs(problem=p, query=q, key_cache=k, value_cache=v,
                 block_table=np.zeros((1, 1), dtype=np.int32), seq_lens=np.array([16], np.int32),
                 softmax_scale=float(sscale), k_scale=np.array([1.0], np.float32),
                 v_scale=np.array([vs], np.float32), candidates=np.array([[3, 11]], np.int32),
                 num_candidates=np.array([2], np.int32))
    o, _ = oracle.paged_decode(inp)
    got = o[0, 0, 0]
    assert got == pytest.approx(float(expected), rel=float(rtol), abs=0)
    if printed != "-":
        assert abs(got - float(printed)) <= float(printed_tol)
    assert np.all(o[0, 0, 1:] == 0)


def folding_case():
    """The query-folding rounding case of the INT8 DynamicSparseAttention page
    ("Numerics", first row of the review-case table), built with numbers of
    our own: per-channel key scales make the products Q0 ks0 = 32768 and
    Q1 ks1 = -32766, which FP16 rounds to 32768 and -32768.  Token 0 has key
    codes (1, 1), token 1 zeros; at softmax scale 8 the exact logits are 16
    and 0, so output channel 0 (value code 1 on token 0) is 1 / (1 + e^-16);
    the folded FP16 query would give 0.5.  Returns (inputs, expected)."""
    D = 256
    p = Problem(rows=1, heads=1, kv_heads=1, head_size=D, v_head_size=D, block_size=16,
                max_blocks_per_row=1, num_pool_blocks=1, cache_dtype="i8",
                k_quant="channel", v_quant="channel", out_dtype="f32")
    q = np.zeros((1, 1, D), dtype=np.float16)
    q[0, 0, 0], q[0, 0, 1] = 2048.0, -2048.0
    ks = np.ones((1, D), dtype=np.float32)
    ks[0, 0], ks[0, 1] = 16.0, 16383.0 / 1024.0
    assert float(np.float32(2048.0) * ks[0, 1]) == 32766.0
    k = np.zeros((1, 16, 1, D), dtype=np.int8)
    v = np.zeros((1, 16, 1, D), dtype=np.int8)
    k[0, 0, 0, :2] = [1, 1]
    v[0, 0, 0, 0] = 1
    inp = Inputs(problem=p, query=q, key_cache=k, value_cache=v,
                 block_table=np.zeros((1, 1), dtype=np.int32), seq_lens=np.array([2], np.int32),
                 softmax_scale=8.0, k_scale=ks, v_scale=np.ones((1, D), np.float32))
    return inp, 1.0 / (1.0 + math.exp(-16.0))


def test_folding_case_closed_form():
    inp, expected = folding_case()
    out, lse = oracle.paged_decode(inp)
    assert out[0, 0, 0] == pytest.approx(expected, rel=1e-13)
    assert np.all(out[0, 0, 1:] == 0)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(16.0) + 1.0), rel=1e-13)


# ---------------------------------------------------------------------------
# quantise-on-write (ONNX Runtime PR #29912, ReshapeAndCache with slot_mapping)
# ---------------------------------------------------------------------------

from oracle import cache_write  # noqa: E402


def test_fp8_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 1, 20000) * np.exp2(rng.integers(-12, 9, 20000)),
                        [0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -9 * 1.5, 1.0625, 1.1875,
                         447.0, 460.0, -463.9]])
    v = v[np.abs(v) < 464].astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = cache_write.fp8_e4m3fn_encode(v)
    assert np.array_equal(got, ref)


def test_fp8_encode_saturates_and_round_trips():
    got = cache_write.fp8_e4m3fn_encode(np.array([464.0, 480.0, 1e30, -500.0, np.inf]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = np.array([oracle.fp8e4m3_to_f64(c) for c in finite])
    assert np.array_equal(cache_write.fp8_e4m3fn_encode(vals), np.array(finite, np.uint8))


def test_int8_encode_rounds_half_even_and_clips():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-140, 140, 5000), np.arange(-130.5, 131, 0.5)]).astype(np.float32)
    ref = np.array([min(127, max(-128, round(float(x)))) for x in v], dtype=np.int8)
    assert np.array_equal(cache_write.int8_encode(v), ref)


def test_reshape_and_cache_writes_only_mapped_slots():
    p = Problem(rows=1, heads=4, kv_heads=2, head_size=64, v_head_size=64, block_size=16,
                max_blocks_per_row=4, num_pool_blocks=4, cache_dtype="i8", k_quant="channel",
                v_quant="tensor")
    rng = np.random.default_rng(2)
    kc = rng.integers(-128, 128, (4, 16, 2, 64)).astype(np.int8)
    vc = rng.integers(-128, 128, (4, 16, 2, 64)).astype(np.int8)
    key = rng.normal(0, 1, (5, 2, 64)).astype(np.float16)
    val = rng.normal(0, 1, (5, 2, 64)).astype(np.float16)
    ks = rng.uniform(0.005, 0.05, (2, 64)).astype(np.float32)
    vs = np.array([0.03], np.float32)
    slots = np.array([3, -1, 63, 64, 17], np.int64)
    k2, v2 = cache_write.reshape_and_cache(p, key, val, slots, ks, vs, kc, vc)
    written = {3: 0, 63: 2, 17: 4}
    for b in range(4):
        for o in range(16):
            slot = b * 16 + o
            if slot in written:
                t = written[slot]
                exp_k = np.clip(np.rint(key[t].astype(np.float32) / ks), -128, 127)
                exp_v = np.clip(np.rint(val[t].astype(np.float32) / np.float32(0.03)), -128, 127)
                assert np.array_equal(k2[b, o], exp_k.astype(np.int8))
                assert np.array_equal(v2[b, o], exp_v.astype(np.int8))
            else:
                assert np.array_equal(k2[b, o], kc[b, o]) and np.array_equal(v2[b, o], vc[b, o])


# ---------------------------------------------------------------------------
# sliding window and logit soft cap (ONNX Runtime PR #29912, "Summary of
# Changes": the paged decode kernel supports both; readings: a window of W
# keeps positions [len - W, len), the cap maps a scaled logit x to
# c tanh(x / c))
# ---------------------------------------------------------------------------

def _windowed(inp, W):
    return Inputs(**{**inp.__dict__, "problem": replace(inp.problem, sliding_window=W)})


def test_window_wider_than_the_row_changes_nothing():
    inp = _small(cache="i8", sink=True, lens=(45, 1, 64, 17))
    o0, l0 = oracle.paged_decode(inp)
    o1, l1 = oracle.paged_decode(_windowed(inp, 64))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_of_one_returns_the_newest_value():
    inp = _windowed(_small(lens=(45, 1, 64, 17)), 1)
    o, l = oracle.paged_decode(inp)
    for r in range(4):
        t = int(inp.seq_lens[r]) - 1
        blk = inp.block_table[r, t // 16]
        for h in range(4):
            assert np.array_equal(o[r, h], inp.value_cache[blk, t % 16, h // 2].astype(np.float64))


def test_window_equals_the_row_started_at_its_first_block():
    """A window that starts on a block boundary attends exactly what a row
    whose table begins at that block attends: outputs are bitwise equal."""
    inp = _small(cache="i8", sink=True, lens=(64, 48, 40, 33))
    W = 32
    win = _windowed(inp, W)
    o1, l1 = oracle.paged_decode(win)
    lens = inp.seq_lens.astype(np.int64)
    for r in range(4):
        lo = max(0, int(lens[r]) - W)
        if lo % 16:
            continue
        bt = np.full_like(inp.block_table, inp.block_table[r, 0])
        nb = inp.block_table.shape[1] - lo // 16
        bt[:, :nb] = inp.block_table[r, lo // 16:]
        shifted = Inputs(**{**inp.__dict__, "block_table": bt,
                            "seq_lens": np.full_like(inp.seq_lens, int(lens[r]) - lo)})
        o2, l2 = oracle.paged_decode(shifted, rows=[r])
        assert np.array_equal(o1[r], o2[r]) and np.array_equal(l1[r], l2[r])


def test_window_ignores_positions_before_it():
    """Poisoning every position before the window (NaN values, extreme keys)
    leaves the output bitwise unchanged."""
    inp = _small(cache="f16", lens=(64, 50, 37, 20))
    W = 19
    o0, l0 = oracle.paged_decode(_windowed(inp, W))
    k2, v2 = inp.key_cache.copy(), inp.value_cache.copy()
    for r in range(4):
        for t in range(max(0, int(inp.seq_lens[r]) - W)):
            blk = inp.block_table[r, t // 16]
            k2[blk, t % 16] = np.float16(60000.0)
            v2[blk, t % 16] = np.float16(np.nan)
    bad = Inputs(**{**inp.__dict__, "key_cache": k2, "value_cache": v2,
                    "problem": replace(inp.problem, sliding_window=W)})
    o1, l1 = oracle.paged_decode(bad)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_on_candidate_lists_filters_them():
    """Gathered rows: the window equals dropping the candidates before it."""
    p = Problem(rows=2, heads=4, kv_heads=1, head_size=16, v_head_size=16, block_size=16,
                max_blocks_per_row=8, num_pool_blocks=0, max_candidates=12, cache_dtype="i8",
                k_quant="channel", v_quant="tensor")
    rng = np.random.default_rng(5)
    cand = np.stack([rng.permutation(128)[:12] for _ in range(2)]).astype(np.int32)
    inp = workloads.make_inputs(p, 5, [128, 100], candidates=cand)
    W = 40
    o1, l1 = oracle.paged_decode(_windowed(inp, W))
    c2 = cand.copy()
    n2 = np.zeros(2, np.int32)
    for r in range(2):
        lo = int(inp.seq_lens[r]) - W
        keep = [c for c in cand[r] if lo <= c < int(inp.seq_lens[r])]
        c2[r, :len(keep)] = keep
        c2[r, len(keep):] = -1
        n2[r] = len(keep)
    o2, l2 = oracle.paged_decode(Inputs(**{**inp.__dict__, "candidates": c2, "num_candidates": n2}))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _two_token_case(x0, x1, cap):
    """One head, two tokens whose scaled logits are x0 and x1 (set by one-hot
    keys against a query of ones, softmax scale 1); value channel 0 is 1 on
    token 0 and 0 on token 1, so O[0] is token 0's weight."""
    D = 16
    p = Problem(rows=1, heads=1, kv_heads=1, head_size=D, v_head_size=D, block_size=16,
                max_blocks_per_row=1, num_pool_blocks=1, cache_dtype="f16", out_dtype="f32",
                softcap=cap)
    q = np.zeros((1, 1, D), dtype=np.float16)
    q[0, 0, :2] = 1.0
    k = np.zeros((1, 16, 1, D), dtype=np.float16)
    v = np.zeros((1, 16, 1, D), dtype=np.float16)
    k[0, 0, 0, 0], k[0, 1, 0, 1] = x0, x1
    v[0, 0, 0, 0] = 1.0
    return Inputs(problem=p, query=q, key_cache=k, value_cache=v,
                  block_table=np.zeros((1, 1), np.int32), seq_lens=np.array([2], np.int32),
                  softmax_scale=1.0)


def test_softcap_closed_form():
    """Cap 2 with logits 2 atanh(1/2) and 0 gives capped logits exactly 1 and
    0: token 0's weight is 1 / (1 + e^-1) and lse = log(e + 1).  Capping
    before the scale, or c tanh(x) without the division, gives other values."""
    x0 = float(np.float16(2.0 * math.atanh(0.5)))
    inp = _two_token_case(x0, 0.0, 2.0)
    o, l = oracle.paged_decode(inp)
    y = 2.0 * math.tanh(x0 / 2.0)  # x0 is the FP16-rounded logit: y is within 1e-3 of 1
    assert abs(y - 1.0) < 1e-3
    assert o[0, 0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-y)), rel=1e-14)
    assert l[0, 0] == pytest.approx(math.log(math.exp(y) + 1.0), rel=1e-14)
    assert o[0, 0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), abs=3e-4)


def test_softcap_bounds_and_limits():
    # a huge logit is held under the cap: lse < cap + log 2
    o, l = oracle.paged_decode(_two_token_case(60000.0, -60000.0, 30.0))
    assert l[0, 0] < 30.0 + math.log(2.0)
    assert o[0, 0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-60.0)), rel=1e-12)
    # a cap far above the logits changes them by at most x^3 / (3 c^2)
    inp = _small(cache="i8", lens=(45, 1, 64, 17))
    o0, l0 = oracle.paged_decode(inp)
    capped = Inputs(**{**inp.__dict__, "problem": replace(inp.problem, softcap=1e4)})
    o1, l1 = oracle.paged_decode(capped)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-6)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-6)
    # and a binding cap does change them
    tight = Inputs(**{**inp.__dict__, "problem": replace(inp.problem, softcap=0.5)})
    o2, _ = oracle.paged_decode(tight)
    assert np.abs(o2 - o0).max() > 1e-3


# ---------------------------------------------------------------------------
# the quantise-on-write quotient and codes against exact rational arithmetic
# (reading: the quotient x / scale is rounded once to FP32, then encoded)
# ---------------------------------------------------------------------------

from fractions import Fraction  # noqa: E402


def _round_to_format(q: Fraction, mant_bits: int, emin: int, vmax: Fraction, sat: bool):
    """Nearest value of a binary format to the rational q, ties to an even
    significand: mant_bits fraction bits, smallest normal exponent emin
    (subnormals below it), largest finite vmax; beyond it +-inf (sat=False,
    past the halfway point to the next binade) or +-vmax (sat=True)."""
    if q == 0:
        return Fraction(0)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, emin) - mant_bits)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v > vmax:
        if sat:
            v = vmax
        else:
            return Fraction(-1 if neg else 1) * 10 ** 60  # stands for infinity
    return -v if neg else v


def rn32(q):
    return _round_to_format(q, 23, -126, Fraction(2 ** 24 - 1, 2 ** 23) * 2 ** 127, False)


def rn16(q):
    return _round_to_format(q, 10, -14, Fraction(65504), False)


def rn_e4m3fn(q):
    return _round_to_format(q, 3, -6, Fraction(448), True)


def _frac_to_float(v: Fraction) -> float:
    return math.copysign(math.inf, v) if abs(v) >= 10 ** 59 else float(v)


def _expected_code(x16, s32, cache):
    """The code of one element from the exact quotient: RN32(x / s), then
    INT8: clip(round half even) / FP8: nearest e4m3fn, ties even, saturating
    / FP16: RN16."""
    q = rn32(Fraction(float(x16)) / Fraction(float(s32)))
    if cache == "i8":
        n = q.numerator // q.denominator
        rem = q - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
            n += 1
        return min(127, max(-128, n))
    if cache == "fp8":
        v = rn_e4m3fn(q)
        mag = abs(v)
        code = int(np.nonzero(cache_write._FP8_VALS == float(mag))[0][0])
        return code | (0x80 if (v < 0 or (v == 0 and q < 0)) else 0)
    v = _frac_to_float(rn16(q))
    # a quotient that rounds to zero keeps its sign (IEEE)
    return math.copysign(0.0, float(x16) / float(s32)) if v == 0 else v


def _writer_samples(seed, n):
    rng = np.random.default_rng(seed)
    x = (rng.normal(0, 1, n) * np.exp2(rng.integers(-20, 12, n))).astype(np.float16)
    x = x[np.isfinite(x)]
    s = (rng.uniform(0.5, 1.0, len(x)) * np.exp2(rng.integers(-30, 20, len(x)))).astype(np.float32)
    return x, s


def test_rational_rounding_helpers_against_numpy_casts():
    """The Fraction-based rounding agrees with IEEE casts of doubles on
    values where those are single roundings (a double holds every product
    and sum used here exactly)."""
    rng = np.random.default_rng(3)
    v = rng.normal(0, 1, 3000) * np.exp2(rng.integers(-160, 130, 3000))
    for x in v:
        assert _frac_to_float(rn32(Fraction(float(x)))) == float(np.float32(x))
    w = rng.normal(0, 1, 3000) * np.exp2(rng.integers(-26, 17, 3000))
    for x in w:
        if abs(x) < 65520:
            assert _frac_to_float(rn16(Fraction(float(x)))) == float(np.float16(x))


@pytest.mark.parametrize("cache", ["i8", "fp8", "f16"])
def test_writer_codes_from_the_exact_quotient(cache):
    """quantize() equals the definition evaluated in exact rationals: the
    quotient x / scale rounded once to FP32, then encoded.  Sampled inputs
    over wide exponent ranges, plus quotients that are exact ties: of INT8
    codes (k + 1/2), of FP8 values, of FP16 values, and FP32 ties in the
    subnormal range (the only FP32 ties a FP16 / FP32 quotient can hit)."""
    x, s = _writer_samples(11, 1500)
    extra_x = [2.5, -3.5, 0.5, -0.5, 126.5, -127.5, 1.0625, 1.1875, 2.0 ** -7 * 3, 1 + 2 ** -11,
               3 * 2 ** -24, -3 * 2 ** -24, 5 * 2 ** -24]
    extra_s = [1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 2.0 ** 126, 2.0 ** 126,
               2.0 ** 126]
    x = np.concatenate([x, np.array(extra_x, np.float16)])
    s = np.concatenate([s, np.array(extra_s, np.float32)])
    got = cache_write.quantize(x, s, cache)
    for i in range(len(x)):
        exp = _expected_code(x[i], s[i], cache)
        if cache == "f16":
            g = float(got[i])
            assert g == exp or (math.isnan(g) and math.isnan(exp)), (x[i], s[i], g, exp)
            assert math.copysign(1, g) == math.copysign(1, exp) or g != 0
        elif cache == "fp8":
            assert int(got[i]) == exp, (x[i], s[i], int(got[i]), exp)
        else:
            assert int(got[i]) == exp, (x[i], s[i], int(got[i]), exp)


def test_writer_fp32_subnormal_quotient_ties():
    """3 * 2^-24 (an FP16 subnormal) / 2^126 = 1.5 * 2^-149 lies halfway
    between the two smallest FP32 subnormals; rounding half to even gives
    2^-148, and 5 * 2^-24 / 2^126 = 2.5 * 2^-149 gives 2^-148 as well."""
    for num in (3, 5):
        q = rn32(Fraction(num * 2 ** -24) / Fraction(2 ** 126))
        assert q == Fraction(2) ** -148
        v = np.float16(num * 2 ** -24).astype(np.float32) / np.float32(2.0 ** 126)
        assert float(v) == 2.0 ** -148


def test_writer_fp16_branch_against_torch():
    """The FP16-cache branch against torch's float32 division and half
    cast (a library routine), over sampled inputs and every finite FP16
    value under three scales."""
    x, s = _writer_samples(12, 20000)
    allx = workloads.every_fp16_value()
    allx = allx[np.isfinite(allx)]
    for xs, ss in ((x, s), (allx, np.float32(0.37)), (allx, np.float32(3.0e-5)),
                   (allx, np.float32(7.5))):
        ref = (torch.from_numpy(xs.astype(np.float32)) / torch.from_numpy(
            np.broadcast_to(np.asarray(ss, np.float32), xs.shape).copy())).half().numpy()
        got = cache_write.quantize(xs, ss, "f16")
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def test_writer_fp16_double_rounding_is_the_stated_reading():
    """Rounding the FP32 quotient to FP16 (the reading taken) is not always
    rounding the exact quotient to FP16: when RN32(x / s) lands on an FP16
    midpoint that the exact quotient misses, the two differ.  Find such
    inputs and check that quantize() follows the FP32-first reading there."""
    rng = np.random.default_rng(5)
    found = 0
    for _ in range(4000):
        x = np.float16(rng.uniform(1, 2) * 2.0 ** int(rng.integers(-3, 4)))
        # an FP16 midpoint T near x / s, and an FP32 scale s = RN32(x / T)
        # nudged by a few ulps so that x / s straddles T by less than an FP32
        # half-ulp
        y = rn16(Fraction(float(x)) / Fraction(float(rng.uniform(0.7, 1.4))))
        ulp16 = Fraction(2) ** (max(y.numerator.bit_length() - y.denominator.bit_length(), -14) - 10)
        T = y + ulp16 / 2
        s0 = np.float32(float(Fraction(float(x)) / T))
        for k in range(-3, 4):
            s = np.float32(s0 + k * np.spacing(s0))
            q = Fraction(float(x)) / Fraction(float(s))
            if rn32(q) == T and q != T:
                exact = _frac_to_float(rn16(q))
                twice = _frac_to_float(rn16(rn32(q)))
                if exact != twice:
                    found += 1
                    got = float(cache_write.quantize(np.array([x]), s, "f16")[0])
                    assert got == twice and got != exact
        if found >= 3:
            break
    assert found >= 3


# ---------------------------------------------------------------------------
# several query tokens per row
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 3, 8])
def test_multitoken_rows_are_causal_attention(T):
    """Several query tokens per row (the DSA page's decode tests take 1, 3
    and 8 query rows of one sequence): token j of a row of length len sees
    the positions [0, len - T + 1 + j) of that row (none when that is not
    positive), through the row's one block table.  Brute force over the
    definition, independent of the expansion into separate rows that the
    GPU tests compare against."""
    p = Problem(rows=3, heads=4, kv_heads=2, head_size=8, v_head_size=8, block_size=4,
                max_blocks_per_row=3, num_pool_blocks=0, cache_dtype="i8", k_quant="tensor",
                v_quant="channel", query_tokens=T)
    lens = [12, 5, 2]  # full capacity, a row shorter than 8 tokens, one shorter than 3
    inp = workloads.make_inputs(p, 60 + T, lens, with_sink=True, softmax_scale=0.37)
    o, l = oracle.paged_decode(workloads.expand_query_tokens(inp), threads=2)
    K = _decode_cache(inp.key_cache, p.cache_dtype)
    V = _decode_cache(inp.value_cache, p.cache_dtype)
    q = inp.query.astype(np.float64)
    group = p.heads // p.kv_heads
    cap = p.max_blocks_per_row * p.block_size
    assert o.shape == (p.rows * T, p.heads, p.v_head_size)
    for r in range(p.rows):
        for j in range(T):
            n = max(0, min(lens[r], cap) - (T - 1 - j))
            qi = r * T + j
            for h in range(p.heads):
                g = h // group
                ks = _scale(inp.k_scale, p.k_quant, g, p.head_size)
                vs = _scale(inp.v_scale, p.v_quant, g, p.v_head_size)
                if n == 0:
                    assert math.isinf(l[qi, h]) and l[qi, h] < 0 and np.all(o[qi, h] == 0)
                    continue
                xs, vrows = [], []
                for t in range(n):
                    blk = int(inp.block_table[r, t // p.block_size])
                    k = K[blk, t % p.block_size, g, :] * ks
                    xs.append(inp.softmax_scale * math.fsum(q[qi, h, d] * k[d] for d in range(p.head_size)))
                    vrows.append(V[blk, t % p.block_size, g, :] * vs)
                m = max(xs)
                w = [math.exp(x - m) for x in xs]
                L = math.fsum(w)
                lse = m + math.log(L)
                sink = 1.0 / (1.0 + math.exp(float(inp.head_sink[h]) - lse))
                exp_o = [math.fsum(w[i] * vrows[i][c] for i in range(n)) / L * sink
                         for c in range(p.v_head_size)]
                assert abs(l[qi, h] - lse) <= 1e-12 * max(1.0, abs(lse))
                np.testing.assert_allclose(o[qi, h], exp_o, rtol=1e-12, atol=1e-14)
