"""Exact code conversion on the GPU.

The PagedAttention page ("Summary of Changes", the int8 -> fp16 fast path)
calls its conversion bit identical, and the INT8 DynamicSparseAttention page
("Summary of Changes" section 1) converts the codes exactly to FP16 before
the FP16 MFMAs.  Rows with one token make every other step exact, so the
outputs expose the conversion itself:

* V side: with one token p = 1 and l = 1, so O[c] = code(c) * v_scale[c],
  one FP32 rounding of an exact product;
* K side: a one-hot query (1 in channel c, softmax scale 1, key scale a power
  of two) gives the logit code(c) * k_scale exactly, and lse = logit.

Every INT8 code and every finite e4m3fn code appears in every channel
position of V across the rows, and under every query head on the K side;
each compiled kernel family (one KV head per CTA with head 256, four or eight
KV heads per CTA with head 128, the latent kernel with its direct-to-LDS
ring) runs with one split (direct output) and with four (the combine)."""
import numpy as np
import pytest

import oracle
import workloads
from workloads import Inputs, Problem
from tests.gpu_util import announce, run_gpu

pytestmark = pytest.mark.gpu


def _codes(cache):
    if cache == "i8":
        return np.arange(-128, 128, dtype=np.int64)
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.int64)


def _value(cache, codes):
    if cache == "i8":
        return codes.astype(np.float64)
    return np.array([oracle.fp8e4m3_to_f64(int(c)) for c in codes])


def _store(cache, codes):
    return codes.astype(np.int8) if cache == "i8" else codes.astype(np.uint8)


def one_token_rows(cache, D, VD, layout, kvh, heads, quant):
    """n one-token rows (n = number of codes); returns inputs and the exact
    expected (out, lse)."""
    C = _codes(cache)
    n = len(C)
    group = heads // kvh
    latent = layout == "latent"
    d = np.arange(D)
    kc = np.empty((n, 16, kvh, D), dtype=np.int64)
    kc[...] = C[0]
    q = np.zeros((n, heads, D), dtype=np.float16)
    hot = np.zeros((n, heads), dtype=np.int64)
    for r in range(n):
        for g in range(kvh):
            kc[r, 0, g] = C[(r + 3 * g + d) % n]
            for h in range(g * group, (g + 1) * group):
                c = (7 * h + r) % D
                hot[r, h] = c
                kc[r, 0, g, c] = C[(r + h) % n]
                q[r, h, c] = 1.0
    if latent:
        vc = None
    else:
        vc = np.empty((n, 16, kvh, VD), dtype=np.int64)
        vc[...] = C[0]
        cc = np.arange(VD)
        for r in range(n):
            for g in range(kvh):
                vc[r, 0, g] = C[(r + 5 * g + 2 * cc + 1) % n]
    rng = np.random.default_rng(17)
    if quant == "tensor":
        ks = np.array([1.0], np.float32)
        vs = np.array([0.0371], np.float32)
    else:
        ks = np.full((kvh, D), 0.125, np.float32)
        vs = rng.uniform(0.005, 0.05, (kvh, VD)).astype(np.float32)
    if latent:
        vs = ks
    p = Problem(rows=n, heads=heads, kv_heads=kvh, head_size=D, v_head_size=VD, block_size=16,
                max_blocks_per_row=4, num_pool_blocks=n, cache_dtype=cache, k_quant=quant,
                v_quant=quant, layout=layout, out_dtype="f32")
    inp = Inputs(problem=p, query=q, key_cache=_store(cache, kc),
                 value_cache=None if latent else _store(cache, vc),
                 block_table=np.tile(np.arange(n, dtype=np.int32)[:, None], (1, 4)),
                 seq_lens=np.ones(n, np.int32), softmax_scale=1.0, k_scale=ks,
                 v_scale=None if latent else vs)
    # exact expectations
    kval = _value(cache, C)
    lse = np.empty((n, heads))
    out = np.empty((n, heads, VD), dtype=np.float32)
    ksg = np.broadcast_to(ks.reshape(-1, D) if quant == "channel" else ks[0], (kvh, D))
    vsg = np.broadcast_to(vs.reshape(-1, vs.size // kvh if quant == "channel" else 1)
                          if quant == "channel" else vs[0], (kvh, VD if not latent else D))
    pos = {int(c): i for i, c in enumerate(C)}
    for r in range(n):
        for h in range(heads):
            g = h // group
            c = hot[r, h]
            lse[r, h] = kval[pos[int(kc[r, 0, g, c])]] * float(ksg[g, c])
            row = kc[r, 0, g, :VD] if latent else vc[r, 0, g]
            vals = np.array([kval[pos[int(x)]] for x in row])
            out[r, h] = (vals * vsg[g, :VD].astype(np.float64)).astype(np.float32)
    return inp, out, lse


SHAPES = [(256, 256, "separate", 2, 24, 0), (128, 128, "separate", 8, 32, 4),
          (128, 128, "separate", 8, 32, 8), (576, 512, "latent", 1, 16, 0)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"D{s[0]}-{s[2]}-kpc{s[5]}")
@pytest.mark.parametrize("cache", ["i8", "fp8"])
@pytest.mark.parametrize("quant", ["tensor", "channel"])
def test_every_code_converts_exactly(shape, cache, quant):
    D, VD, layout, kvh, heads, kpc = shape
    inp, out, lse = one_token_rows(cache, D, VD, layout, kvh, heads, quant)
    ref, ref_lse = oracle.paged_decode(inp)
    # the oracle agrees with the closed form (exact decode of every code)
    assert np.array_equal(ref_lse, lse)
    assert np.array_equal(ref.astype(np.float32), out)
    for S in (1, 4):
        announce(f"exact codes {cache} {quant} D={D} {layout} kpc={kpc} S={S}")
        geo = dict(splits_override=S, min_chunk=16)
        if kpc:
            geo["kv_heads_per_cta"] = kpc
        got, got_lse, g = run_gpu(inp, **geo)
        assert g.num_splits == S
        bad = np.argwhere(got.astype(np.float32) != out)
        assert bad.size == 0, f"V side: {len(bad)} mismatches, first at {bad[0]}"
        badk = np.argwhere(got_lse != lse)
        assert badk.size == 0, f"K side: {len(badk)} mismatches, first at {badk[0]}"
