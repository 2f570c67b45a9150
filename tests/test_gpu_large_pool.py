"""Pools larger than 4 GiB per cache: small problems whose pool blocks are
moved to the top of a cache of more than 2^32 bytes (the block table
follows them), so every kernel's byte offsets into the pool need more than
32 bits.  The decode results are compared with the oracle of the small
problem (the values are the same); the cache writer is checked bit-exactly
against the oracle's writer at slots past 2^32 bytes.

A pool of this size is what a serving process holds (the PagedAttention
page's cache is one pre-allocated pool shared by all sequences); the blocks
below the moved ones are never written, so an offset that lost its high
bits would read other memory of the same allocation and fail the
comparison."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, assert_close_to_oracle
from workloads import Problem

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32


def _lift_cache(c, top, big):
    import torch

    if c is None:
        return None
    out = torch.empty((big,) + tuple(c.shape[1:]), dtype=c.dtype, device=c.device)
    out[top:].copy_(c)
    return out


def _lifted(d):
    """The device inputs with the pool moved up by `top` blocks, `top` chosen
    so the first moved block starts 256 MiB past 4 GiB."""
    import torch

    nb = int(d.key_cache.shape[0])
    blk_bytes = d.key_cache[0].numel() * d.key_cache.element_size()
    top = -(-(FOUR_GIB + (256 << 20)) // blk_bytes)
    big = top + nb
    bt = d.block_table
    valid = (bt >= 0) & (bt < nb)
    lifted_bt = torch.where(valid, bt + top, torch.where(bt >= nb, bt - nb + big, bt))
    return (_lift_cache(d.key_cache, top, big), _lift_cache(d.value_cache, top, big),
            lifted_bt.contiguous(), big, top)


def _decode_lifted(inp, **geo):
    import torch

    import quantized_paged_kv_amd as pkv
    from workloads.device import to_device

    d = to_device(inp, "cuda")
    kc, vc, bt, big, top = _lifted(d)
    assert top * d.key_cache[0].numel() * d.key_cache.element_size() > FOUR_GIB
    kw = dict(d.problem_kwargs, num_pool_blocks=big)
    prob = pkv.make_problem(**kw)
    g = pkv.split_geometry(prob, **geo)
    ws = pkv.workspace_for(g)
    p = inp.problem
    qrows = p.rows * max(1, p.query_tokens)
    out = torch.full((qrows, p.heads, p.v_head_size), float("nan"), dtype=torch.float16,
                     device="cuda")
    lse = torch.full((qrows, p.heads), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_decode_attention(prob, g, d.query, kc, vc, bt, d.seq_lens, d.candidates,
                               d.num_candidates, d.k_scale, d.v_scale, d.softmax_scale,
                               d.head_sink, out, lse, ws)
    torch.cuda.synchronize()
    res = out.double().cpu().numpy(), lse.double().cpu().numpy(), g
    del kc, vc, d, ws
    torch.cuda.empty_cache()
    return res


# (name, problem, gathered, query tokens): one case per kernel family
CASES = {
    # four KV heads per CTA (the continuous-batching shape, FP16)
    "kvp_f16": (dict(heads=32, kv_heads=8, head_size=128, v_head_size=128, block_size=16,
                     cache_dtype="f16", k_quant="none", v_quant="none"), False, 1),
    # one KV head per CTA, dense INT8 per-channel, head 256
    "split_i8": (dict(heads=24, kv_heads=2, head_size=256, v_head_size=256, block_size=16,
                      cache_dtype="i8", k_quant="channel", v_quant="channel"), False, 1),
    # gathered candidates, INT8 per-channel, head 256
    "gathered_i8": (dict(heads=24, kv_heads=2, head_size=256, v_head_size=256, block_size=16,
                         cache_dtype="i8", k_quant="channel", v_quant="channel"), True, 1),
    # the absorbed-MLA latent layout, FP8
    "latent_fp8": (dict(heads=16, kv_heads=1, head_size=576, v_head_size=512, block_size=64,
                        cache_dtype="fp8", k_quant="tensor", v_quant="tensor",
                        layout="latent"), False, 1),
    # gathered latent rows, FP16
    "latent_gathered_f16": (dict(heads=16, kv_heads=1, head_size=576, v_head_size=512,
                                 block_size=64, cache_dtype="f16", k_quant="none",
                                 v_quant="none", layout="latent"), True, 1),
    # eight query tokens per row (two head blocks per wave), FP8
    "multitoken_fp8": (dict(heads=32, kv_heads=8, head_size=128, v_head_size=128,
                            block_size=16, cache_dtype="fp8", k_quant="tensor",
                            v_quant="tensor"), False, 8),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("S", [0, 3])
def test_decode_over_a_pool_past_4gib(name, S):
    kw, gathered, T = CASES[name]
    rows, ctx = 3, 1024
    nc = 200 if gathered else 0
    p = Problem(rows=rows, max_blocks_per_row=ctx // kw["block_size"], num_pool_blocks=0,
                max_candidates=nc, query_tokens=T, **kw)
    rng = np.random.default_rng(31)
    lens = np.array([ctx, 517, 1])
    cand = ncand = None
    if gathered:
        cand = rng.integers(-2, ctx + 2, size=(rows, nc)).astype(np.int32)
        ncand = np.array([nc, 77, 5])
    inp = workloads.make_inputs(p, 31, lens, with_sink=True, candidates=cand,
                                num_candidates=ncand, softmax_scale=1.0 / np.sqrt(p.head_size))
    ref_inp = workloads.expand_query_tokens(inp) if T > 1 else inp
    ref, ref_lse = oracle.paged_decode(ref_inp)
    geo = dict(splits_override=S, min_chunk=16) if S else {}
    announce(f"pool past 4 GiB: {name} S={S or 'auto'}")
    got, lse, g = _decode_lifted(inp, **geo)
    if S:
        assert g.num_splits == S
    assert_close_to_oracle(got, lse, ref, ref_lse, what=f"{name} pool past 4 GiB S={S}")


@pytest.mark.parametrize("cache,quant,lay", [("i8", "channel", "separate"),
                                             ("fp8", "tensor", "latent"),
                                             ("f16", "none", "separate")])
def test_writer_into_a_pool_past_4gib(cache, quant, lay):
    """Slots past 2^32 bytes of the cache: the written rows are bit-exact the
    oracle writer's at the same slots of the small pool, and nothing else of
    the moved region changes."""
    import torch

    import quantized_paged_kv_amd as pkv
    from oracle import cache_write
    from workloads.device import problem_kwargs

    latent = lay == "latent"
    D, VD = (576, 512) if latent else (128, 128)
    KVH = 1 if latent else 4
    B, nb = 16, 64
    p = Problem(rows=1, heads=KVH * 4, kv_heads=KVH, head_size=D, v_head_size=VD, block_size=B,
                max_blocks_per_row=nb, num_pool_blocks=nb, cache_dtype=cache, k_quant=quant,
                v_quant="none" if latent else quant, layout=lay)
    rng = np.random.default_rng(41)
    slots = rng.permutation(nb * B)[:300].astype(np.int64)
    nt = workloads.new_tokens(p, len(slots), seed=42, slots=slots)
    kc = np.zeros((nb, B, KVH, D), dtype=workloads.code_dtype(cache))
    vc = None if latent else np.zeros((nb, B, KVH, VD), dtype=workloads.code_dtype(cache))
    ref_k, ref_v = cache_write.reshape_and_cache(p, nt.key, nt.value, nt.slot_mapping,
                                                 nt.k_scale, nt.v_scale, kc, vc)

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.float16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
        return torch.from_numpy(a).cuda()

    dk0, dv0 = dev(kc), dev(vc)
    blk_bytes = dk0[0].numel() * dk0.element_size()
    top = -(-(FOUR_GIB + (256 << 20)) // blk_bytes)
    big = top + nb
    dk, dv = _lift_cache(dk0, top, big), _lift_cache(dv0, top, big)
    prob = pkv.make_problem(**dict(problem_kwargs(p), num_pool_blocks=big))
    announce(f"writer into a pool past 4 GiB: {cache} {quant} {lay}")
    pkv.reshape_and_cache(prob, dev(nt.key), dev(nt.value), dev(nt.slot_mapping + top * B),
                          dev(nt.k_scale), dev(nt.v_scale), dk, dv)
    torch.cuda.synchronize()

    def top_bytes(t):
        return t[top:].cpu().contiguous().view(-1).view(torch.uint8).numpy()

    assert np.array_equal(top_bytes(dk), ref_k.view(np.uint8).reshape(-1)), "key cache differs"
    if dv is not None:
        assert np.array_equal(top_bytes(dv), ref_v.view(np.uint8).reshape(-1)), "value cache differs"
    del dk, dv
    torch.cuda.empty_cache()
