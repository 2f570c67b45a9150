"""Host threads calling the library at once, each on its own HIP stream with
its own workspace and outputs: the library's only shared state is the
per-device CU-count and occupancy cache (behind a mutex) and its error text
is per thread, so every call must give bitwise what the same call gives
alone, and meet the oracle.  Serving processes issue decode steps of
different batches from several threads and streams this way (the
PagedAttention page's operator runs on the caller's stream)."""
import threading

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import announce, assert_close_to_oracle
from workloads import Problem

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(61)
    out = []
    # four KV heads per CTA, FP16
    p = Problem(rows=16, heads=32, kv_heads=8, head_size=128, v_head_size=128, block_size=16,
                max_blocks_per_row=64, num_pool_blocks=0, cache_dtype="f16")
    out.append(workloads.make_inputs(p, 61, rng.integers(0, 1025, size=16), with_sink=True,
                                     softmax_scale=1 / np.sqrt(128)))
    # one KV head per CTA, INT8 per-channel, head 256
    p = Problem(rows=3, heads=24, kv_heads=2, head_size=256, v_head_size=256, block_size=16,
                max_blocks_per_row=128, num_pool_blocks=0, cache_dtype="i8", k_quant="channel",
                v_quant="channel")
    out.append(workloads.make_inputs(p, 62, [2048, 700, 1], softmax_scale=0.0625))
    # gathered candidates
    nc = 300
    p = Problem(rows=8, heads=24, kv_heads=2, head_size=256, v_head_size=256, block_size=16,
                max_blocks_per_row=64, num_pool_blocks=0, max_candidates=nc, cache_dtype="i8",
                k_quant="channel", v_quant="channel")
    out.append(workloads.make_inputs(p, 63, 1024, candidates=rng.integers(-2, 1026, size=(8, nc)),
                                     num_candidates=rng.integers(0, nc + 1, size=8),
                                     softmax_scale=0.0625))
    # latent FP8
    p = Problem(rows=8, heads=16, kv_heads=1, head_size=576, v_head_size=512, block_size=64,
                max_blocks_per_row=16, num_pool_blocks=0, cache_dtype="fp8", k_quant="tensor",
                v_quant="tensor", layout="latent")
    out.append(workloads.make_inputs(p, 64, rng.integers(0, 1025, size=8), with_sink=True,
                                     softmax_scale=1 / 24))
    return out


def _run(inp, d, stream, reps):
    """`reps` decode steps of `inp` on `stream` with a geometry, workspace and
    outputs of this call's own; returns (out, lse, num_splits)."""
    import torch

    import quantized_paged_kv_amd as pkv

    prob = pkv.make_problem(**d.problem_kwargs)
    g = pkv.split_geometry(prob)
    p = inp.problem
    with torch.cuda.stream(stream):
        ws = pkv.workspace_for(g)
        out = torch.full((p.rows, p.heads, p.v_head_size), float("nan"), dtype=torch.float16,
                         device="cuda")
        lse = torch.full((p.rows, p.heads), float("nan"), dtype=torch.float32, device="cuda")
        for _ in range(reps):
            pkv.paged_decode_attention(prob, g, d.query, d.key_cache, d.value_cache,
                                       d.block_table, d.seq_lens, d.candidates, d.num_candidates,
                                       d.k_scale, d.v_scale, d.softmax_scale, d.head_sink, out,
                                       lse, ws, stream=stream)
    stream.synchronize()
    return out.cpu(), lse.cpu(), g.num_splits


def test_threads_on_their_own_streams():
    import torch

    import quantized_paged_kv_amd as pkv
    from workloads.device import to_device

    inputs = _cases()
    devs = [to_device(inp, "cuda") for inp in inputs]
    torch.cuda.synchronize()
    n_threads = 2 * len(inputs)  # two threads per problem
    start = threading.Barrier(n_threads + 1)
    results = [None] * n_threads
    errors = []

    def worker(i):
        try:
            k = i % len(inputs)
            stream = torch.cuda.Stream()
            start.wait(timeout=60)
            if i == 0:
                # an error in one thread leaves the others' calls and text alone
                bad = pkv.make_problem(4, 8, 2, 96, 96, 16, 8, 64)
                with pytest.raises(pkv.PkvError) as e:
                    pkv.split_geometry(bad)
                assert "96" in str(e.value)
            results[i] = _run(inputs[k], devs[k], stream, reps=5)
        except BaseException as e:  # noqa: BLE001 -- re-raised below
            errors.append((i, e))

    announce(f"{n_threads} threads, {len(inputs)} problems, one stream each")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    start.wait(timeout=60)
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors

    for k, inp in enumerate(inputs):
        alone = _run(inp, devs[k], torch.cuda.current_stream(), reps=1)
        ref, ref_lse = oracle.paged_decode(inp)
        for i in range(k, n_threads, len(inputs)):
            out, lse, S = results[i]
            assert S == alone[2]
            assert torch.equal(out, alone[0]) and torch.equal(lse, alone[1]), f"problem {k} thread {i}"
        assert_close_to_oracle(alone[0].double().numpy(), alone[1].double().numpy(), ref, ref_lse,
                               what=f"problem {k}")
