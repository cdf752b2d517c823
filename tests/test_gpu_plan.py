"""paged_attention_decode with its launch plan (the plan kernel's items,
worker descriptors and, where tables share a prefix, groups read once on the
matrix cores): outputs against the oracle's decode, which knows nothing of
plans or groups.

Covers forked candidates of every shape family (MHA and query groups, 16-bit
and fp8, block sizes 16 and 32, groups cut to the 16-row limit), the
library-sized split and fixed 16- and 64-token runs, batches above the
planner's 1024-sequence LDS capacity (state in the workspace), mixed batches
of forked and independent sequences with empty ones, caller-sized
partitions over worker spans of several partitions, and bitwise
reproducibility ("vLLM — 把操作系统的分页搬进 GPU KV cache": core mechanism 3
and case 2 for the sharing; core mechanisms for the table walk)."""
import numpy as np
import pytest

import workloads as W
from oracle.run import OracleRun, check_close
from test_gpu_grouped import CASES

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pt", [0, 16, 64])
@pytest.mark.parametrize("name", list(CASES))
def test_plain_decode_of_shared_prefixes(name, pt):
    from gpu_harness import run_gpu
    wl = CASES[name]
    if pt % wl.block_size:
        pytest.skip("runs are whole blocks")
    got = run_gpu(wl, partition_tokens=pt)
    ref = OracleRun(wl)
    assert np.isfinite(got["out"]).all()
    check_close(got["out"], ref.decode(), wl.kv_dtype)


def _forked(name, index, prompts, n, hq=4, hkv=2, kv="f16", q="f16", bs=16):
    parent = [p for p in range(len(prompts)) for _ in range(n)]
    return W._make(name, index, hq, hkv, 128, kv, q, bs, prompt_lens=prompts, parent=parent)


LARGE = {
    # above the planner's LDS capacity: its per-sequence state lives in the workspace
    "flat_1100_bf16": W._make("flat_1100_bf16", 60, 2, 2, 128, "bf16", "bf16", 16,
                              ctx_lens=(np.random.default_rng(60).integers(1, 120, size=1100)).tolist()),
    "forked_1100_f16": _forked("forked_1100_f16", 61, [16 + (7 * i) % 90 for i in range(275)], 4),
    "forked_1100_fp8_gqa": _forked("forked_1100_fp8_gqa", 62, [40 + (5 * i) % 60 for i in range(275)], 4,
                                   hq=8, hkv=2, kv="fp8e4m3", q="bf16"),
}


@pytest.mark.parametrize("pt", [0, 32])
@pytest.mark.parametrize("name", list(LARGE))
def test_batches_past_the_planner_lds(name, pt):
    from gpu_harness import run_gpu
    wl = LARGE[name]
    got = run_gpu(wl, partition_tokens=pt)
    check_close(got["out"], OracleRun(wl).decode(), wl.kv_dtype)


# Caller-sized partitions over a stream longer than the worker grid: every
# worker streams a span of several partitions in one pass, leaving a record
# at each partition boundary it crosses.  One-block partitions put a
# boundary at the end of every run; one wave per CU makes the spans long.
SPANS = {
    "spans_fp8_gqa4": W.config_c5("fp8e4m3", num_seqs=64, lo=200, hi=1200, hq=8, hkv=2, index=64,
                                  name="spans_fp8_gqa4"),
    "spans_bf16_gqa8": W.config_c5("bf16", num_seqs=40, lo=100, hi=1500, hq=16, hkv=2, index=65,
                                   name="spans_bf16_gqa8"),
    "spans_f16_mha": W._make("spans_f16_mha", 66, 4, 4, 128, "f16", "f16", 16,
                             ctx_lens=np.random.default_rng(66).integers(1, 900, size=48).tolist()),
    "spans_bf16_gqa4_bs32": W._make("spans_bf16_gqa4_bs32", 67, 8, 2, 128, "bf16", "bf16", 32,
                                    ctx_lens=np.random.default_rng(67).integers(1, 2000, size=40).tolist()),
    # 16 query rows per kv head (one part fits the LDS), 2 rows, and head
    # dims 64 and 256 (at 256 the tile staging leaves no room: parts are
    # stored as they finish)
    "spans_bf16_gqa16": W._make("spans_bf16_gqa16", 68, 16, 1, 128, "bf16", "bf16", 16,
                                ctx_lens=np.random.default_rng(68).integers(1, 1500, size=48).tolist()),
    "spans_f16_gqa2_d64": W._make("spans_f16_gqa2_d64", 69, 4, 2, 64, "f16", "f16", 16,
                                  ctx_lens=np.random.default_rng(69).integers(1, 1500, size=48).tolist()),
    "spans_fp8_gqa4_d256_f16q": W._make("spans_fp8_gqa4_d256_f16q", 70, 8, 2, 256, "fp8e4m3", "f16", 16,
                                        ctx_lens=np.random.default_rng(70).integers(1, 1200, size=32).tolist()),
}


@pytest.mark.parametrize("waves", [1, 8])
@pytest.mark.parametrize("pt", [16, 32, 64, 160, 512])
@pytest.mark.parametrize("name", list(SPANS))
def test_partitions_over_worker_spans(name, pt, waves, monkeypatch):
    from gpu_harness import run_gpu
    wl = SPANS[name]
    if pt % wl.block_size:
        pytest.skip("partitions are whole blocks")
    monkeypatch.setenv("PAGEDKV_DECODE_WAVES_PER_CU", str(waves))   # read when the pool is made
    got = run_gpu(wl, partition_tokens=pt)
    assert np.isfinite(got["out"]).all()
    check_close(got["out"], _ref(wl), wl.kv_dtype)


_REFS = {}


def _ref(wl):
    if wl.name not in _REFS:
        _REFS.clear()
        _REFS[wl.name] = OracleRun(wl).decode()
    return _REFS[wl.name]


def test_mixed_batch_with_empty_contexts():
    """Forked groups between independent sequences, some contexts empty:
    empty rows are zero, the rest match the oracle."""
    import torch
    from gpu_harness import announce, run_gpu
    wl = _forked("mixed_f16", 63, [95, 30, 200, 17, 64, 5], 3)
    announce("mixed batch with empty contexts")
    got = run_gpu(wl)
    sess, q = got["session"], got["q"]
    lens = sess.context_lens.clone()
    empty = [1, 7, 8, 17]
    lens[empty] = 0
    out = __import__("paged_kv_cache_449_amd").paged_attention_decode(sess.pool, q, sess.block_tables, lens, wl.scale)
    torch.cuda.synchronize()
    got2 = out.float().cpu().double().numpy()
    assert not got2[empty].any()
    keep = [s for s in range(wl.num_seqs) if s not in empty]
    check_close(got2[keep], OracleRun(wl).decode()[keep], wl.kv_dtype)


@pytest.mark.parametrize("name", ["c4s_cow_f16", "gqa4_fp8", "many_groups_f16"])
def test_grouped_plans_are_bitwise_reproducible(name):
    from gpu_harness import run_gpu
    got = run_gpu(CASES[name], partition_tokens=16, repeat=3)
    for o in got["outs"][1:]:
        assert np.array_equal(o, got["outs"][0])


@pytest.mark.parametrize("name,pt", [("c3s_bf16_bs16", 0), ("c4s_cow_f16", 0), ("c4s_cow_f16", 16),
                                     ("c5s_fp8", 512), ("c5s_fp8", 0), ("c1_tiny_f32", 0)])
def test_one_plan_serves_every_layer(name, pt):
    """paged_attention_plan once, then paged_attention_decode_planned for
    several 'layers' -- other queries, and a second pool of the same shape
    read through the same tables -- each bit-identical to the one-call
    paged_attention_decode of that layer."""
    import torch
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce, run_gpu
    wl = W.small_configs()[name]
    got = run_gpu(wl, partition_tokens=pt)
    sess, q = got["session"], got["q"]
    announce(f"one plan, several layers: {name} pt={pt}")
    pool = sess.pool
    pool2 = pk.KVPool(pool.num_blocks, pool.block_size, pool.num_kv_heads, pool.head_dim, pool.dtype, pool.device,
                      pool.k_scale, pool.v_scale)
    if pool.dtype == torch.float8_e4m3fn:   # flip the sign bit: an exact, different layer
        pool2.k_cache.view(torch.uint8).copy_(pool.k_cache.view(torch.uint8) ^ 0x80)
        pool2.v_cache.view(torch.uint8).copy_(pool.v_cache.view(torch.uint8) ^ 0x80)
    else:
        pool2.k_cache.copy_(-pool.k_cache)
        pool2.v_cache.copy_(pool.v_cache * 2)
    bt, cl = sess.block_tables, sess.context_lens
    layers = [(pool, q), (pool, (-q).contiguous()), (pool2, q), (pool2, (q * 2).contiguous())]
    ws = pk.paged_attention_plan(pool, q, bt, cl, partition_tokens=pt)
    planned = [pk.paged_attention_decode_planned(pl, qq, bt, cl, wl.scale, ws, partition_tokens=pt)
               for pl, qq in layers]
    torch.cuda.synchronize()
    for (pl, qq), o in zip(layers, planned):
        ref = pk.paged_attention_decode(pl, qq, bt, cl, wl.scale, partition_tokens=pt)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.uint8), ref.view(torch.uint8))
    check_close(planned[0].float().cpu().double().numpy(), OracleRun(wl).decode(), wl.kv_dtype)


def test_plan_call_checks_its_arguments():
    import torch
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce, device
    announce("plan argument checks")
    dev = device()
    pool = pk.KVPool(8, 16, 2, 64, torch.bfloat16, dev)
    L = pk.lib()
    bt = torch.zeros(2, 1, dtype=torch.int32, device=dev)
    cl = torch.ones(2, dtype=torch.int32, device=dev)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    assert L.paged_attention_plan(pool.handle, pk.KV_BF16, None, 1, cl.data_ptr(), 2, 2, 0, ws.data_ptr(),
                                  ws.numel(), None) == pk.KV_ERR_INVALID_ARG
    assert L.paged_attention_plan(pool.handle, pk.KV_BF16, bt.data_ptr(), 1, cl.data_ptr(), 2, 3, 0, ws.data_ptr(),
                                  ws.numel(), None) == pk.KV_ERR_INVALID_ARG     # 3 q heads over 2 kv heads
    assert L.paged_attention_plan(pool.handle, pk.KV_BF16, bt.data_ptr(), 1, cl.data_ptr(), 2, 2, 0, ws.data_ptr(),
                                  16, None) == pk.KV_ERR_WORKSPACE
    assert L.paged_attention_plan(pool.handle, pk.KV_BF16, bt.data_ptr(), 1, cl.data_ptr(), 2, 2, 0, ws.data_ptr(),
                                  ws.numel(), None) == pk.KV_OK
    torch.cuda.synchronize()
