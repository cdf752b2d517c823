"""The allocation-free decode entry point (paged_attention_decode_noalloc),
called through the C ABI, against paged_attention_decode on the same inputs:
two calls in a row on one device's scratch area, the second with a smaller
batch, each bit-identical to the workspace call and within the oracle's
tolerance; and a shape that needs more than the area is refused."""
import ctypes

import numpy as np
import pytest
import torch

import bench
import workloads as W
from oracle.run import OracleRun, check_close

pytestmark = pytest.mark.gpu


def _noalloc(pk, pool, q, tables, lens, scale, out, pt):
    L = pk.lib()
    st = L.paged_attention_decode_noalloc(pool.handle, q.data_ptr(), pk.DTYPE_CODE[q.dtype], out.data_ptr(),
                                          tables.data_ptr(), tables.shape[1], lens.data_ptr(), q.shape[0],
                                          q.shape[1], ctypes.c_float(scale), pt,
                                          torch.cuda.current_stream().cuda_stream)
    return st


@pytest.mark.parametrize("name,pt", [("c3s_bf16_bs16", 0), ("c5s_fp8", 16), ("c4s_cow_f16", 0)])
def test_noalloc_matches_workspace_call(name, pt):
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce, device
    announce(f"noalloc {name} pt={pt}")
    wl = W.small_configs()[name]
    dev = device()
    sess, q, kn, vn = bench.build_session(wl, dev)
    ref = sess.step(q, kn, vn, partition_tokens=pt, scale=wl.scale)
    torch.cuda.synchronize(dev)
    want = OracleRun(wl).decode()
    tables, lens = sess.block_tables, sess.context_lens
    # call 1: the whole batch; call 2: a smaller batch (its first sequences)
    for k in (wl.num_seqs, max(1, wl.num_seqs // 2)):
        qk, tk, lk = q[:k].contiguous(), tables[:k].contiguous(), lens[:k].contiguous()
        out = torch.full_like(qk, float("nan"))
        assert _noalloc(pk, sess.pool, qk, tk, lk, wl.scale, out, pt) == pk.KV_OK
        base = pk.paged_attention_decode(sess.pool, qk, tk, lk, wl.scale, partition_tokens=pt)
        torch.cuda.synchronize(dev)
        assert torch.equal(out.view(torch.uint8), base.view(torch.uint8)), k
        if k == wl.num_seqs:
            assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8))
        check_close(out.float().cpu().double().numpy(), want[:k], wl.kv_dtype)


def test_noalloc_refuses_shapes_past_its_area():
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce, device
    announce("noalloc size limit")
    dev = device()
    pool = pk.KVPool(64, 16, 8, 128, torch.bfloat16, dev)
    S, Hq, mb = 64, 64, 32
    need = pk.paged_attention_workspace_size(pool, S, Hq, mb, 16)
    assert need > pk.DECODE_SCRATCH_BYTES
    q = torch.zeros(S, Hq, 128, dtype=torch.bfloat16, device=dev)
    out = torch.zeros_like(q)
    tables = torch.zeros(S, mb, dtype=torch.int32, device=dev)
    lens = torch.ones(S, dtype=torch.int32, device=dev)
    assert _noalloc(pk, pool, q, tables, lens, 0.1, out, 16) == pk.KV_ERR_WORKSPACE
    torch.cuda.synchronize(dev)
    assert not out.any()   # nothing was enqueued
