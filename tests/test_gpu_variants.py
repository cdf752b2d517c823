"""GPU parity of the decode and multi-token paths on the variant workloads:
block sizes 8 and 64, 8:1 query groups, per-kv-head fp8 scales (bf16 and f16
queries, decode and multi-token).  Pools must match the oracle byte for byte,
outputs within the fp8 / 16-bit tolerances; full sizes are checked on sampled
sequences in the configuration the benchmark times."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle.run import OracleRun, check_close

pytestmark = pytest.mark.gpu

SMALL = list(W.small_variant_configs())


@pytest.mark.parametrize("name", SMALL)
def test_variant_matches_oracle(name):
    from gpu_harness import run_gpu, run_gpu_prefill
    wl = W.small_variant_configs()[name]
    got = run_gpu_prefill(wl) if wl.multi_token else run_gpu(wl)
    ref = OracleRun(wl)
    assert np.array_equal(got["k"], ref.pool.k), "K pool bytes differ"
    assert np.array_equal(got["v"], ref.pool.v), "V pool bytes differ"
    want = ref.prefill() if wl.multi_token else ref.decode()
    assert np.isfinite(got["out"]).all()
    check_close(got["out"], want, wl.kv_dtype)


@pytest.mark.parametrize("pt", [16, 512])
def test_head_scales_with_splits(pt):
    from gpu_harness import run_gpu
    wl = W.small_variant_configs()["c5s_fp8_headscale"]
    check_close(run_gpu(wl, partition_tokens=pt)["out"], OracleRun(wl).decode(), wl.kv_dtype)


def test_head_scale_arguments():
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce
    announce("head scale arguments")
    dev = torch.device("cuda", 0)
    pool = pk.KVPool(4, 16, 2, 64, torch.float8_e4m3fn, dev)
    L = pk.lib()
    k = torch.ones(2, dtype=torch.float32, device=dev)
    assert L.kv_pool_set_head_scales(pool.handle, k.data_ptr(), None, None) == pk.KV_ERR_INVALID_ARG
    assert L.kv_pool_set_head_scales(pool.handle, None, k.data_ptr(), None) == pk.KV_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        pk.kv_pool_set_head_scales(pool, [1.0, 0.0], [1.0, 1.0])
    with pytest.raises(ValueError):
        pk.kv_pool_set_head_scales(pool, [1.0, float("nan")], [1.0, 1.0])
    pk.kv_pool_set_head_scales(pool, [1.0, 2.0], [0.5, 0.25])
    pk.kv_pool_set_head_scales(pool, None, None)
    bf = pk.KVPool(4, 16, 2, 64, torch.bfloat16, dev)
    assert L.kv_pool_set_head_scales(bf.handle, k.data_ptr(), k.data_ptr(), None) == pk.KV_ERR_INVALID_ARG


def test_head_scales_follow_stream_order():
    """Per-head scale updates are ordered with the attention calls on one
    stream: doubling every V scale (an exact power of two) doubles the output
    bit for bit, and restoring the scales, with no synchronisation between,
    restores the output."""
    import paged_kv_cache_449_amd as pk
    from gpu_harness import run_gpu
    wl = W.small_variant_configs()["c5s_fp8_headscale"]
    got = run_gpu(wl, partition_tokens=16)
    sess, q = got["session"], got["q"]
    ks, vs = W.fp8_head_scales(wl)
    outs = []
    for vmul in (2.0, 1.0, 4.0):
        pk.kv_pool_set_head_scales(sess.pool, ks, vs * vmul)
        outs.append(sess.attend(q, partition_tokens=16, scale=wl.scale))
    torch.cuda.synchronize()
    base = torch.from_numpy(got["out"]).to(torch.bfloat16)
    assert torch.equal(outs[1].cpu(), base)
    assert torch.equal(outs[0].cpu(), (base.float() * 2).to(torch.bfloat16))
    assert torch.equal(outs[2].cpu(), (base.float() * 4).to(torch.bfloat16))


@pytest.mark.parametrize("name", ["c5s_gqa16_bf16", "c5s_gqa16_fp8_f16"])
@pytest.mark.parametrize("pt", [0, 16])
def test_sixteen_query_heads_per_kv_head(name, pt):
    """16 query heads per kv head fill the 16 rows of a matrix-core tile."""
    from gpu_harness import run_gpu
    wl = W.small_variant_configs()[name]
    check_close(run_gpu(wl, partition_tokens=pt)["out"], OracleRun(wl).decode(), wl.kv_dtype)


def test_sixteen_query_heads_need_the_matrix_cores(monkeypatch):
    """The vector-ALU run holds at most 8 query rows per kv head, so a pool
    made with the matrix cores switched off rejects 16:1 decode."""
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce
    announce("16:1 without matrix cores")
    monkeypatch.setenv("PAGEDKV_DECODE_MFMA", "0")
    dev = torch.device("cuda", 0)
    pool = pk.KVPool(8, 16, 1, 128, torch.bfloat16, dev)
    q = torch.zeros(2, 16, 128, dtype=torch.bfloat16, device=dev)
    tables = torch.zeros(2, 1, dtype=torch.int32, device=dev)
    lens = torch.ones(2, dtype=torch.int32, device=dev)
    with pytest.raises(pk.PagedKVError) as e:
        pk.paged_attention_decode(pool, q, tables, lens, 0.1)
    assert e.value.status == pk.KV_ERR_UNSUPPORTED


@pytest.mark.slow
@pytest.mark.parametrize("name", list(W.variant_configs()))
def test_variant_full_size_every_sequence(name):
    from gpu_harness import run_gpu
    from test_gpu_full import check_all
    wl = W.variant_configs()[name]
    check_all(wl, run_gpu(wl))
