"""GPU edge cases: number formats, degenerate lengths, every supported shape
family, host-side error statuses, and workspace reuse across calls."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.run import OracleRun, check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    import paged_kv_cache_449_amd as pk
    return pk


@pytest.fixture(scope="module")
def gpu():
    from gpu_harness import run_gpu
    return run_gpu


def _dev():
    return torch.device("cuda", 0)


def test_fp8_codes_decode_exactly(pk):
    """All 256 E4M3FN codes read back through decode with a one-token
    context: out = decode(code) * v_scale exactly (p = 1, l = 1)."""
    from gpu_harness import announce
    announce("fp8 codes")
    dev = _dev()
    pool = pk.KVPool(4, 16, 2, 128, torch.float8_e4m3fn, dev, 1.0, 1.0)
    pool.k_cache.view(torch.uint8).zero_()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128)
    pool.v_cache.view(torch.uint8)[3, :, 0, :] = codes.to(dev)
    q = torch.randn(1, 2, 128, device=dev)
    bt = torch.tensor([[3]], dtype=torch.int32, device=dev)
    cl = torch.tensor([1], dtype=torch.int32, device=dev)
    out = pk.paged_attention_decode(pool, q, bt, cl, 0.1).cpu().double().numpy()
    want = np.array([oracle.e4m3_to_f64(c) for c in range(256)]).reshape(2, 128)
    np.testing.assert_array_equal(np.isnan(out[0]), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(out[0][ok], want[ok])


@pytest.mark.parametrize("qdt", [torch.bfloat16, torch.float16])
def test_fp8_codes_decode_exactly_on_matrix_cores(pk, qdt):
    """The same exhaustive check with a query group of 2 (matrix-core path,
    where codes are widened to the 16-bit operand type): one-token context,
    so p = 1 and out = decode(code) * v_scale, exactly representable."""
    from gpu_harness import announce
    announce(f"fp8 codes, query group, q {qdt}")
    dev = _dev()
    pool = pk.KVPool(4, 16, 1, 128, torch.float8_e4m3fn, dev, 1.0, 0.5)
    pool.k_cache.view(torch.uint8).zero_()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128)
    for half in range(2):
        pool.v_cache.view(torch.uint8)[2, 0, 0, :] = codes[half].to(dev)
        q = torch.randn(1, 2, 128, device=dev).to(qdt)
        bt = torch.tensor([[2]], dtype=torch.int32, device=dev)
        cl = torch.tensor([1], dtype=torch.int32, device=dev)
        out = pk.paged_attention_decode(pool, q, bt, cl, 0.1).cpu().double().numpy()
        want = np.array([oracle.e4m3_to_f64(c) * 0.5 for c in range(128 * half, 128 * half + 128)])
        for g in range(2):
            np.testing.assert_array_equal(np.isnan(out[0, g]), np.isnan(want))
            ok = ~np.isnan(want)    # every finite code * 0.5 is exact in bf16 and f16
            np.testing.assert_array_equal(out[0, g][ok], want[ok])


def test_fp8_scale_applies_to_values(pk):
    dev = _dev()
    pool = pk.KVPool(2, 16, 1, 128, torch.float8_e4m3fn, dev, 0.5, 0.25)
    pool.k_cache.view(torch.uint8).zero_()
    pool.v_cache.view(torch.uint8).fill_(0x38)      # 1.0
    q = torch.randn(1, 1, 128, device=dev)
    bt = torch.tensor([[1]], dtype=torch.int32, device=dev)
    cl = torch.tensor([5], dtype=torch.int32, device=dev)
    out = pk.paged_attention_decode(pool, q, bt, cl, 0.1).cpu()
    torch.testing.assert_close(out, torch.full_like(out, 0.25), rtol=1e-6, atol=0)


@pytest.mark.parametrize("kv,hq,hkv,pt", [("bf16", 8, 2, 0), ("fp8e4m3", 8, 2, 32), ("f16", 4, 4, 0)])
@pytest.mark.parametrize("scale", [-0.11, 0.0, 0.9])
def test_scale_sign_and_zero(pk, gpu, kv, hq, hkv, pt, scale):
    """The matrix-core runs scale scores inside the exponent and take the row
    max before scaling: a negative scale (q's sign flipped), a zero one
    (every token weighs the same) and a large one match the oracle, on the
    matrix-core (query groups, with and without caller partitions) and the
    vector-ALU path."""
    wl = W._make(f"scale_{kv}_{hq}", 92, hq, hkv, 128, kv, "bf16" if kv != "f16" else "f16", 16,
                 ctx_lens=[300, 45, 7, 130])
    got = gpu(wl, partition_tokens=pt)
    sess, q = got["session"], got["q"]
    out = pk.paged_attention_decode(sess.pool, q, sess.block_tables, sess.context_lens, scale, partition_tokens=pt)
    torch.cuda.synchronize()
    ref = OracleRun(wl)
    want = ref.pool.decode(ref.q, wl.q_dtype, ref.tables, wl.context_lens, scale, wl.num_q_heads)
    check_close(out.float().cpu().double().numpy(), want, wl.kv_dtype)


def test_empty_context_gives_zero_rows(pk):
    wl = W.custom("empty", 4, 4, 128, "f16", "f16", 16, [30, 47, 1, 64], index=91)
    from gpu_harness import run_gpu
    got = run_gpu(wl)
    sess = got["session"]
    q = W.q_values(wl).to(_dev())
    lens = sess.context_lens.clone()
    lens[1] = 0
    out = pk.paged_attention_decode(sess.pool, q, sess.block_tables, lens, wl.scale).cpu().double().numpy()
    assert np.all(out[1] == 0)
    ref = OracleRun(wl).decode([0, 2, 3])
    check_close(out[[0, 2, 3]], ref[[0, 2, 3]], wl.kv_dtype)


def test_context_fills_whole_table(gpu):
    wl = W.custom("full_table", 2, 2, 128, "bf16", "bf16", 16, [64, 48, 17], index=92)
    got = gpu(wl)
    assert got["tables"].shape[1] * 16 == 64
    check_close(got["out"], OracleRun(wl).decode(), wl.kv_dtype)


SHAPES = [
    # name, Hq, Hkv, D, kv, q, bs, lens
    ("d64_bs8_f16", 3, 3, 64, "f16", "f16", 8, [5, 8, 9, 77, 130]),
    ("d64_f32_g2", 4, 2, 64, "f32", "f32", 16, [17, 100, 3]),
    ("d128_f32", 2, 2, 128, "f32", "f32", 32, [33, 250]),
    ("d256_bs64_bf16", 2, 1, 256, "bf16", "bf16", 64, [63, 64, 65, 300]),
    ("d256_f32_g4", 4, 1, 256, "f32", "f32", 16, [40, 161]),
    ("d128_fp8_qf16_g8", 16, 2, 128, "fp8e4m3", "f16", 16, [31, 500, 129]),
    ("d128_fp8_qf32", 2, 2, 128, "fp8e4m3", "f32", 16, [200, 7]),
    ("d256_fp8_g4", 8, 2, 256, "fp8e4m3", "bf16", 32, [100, 401]),
    ("d64_fp8_g2", 4, 2, 64, "fp8e4m3", "bf16", 16, [16, 90, 333]),
    ("d128_bf16_g2_bs8", 4, 2, 128, "bf16", "bf16", 8, [8, 9, 600]),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("pt_blocks", [0, 1, 3])
def test_shape_families(gpu, shape, pt_blocks):
    name, hq, hkv, d, kv, q, bs, lens = shape
    wl = W.custom(name, hq, hkv, d, kv, q, bs, lens, index=93)
    got = gpu(wl, partition_tokens=pt_blocks * bs)
    ref = OracleRun(wl)
    assert np.array_equal(got["k"], ref.pool.k) and np.array_equal(got["v"], ref.pool.v)
    check_close(got["out"], ref.decode(), wl.kv_dtype)


@pytest.mark.parametrize("kv,q,g", [("bf16", "bf16", 4), ("fp8e4m3", "bf16", 8), ("f16", "f16", 2)])
def test_short_contexts_on_matrix_cores(gpu, kv, q, g):
    """Contexts of a few tokens on the matrix-core path: the weights cannot
    average rounding out, so these rows test the precision of P itself."""
    lens = [2, 3, 4, 5, 2, 3, 2, 6, 7, 8, 2, 3, 9, 2, 4, 16, 17, 3, 2, 5] * 3
    wl = W.custom(f"short_{kv}_g{g}", 2 * g, 2, 128, kv, q, 16, lens, index=94)
    check_close(gpu(wl)["out"], OracleRun(wl).decode(), wl.kv_dtype)


def test_host_side_errors(pk):
    dev = _dev()
    pool = pk.KVPool(8, 16, 2, 128, torch.float16, dev)
    L = pk.lib()
    q = torch.zeros(2, 4, 128, dtype=torch.float16, device=dev)
    out = torch.empty_like(q)
    bt = torch.zeros(2, 2, dtype=torch.int32, device=dev)
    cl = torch.ones(2, dtype=torch.int32, device=dev)
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)
    need = pk.paged_attention_workspace_size(pool, 2, 4, 2, 0)
    st = torch.cuda.current_stream().cuda_stream

    def call(qd=pk.KV_F16, hq=4, pt=0, ws_bytes=None, qptr=None, wsptr=None):
        return L.paged_attention_decode(pool.handle, qptr or q.data_ptr(), qd, out.data_ptr(), bt.data_ptr(), 2,
                                        cl.data_ptr(), 2, hq, 0.1, pt, wsptr or ws.data_ptr(),
                                        need if ws_bytes is None else ws_bytes, st)

    assert call() == pk.KV_OK
    assert call(ws_bytes=need - 1) == pk.KV_ERR_WORKSPACE
    assert call(wsptr=ws.data_ptr() + 16) == pk.KV_ERR_WORKSPACE
    assert call(qd=pk.KV_BF16) == pk.KV_ERR_UNSUPPORTED
    assert call(hq=6) == pk.KV_ERR_UNSUPPORTED
    assert call(hq=3) == pk.KV_ERR_INVALID_ARG
    assert call(pt=24) == pk.KV_ERR_INVALID_ARG
    assert call(qptr=q.data_ptr() + 2) == pk.KV_ERR_INVALID_ARG
    assert L.kv_pool_set_scales(pool.handle, 1.0, 1.0) == pk.KV_ERR_INVALID_ARG   # not an fp8 pool
    k = torch.zeros(1, 2, 128, dtype=torch.bfloat16, device=dev)
    slots = torch.zeros(1, dtype=torch.int64, device=dev)
    assert L.reshape_and_cache(pool.handle, k.data_ptr(), k.data_ptr(), pk.KV_BF16, slots.data_ptr(), 1, st) == \
        pk.KV_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_library_owned_pool_roundtrip(pk):
    p = pk.kv_pool_create(32, 16, 4, 64, torch.bfloat16)
    kp, vp = ctypes.c_void_p(), ctypes.c_void_p()
    n = ctypes.c_size_t()
    st = (ctypes.c_int64 * 4)()
    assert pk.lib().kv_pool_info(p.handle, ctypes.byref(kp), ctypes.byref(vp), ctypes.byref(n), st) == 0
    assert n.value == 32 * 4 * 16 * 64 * 2 and kp.value and vp.value
    assert tuple(st) == (4 * 16 * 64, 16 * 64, 64, 1)
    p.close()


def test_workspace_reuse_with_smaller_batch(pk, gpu):
    """Back-to-back decodes of different sizes on one workspace: the counters
    left by the first call must not disturb the second."""
    wl = W.small_configs()["c3s_bf16_bs16"]
    got = gpu(wl, partition_tokens=16)
    sess = got["session"]
    q = W.q_values(wl).to(_dev())
    ref = OracleRun(wl).decode()
    sub = [1, 4, 7]
    idx = torch.tensor(sub, device=_dev())
    for _ in range(2):
        o_all = pk.paged_attention_decode(sess.pool, q, sess.block_tables, sess.context_lens, wl.scale,
                                          partition_tokens=16).cpu().double().numpy()
        o_sub = pk.paged_attention_decode(sess.pool, q[idx].contiguous(), sess.block_tables[idx].contiguous(),
                                          sess.context_lens[idx].contiguous(), wl.scale,
                                          partition_tokens=16).cpu().double().numpy()
        check_close(o_all, ref, wl.kv_dtype)
        check_close(o_sub, ref[sub], wl.kv_dtype)


def test_partition_lengthened_past_counter_slots(pk, gpu):
    """A caller-sized split that would need more runs than there are arrival
    counters (64 sequences x 32 kv heads x 63 table entries at one block per
    run: 129,024) has its runs lengthened to two blocks; the result still
    matches the oracle on sampled sequences."""
    lens = [1000 - 7 * (i % 5) for i in range(64)]
    wl = W.custom("many_runs_bf16", 32, 32, 128, "bf16", "bf16", 16, lens, index=95)
    mb = wl.max_blocks_per_seq
    assert 64 * 32 * mb > 65528
    pool = pk.KVPool(8, 16, 32, 128, torch.bfloat16, _dev())
    one_block = pk.paged_attention_workspace_size(pool, 64, 32, mb, 16)
    two_blocks = pk.paged_attention_workspace_size(pool, 64, 32, mb, 32)
    assert one_block == two_blocks   # the same plan: runs of two blocks
    got = gpu(wl, partition_tokens=16)
    assert np.isfinite(got["out"]).all()
    seqs = [0, 17, 40, 63]
    ref = OracleRun(wl, prompts=sorted({wl.parent[s] for s in seqs}))
    check_close(got["out"][seqs], ref.decode(seqs)[seqs], wl.kv_dtype)
