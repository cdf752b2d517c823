"""GPU parity of multi-token causal paged attention (chunked prefill and
speculative verification) through the C ABI against the CPU oracle.

  * pools after the step's cache writes: whole-pool byte equality;
  * output: |gpu - oracle| <= atol + rtol |oracle| elementwise with the
    decode tolerances (the kernel computes in the same precisions), every
    unowned slot poisoned with NaN bytes;
  * at the full sizes: sampled sequences (the oracle computes them one by
    one) plus properties checked on every row (finite, bitwise repeatable);
  * every launch shape: one-wave 16-row tiles, split work-group row blocks
    and one work-group per row block (forced with PAGEDKV_PREFILL_PATH; the
    full sizes use the library's choice).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle.run import OracleRun, check_close

pytestmark = pytest.mark.gpu

SMALL = list(W.small_multi_token_configs())
ALL_SMALL = {**W.small_multi_token_configs(),
             **{k: v for k, v in W.small_variant_configs().items() if v.multi_token}}


@pytest.fixture(scope="module")
def gpu():
    from gpu_harness import run_gpu_prefill
    return run_gpu_prefill


@pytest.fixture(params=["auto", "wave", "group", "unit"])
def path(request, monkeypatch):
    """The library picks one-wave 16-row tiles, split work-group row blocks
    or one work-group per row block from the rows per sequence; each is
    forced here as well."""
    if request.param != "auto":
        monkeypatch.setenv("PAGEDKV_PREFILL_PATH", request.param)
    from gpu_harness import announce
    announce(f"prefill path {request.param}")
    return request.param


@pytest.mark.parametrize("name", list(ALL_SMALL))
def test_prefill_matches_oracle(gpu, name, path):
    wl = ALL_SMALL[name]
    got = gpu(wl)
    ref = OracleRun(wl)
    np.testing.assert_array_equal(got["tables"], ref.tables)
    np.testing.assert_array_equal(got["slots"], ref.plan["new_slots"])
    assert np.array_equal(got["k"], ref.pool.k), "K pool bytes differ"
    assert np.array_equal(got["v"], ref.pool.v), "V pool bytes differ"
    assert np.isfinite(got["out"]).all()
    check_close(got["out"], ref.prefill(), wl.kv_dtype)


@pytest.mark.parametrize("G,D,kv,q", [(1, 128, "bf16", "bf16"), (2, 64, "f16", "f16"), (4, 128, "fp8e4m3", "bf16"),
                                      (8, 256, "bf16", "bf16"), (16, 64, "fp8e4m3", "f16")])
def test_ragged_and_empty_query_counts(gpu, G, D, kv, q, path):
    """Sequences with no new tokens, one, a partial tile, several tiles,
    chunks that start mid-block and chunks equal to the whole context."""
    ctx = [50, 17, 64, 5, 130, 33]
    qn = [0, 1, 13, 5, 40, 0]
    wl = W._make(f"ragged_g{G}_d{D}_{kv}", 12 + G, 2 * G, 2, D, kv, q, 16, ctx_lens=ctx, query_lens=qn)
    got = gpu(wl)
    check_close(got["out"], OracleRun(wl).prefill(), wl.kv_dtype)


@pytest.mark.parametrize("S", [256, 300])
def test_units_at_and_past_the_rank_limit(gpu, S, monkeypatch):
    """One work-group per row block with as many sequences as the kernel ranks
    (longest first) and with more (dispatch order), some without new rows."""
    monkeypatch.setenv("PAGEDKV_PREFILL_PATH", "unit")
    rng = np.random.default_rng(S)
    ctx = rng.integers(1, 60, size=S)
    qn = np.minimum(ctx, rng.integers(0, 40, size=S))
    qn[::9] = 0
    wl = W._make(f"units_{S}", 15, 8, 2, 64, "bf16", "bf16", 16, ctx_lens=ctx.tolist(), query_lens=qn.tolist())
    check_close(gpu(wl)["out"], OracleRun(wl).prefill(), wl.kv_dtype)


@pytest.mark.parametrize("value", [99840.0, 1.0e30, float("nan")])
def test_bf16_values_out_of_f16_range(gpu, value, monkeypatch):
    """bf16 pools stage V as f16 in the row-block kernel and run a block again
    with bf16 V when a value is out of f16's range: one large V element in
    one cached token (past f16's range, far past it, a NaN) still gives
    the oracle's output (NaN: the rows that see it are NaN, the rest match)."""
    monkeypatch.setenv("PAGEDKV_PREFILL_PATH", "unit")
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce
    wl = W._make("bf16_range", 16, 8, 2, 128, "bf16", "bf16", 16, ctx_lens=[300, 180, 90], query_lens=[140, 40, 90])
    got = gpu(wl)
    sess, q = got["session"], got["q"]
    ref = OracleRun(wl)
    s, h, slot, e = 1, 1, 3, 77                        # cached token 3 of sequence 1, kv head 1, element 77
    blk = int(ref.tables[s][0])
    bits = np.array([value], dtype=np.float32).view(np.uint32)[0] >> 16
    off = ((blk * wl.num_kv_heads + h) * wl.block_size + slot) * wl.head_dim + e
    ref.pool.v.view(np.uint16)[off] = bits
    sess.pool.v_cache.view(torch.int16).view(-1)[off] = int(np.array([bits], dtype=np.uint16).view(np.int16)[0])
    announce(f"bf16 V element {value} at sequence {s} kv head {h}")
    out = pk.paged_attention_prefill(sess.pool, q, sess.block_tables, sess.context_lens, sess.query_start, wl.scale)
    torch.cuda.synchronize()
    got2 = out.float().cpu().double().numpy()
    want = ref.prefill()
    if value != value:
        bad = np.isnan(want)
        assert bad.any() and np.array_equal(np.isnan(got2), bad)
        check_close(np.where(bad, 0, got2), np.where(bad, 0, want), wl.kv_dtype)
    else:
        assert np.isfinite(want).all()
        check_close(got2, want, wl.kv_dtype)


@pytest.mark.parametrize("kv", ["bf16", "fp8e4m3"])
@pytest.mark.parametrize("scale", [-0.11, 0.0, 0.9])
def test_scale_sign_and_zero(gpu, kv, scale, path):
    """The score scale enters inside the exponent and the row max is taken
    before scaling: a negative scale (q's sign flipped), a zero one (every
    visible token weighs the same) and a large one match the oracle."""
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce
    wl = W._make(f"scale_{kv}", 17, 8, 2, 128, kv, "bf16", 16, ctx_lens=[200, 70, 33], query_lens=[150, 70, 20])
    got = gpu(wl)
    sess, q = got["session"], got["q"]
    announce(f"prefill scale {scale} {kv}")
    out = pk.paged_attention_prefill(sess.pool, q, sess.block_tables, sess.context_lens, sess.query_start, scale)
    torch.cuda.synchronize()
    ref = OracleRun(wl)
    want = ref.pool.prefill(ref.q, wl.q_dtype, ref.tables, wl.context_lens, wl.query_start, scale, wl.num_q_heads)
    check_close(out.float().cpu().double().numpy(), want, wl.kv_dtype)


def test_one_new_token_matches_decode_oracle(gpu):
    """m = 1 for every sequence is the decode step: the multi-token kernel
    agrees with the oracle's decode."""
    base = W.small_configs()["c5s_bf16"]
    wl = W._make("m1_gqa", 13, base.num_q_heads, base.num_kv_heads, base.head_dim, "bf16", "bf16", 16,
                 ctx_lens=list(base.context_lens), query_lens=[1] * base.num_seqs)
    got = gpu(wl)
    check_close(got["out"], OracleRun(wl).decode(), wl.kv_dtype)


def test_block_size_32(gpu, path):
    wl = W._make("bs32", 14, 8, 2, 128, "bf16", "bf16", 32, ctx_lens=[100, 64, 31], query_lens=[70, 33, 31])
    check_close(gpu(wl)["out"], OracleRun(wl).prefill(), wl.kv_dtype)


def test_repeat_is_bitwise_deterministic(gpu, path):
    wl = W.small_multi_token_configs()["p3s_fp8"]
    got = gpu(wl, repeat=3)
    for o in got["outs"][1:]:
        assert np.array_equal(o, got["outs"][0])


@pytest.mark.parametrize("name", list(W.multi_token_configs()))
def test_full_size_sampled(gpu, name):
    wl = W.multi_token_configs()[name]
    got = gpu(wl, repeat=2)
    out = got["out"]
    assert np.isfinite(out).all()
    assert np.array_equal(got["outs"][1], out)
    ref = OracleRun(wl)
    rng = np.random.default_rng(5)
    qs = wl.query_start
    for s in sorted(rng.choice(wl.num_seqs, size=min(4, wl.num_seqs), replace=False).tolist()):
        m = int(qs[s + 1] - qs[s])
        for a, b in {(0, min(m, 8)), (max(0, m - 8), m)}:   # the first and the last rows
            check_close(out[qs[s] + a:qs[s] + b], ref.prefill_rows(s, a, b), wl.kv_dtype)
