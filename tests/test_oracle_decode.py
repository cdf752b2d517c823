"""Pins for the oracle's paged decode attention.

* Library routine: torch's scaled_dot_product_attention in fp64, fed with each
  sequence's K/V assembled directly from the generator's per-token values
  (never through a pool or a block table), with the GQA head grouping of the
  library routine (enable_gqa).  Any slip in the oracle's paging (wrong block,
  slot, head or offset), scale, sign or softmax shows up here.
* Closed forms: one token -> its V exactly; q = 0 or equal keys -> mean of V;
  one dominant key -> its V.
* Invariants the pages fix: the result does not depend on where blocks lie in
  the pool (any permutation, including the identity i.e. a contiguous layout),
  and bytes outside the owned slots are never read.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.run import OracleRun


def _dequant(x, wl, scale):
    """K/V values as the pool holds them, in fp64: the source values for
    non-fp8 pools; for fp8 pools torch's own RNE cast of fp32(x)/scale."""
    if wl.kv_dtype != "fp8e4m3":
        return x.to(torch.float64)
    xs = (x.float() / torch.tensor(scale, dtype=torch.float32))
    return xs.to(torch.float8_e4m3fn).to(torch.float64) * scale


def _sdpa_expected(wl, run):
    q = run.q.to(torch.float64)
    kn, vn = W.new_kv(wl)
    out = np.zeros((wl.num_seqs, wl.num_q_heads, wl.head_dim))
    cache = {}
    for s, p in enumerate(wl.parent):
        if p not in cache:
            cache[p] = W.prompt_kv(wl, p)
        kp, vp = cache[p]
        k = torch.cat([kp, kn[s:s + 1]], 0)   # [n][Hkv][d]
        v = torch.cat([vp, vn[s:s + 1]], 0)
        k = _dequant(k, wl, run.k_scale).permute(1, 0, 2).unsqueeze(0)  # [1][Hkv][n][d]
        v = _dequant(v, wl, run.v_scale).permute(1, 0, 2).unsqueeze(0)
        qq = q[s].unsqueeze(0).unsqueeze(2)                                # [1][Hq][1][d]
        o = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=wl.scale, enable_gqa=True)
        out[s] = o[0, :, 0, :].numpy()
    return out


@pytest.mark.parametrize("name", ["c1_tiny_f32", "c2s_f16", "c3s_bf16_bs16", "c3s_bf16_bs32", "c4s_cow_f16",
                                  "c4s_aligned_f16", "c5s_fp8", "c5s_bf16"])
def test_oracle_matches_sdpa(name):
    wl = W.small_configs()[name]
    run = OracleRun(wl)
    got = run.decode()
    want = _sdpa_expected(wl, run)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_gqa_grouping_is_contiguous():
    # GQA: query head h reads kv head h // (Hq/Hkv); a mapping h % Hkv would
    # disagree with the library routine.  Checked on a case where it matters.
    wl = W.small_configs()["c5s_bf16"]
    assert wl.group > 1 and wl.num_kv_heads > 1
    run = OracleRun(wl)
    np.testing.assert_allclose(run.decode(), _sdpa_expected(wl, run), rtol=1e-10, atol=1e-12)


def test_single_token_returns_its_value_exactly():
    wl = W.config_c1()          # sequence 0 has context length 1
    run = OracleRun(wl)
    out = run.decode()
    _, vn = W.new_kv(wl)
    assert wl.context_lens[0] == 1
    np.testing.assert_array_equal(out[0], vn[0].to(torch.float64).numpy())


def _pool_with(wl, k_tok, v_tok):
    """Oracle pool holding the given per-token K/V of one sequence (contiguous
    placement), for closed-form cases."""
    n = k_tok.shape[0]
    pool = oracle.HostPool(-(-n // wl.block_size) + 1, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    slots = np.arange(n, dtype=np.int64)
    pool.reshape_and_cache(k_tok, v_tok, wl.src_dtype, slots)
    tables = np.arange(-(-n // wl.block_size), dtype=np.int32)[None, :]
    return pool, tables


def test_zero_query_gives_mean_of_values():
    wl = W.custom("closed", 2, 2, 64, "f32", "f32", 16, [37])
    g = torch.Generator().manual_seed(3)
    k = torch.randn(37, 2, 64, generator=g)
    v = torch.randn(37, 2, 64, generator=g)
    pool, tables = _pool_with(wl, k, v)
    q = torch.zeros(1, 2, 64)
    out = pool.decode(q, "f32", tables, np.array([37], np.int32), 0.125, 2)
    np.testing.assert_allclose(out[0], v.double().mean(0).numpy(), rtol=1e-13, atol=1e-14)


def test_equal_keys_give_mean_of_values():
    wl = W.custom("closed", 1, 1, 64, "f32", "f32", 16, [50])
    g = torch.Generator().manual_seed(4)
    k = torch.randn(1, 1, 64, generator=g).expand(50, 1, 64).contiguous()
    v = torch.randn(50, 1, 64, generator=g)
    pool, tables = _pool_with(wl, k, v)
    q = torch.randn(1, 1, 64, generator=g)
    out = pool.decode(q, "f32", tables, np.array([50], np.int32), 0.125, 1)
    np.testing.assert_allclose(out[0, 0], v[:, 0].double().mean(0).numpy(), rtol=1e-13, atol=1e-14)


def test_dominant_key_selects_its_value():
    wl = W.custom("closed", 1, 1, 64, "f32", "f32", 16, [40])
    g = torch.Generator().manual_seed(5)
    k = torch.randn(40, 1, 64, generator=g) * 0.01
    v = torch.randn(40, 1, 64, generator=g)
    q = torch.ones(1, 1, 64)
    k[29, 0, :] = 10.0          # score 640 * scale vs ~0 for every other key
    pool, tables = _pool_with(wl, k, v)
    out = pool.decode(q, "f32", tables, np.array([40], np.int32), 1.0, 1)
    np.testing.assert_allclose(out[0, 0], v[29, 0].double().numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["c2s_f16", "c4s_cow_f16", "c5s_fp8"])
def test_placement_invariance(name):
    wl = W.small_configs()[name]
    base = OracleRun(wl).decode()
    rng = np.random.default_rng(11)
    for order in [np.arange(wl.num_blocks), rng.permutation(wl.num_blocks), np.arange(wl.num_blocks)[::-1]]:
        got = OracleRun(wl, free_order=order.astype(np.int32)).decode()
        np.testing.assert_array_equal(got, base)


def test_unowned_bytes_are_never_read():
    wl = W.small_configs()["c3s_bf16_bs16"]
    run = OracleRun(wl)
    base = run.decode()
    # every element still holding the all-ones poison (a NaN that no write
    # produces) is an unowned slot: overwrite it with other garbage
    for buf in (run.pool.k, run.pool.v):
        elems = buf.view(np.uint16)
        poison = elems == 0xFFFF
        assert poison.any()
        elems[poison] = 0x7F00
    np.testing.assert_array_equal(run.decode(), base)


def test_rejects_bad_lengths_and_blocks():
    wl = W.small_configs()["c2s_f16"]
    run = OracleRun(wl)
    lens = wl.context_lens.copy()
    lens[0] = 0
    with pytest.raises(oracle.OracleError):
        run.pool.decode(run.q, wl.q_dtype, run.tables, lens, wl.scale, wl.num_q_heads)
    t = run.tables.copy()
    t[0, 0] = wl.num_blocks
    with pytest.raises(oracle.OracleError):
        run.pool.decode(run.q, wl.q_dtype, t, wl.context_lens, wl.scale, wl.num_q_heads)
