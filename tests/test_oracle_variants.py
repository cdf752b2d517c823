"""Pins for the oracle on the variant workloads: block sizes 8 and 64, 8:1
query groups, and per-kv-head fp8 scales.

* Library routine: fp64 SDPA (enable_gqa) on K/V assembled from the
  generator's per-token values; for fp8 pools each head's values go through
  torch's own RNE cast of fp32(x) / scale_h, then times scale_h.
* Special case: per-head scales that all equal the per-tensor scale give
  bit-identical pools and outputs to the per-tensor path.
* Multi-token: the causal check with per-head scales.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import HostPool
from oracle.run import OracleRun


def _dequant_heads(x, wl, scales):
    """[n][H][d] source values -> fp64 as an fp8 pool with per-head scales holds them."""
    s = torch.tensor(scales, dtype=torch.float32)[None, :, None]
    codes = (x.float() / s).to(torch.float8_e4m3fn)
    return codes.to(torch.float64) * s.to(torch.float64)


def _kv(wl, run, p, kn, vn, a, b):
    kp, vp = W.prompt_kv(wl, p)
    k, v = torch.cat([kp, kn[a:b]], 0), torch.cat([vp, vn[a:b]], 0)
    if wl.kv_dtype != "fp8e4m3":
        return k.to(torch.float64), v.to(torch.float64)
    if wl.head_scales:
        ks, vs = run.head_scales
        return _dequant_heads(k, wl, ks), _dequant_heads(v, wl, vs)
    return _dequant_heads(k, wl, [run.k_scale] * wl.num_kv_heads), _dequant_heads(v, wl, [run.v_scale] * wl.num_kv_heads)


def _sdpa(wl, run):
    q = run.q.to(torch.float64)
    kn, vn = W.new_kv(wl)
    qs = wl.query_start
    out = np.zeros((wl.total_q, wl.num_q_heads, wl.head_dim))
    for s, p in enumerate(wl.parent):
        a, b = int(qs[s]), int(qs[s + 1])
        if a == b:
            continue
        k, v = _kv(wl, run, p, kn, vn, a, b)
        k, v = k.permute(1, 0, 2).unsqueeze(0), v.permute(1, 0, 2).unsqueeze(0)
        n, m = k.shape[2], b - a
        mask = torch.arange(n).unsqueeze(0) <= torch.arange(n - m, n).unsqueeze(1)
        o = torch.nn.functional.scaled_dot_product_attention(q[a:b].permute(1, 0, 2).unsqueeze(0), k, v,
                                                             attn_mask=mask, scale=wl.scale, enable_gqa=True)
        out[a:b] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("name", list(W.small_variant_configs()))
def test_variants_match_sdpa(name):
    wl = W.small_variant_configs()[name]
    run = OracleRun(wl)
    got = run.prefill() if wl.multi_token else run.decode()
    np.testing.assert_allclose(got, _sdpa(wl, run), rtol=1e-10, atol=1e-12)


def test_head_scales_differ_across_heads():
    wl = W.small_variant_configs()["c5s_fp8_headscale"]
    ks, vs = W.fp8_head_scales(wl)
    assert ks.max() / ks.min() > 8 and vs.max() / vs.min() > 8


def test_equal_head_scales_reduce_to_the_tensor_scale():
    wl = W.small_configs()["c5s_fp8"]
    base = OracleRun(wl)
    H = wl.num_kv_heads
    hs = (np.full(H, base.k_scale, dtype=np.float32), np.full(H, base.v_scale, dtype=np.float32))
    pool = HostPool(wl.num_blocks, wl.block_size, H, wl.head_dim, wl.kv_dtype, 1.0, 1.0, head_scales=hs)
    for p in range(wl.num_prompts):
        k, v = W.prompt_kv(wl, p)
        pool.reshape_and_cache(k, v, wl.src_dtype, base.plan["prompt_slots"][p])
    pool.copy_blocks(base.plan["pairs"])
    kn, vn = W.new_kv(wl)
    pool.reshape_and_cache(kn, vn, wl.src_dtype, base.plan["new_slots"])
    assert np.array_equal(pool.k, base.pool.k) and np.array_equal(pool.v, base.pool.v)
    got = pool.decode(base.q, wl.q_dtype, base.tables, wl.context_lens, wl.scale, wl.num_q_heads)
    np.testing.assert_array_equal(got, base.decode())
