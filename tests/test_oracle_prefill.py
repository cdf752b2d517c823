"""Pins for the oracle's multi-token causal paged attention (chunked prefill,
verification of speculative tokens).

* Library routine: torch's scaled_dot_product_attention in fp64 with an
  explicit boolean causal mask (query row i of a sequence with n tokens and m
  new ones may see tokens 0 .. n - m + i), fed with K/V assembled directly from
  the generator's per-token values -- never through a pool or block table --
  and the library's own GQA grouping.
* Closed forms: a chunk with no cached prefix -> its first row is V[0] exactly.
* Invariants: the last row of every sequence is the decode of the whole
  context; rows never depend on later tokens (overwriting the K/V of tokens a
  row may not see leaves it bit-identical); a sequence with no new tokens
  writes nothing.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle.run import OracleRun
from test_oracle_decode import _dequant


def _sdpa_causal(wl, run):
    q = run.q.to(torch.float64)
    kn, vn = W.new_kv(wl)
    qs = wl.query_start
    out = np.zeros((wl.total_q, wl.num_q_heads, wl.head_dim))
    for s, p in enumerate(wl.parent):
        a, b = int(qs[s]), int(qs[s + 1])
        if a == b:
            continue
        kp, vp = W.prompt_kv(wl, p)
        k = _dequant(torch.cat([kp, kn[a:b]], 0), wl, run.k_scale).permute(1, 0, 2).unsqueeze(0)
        v = _dequant(torch.cat([vp, vn[a:b]], 0), wl, run.v_scale).permute(1, 0, 2).unsqueeze(0)
        n, m = k.shape[2], b - a
        pos = torch.arange(n - m, n).unsqueeze(1)                  # position of each query row
        mask = torch.arange(n).unsqueeze(0) <= pos                  # [m][n], True = may attend
        qq = q[a:b].permute(1, 0, 2).unsqueeze(0)                   # [1][Hq][m][d]
        o = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask, scale=wl.scale,
                                                             enable_gqa=True)
        out[a:b] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("name", list(W.small_multi_token_configs()))
def test_oracle_prefill_matches_causal_sdpa(name):
    wl = W.small_multi_token_configs()[name]
    run = OracleRun(wl)
    np.testing.assert_allclose(run.prefill(), _sdpa_causal(wl, run), rtol=1e-10, atol=1e-12)


def test_chunk_without_prefix_starts_with_its_first_value():
    wl = W.small_multi_token_configs()["p4s_f16_g16"]     # sequence 0: 40 new tokens, nothing cached
    assert wl.prompt_lens[0] == 0
    run = OracleRun(wl)
    out = run.prefill()
    _, vn = W.new_kv(wl)
    for h in range(wl.num_q_heads):
        np.testing.assert_array_equal(out[0, h], vn[0, h // wl.group].to(torch.float64).numpy())


@pytest.mark.parametrize("name", ["p2s_bf16", "p3s_fp8", "p5s_fp8_f16_g8"])
def test_last_row_is_decode_of_whole_context(name):
    wl = W.small_multi_token_configs()[name]
    run = OracleRun(wl)
    out = run.prefill()
    last = wl.query_start[1:] - 1
    q_last = run.q[torch.as_tensor(last, dtype=torch.long)].contiguous()
    dec = run.pool.decode(q_last, wl.q_dtype, run.tables, wl.context_lens, wl.scale, wl.num_q_heads)
    np.testing.assert_array_equal(out[last], dec)


def test_rows_do_not_see_later_tokens():
    wl = W.small_multi_token_configs()["p1s_bf16"]
    run = OracleRun(wl)
    before = run.prefill()
    # Overwrite the K/V of each sequence's last new token; only its last row sees it.
    bs, qs, H = wl.block_size, wl.query_start, wl.num_kv_heads
    row = run.pool.block_bytes // (H * bs)          # bytes of one (head, slot) row
    for s in range(wl.num_seqs):
        t = int(wl.context_lens[s]) - 1
        blk = int(run.tables[s][t // bs])
        for h in range(H):
            off = ((blk * H + h) * bs + t % bs) * row
            run.pool.k[off:off + row] = 0x3C
            run.pool.v[off:off + row] = 0x3C
    after = run.prefill()
    last = qs[1:] - 1
    keep = np.setdiff1d(np.arange(wl.total_q), last)
    np.testing.assert_array_equal(after[keep], before[keep])
    assert not np.array_equal(after[last], before[last])


def test_sequence_without_new_tokens_is_skipped():
    wl = W._make("p0", 11, 4, 2, 64, "bf16", "bf16", 16, ctx_lens=[20, 33, 9], query_lens=[3, 0, 2])
    run = OracleRun(wl)
    out = run.prefill()
    assert out.shape[0] == 5
    np.testing.assert_allclose(out, _sdpa_causal(wl, run), rtol=1e-10, atol=1e-12)


def test_row_subset_equals_full_rows():
    wl = W.small_multi_token_configs()["p1s_bf16"]
    run = OracleRun(wl)
    full = run.prefill()
    qs = wl.query_start
    for s in range(wl.num_seqs):
        m = int(qs[s + 1] - qs[s])
        for a, b in [(0, 3), (m - 5, m), (7, 20)]:
            np.testing.assert_array_equal(run.prefill_rows(s, a, b), full[qs[s] + a:qs[s] + b])
