"""GPU parity of prefix-grouped decode (paged_attention_decode_grouped):
forked candidates read their shared prompt blocks once per group.  Outputs
must match the oracle's decode (which knows nothing of groups) within the
decode tolerances, on MHA and GQA query groups, 16-bit and fp8 pools, groups
cut to the 16-row limit by the host helper or by the library, more groups
than one 64-lane slice of group starts, and groups whose stated sharing is
zero or longer than the contexts."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle.run import OracleRun, check_close

pytestmark = pytest.mark.gpu


def _shared_wl(name, index, hq, hkv, kv, q, prompt_lens, n, head_scales=False, bs=16):
    parent = [p for p in range(len(prompt_lens)) for _ in range(n)]
    return W._make(name, index, hq, hkv, 128, kv, q, bs, prompt_lens=prompt_lens, parent=parent,
                   head_scales=head_scales)


CASES = {
    "c4s_cow_f16": W.small_configs()["c4s_cow_f16"],
    "c4s_aligned_f16": W.small_configs()["c4s_aligned_f16"],
    "c4s_same_f16": W.small_configs()["c4s_same_f16"],
    "gqa4_bf16": _shared_wl("gqa4_bf16", 40, 8, 2, "bf16", "bf16", [95, 80, 130], 4),
    "gqa4_fp8": _shared_wl("gqa4_fp8", 41, 8, 2, "fp8e4m3", "bf16", [95, 80, 130], 4),
    "gqa8_f16_split": _shared_wl("gqa8_f16_split", 42, 16, 2, "f16", "f16", [63, 200], 4),
    "mha_bf16_n6": _shared_wl("mha_bf16_n6", 43, 4, 4, "bf16", "bf16", [33, 47], 6),
    "gqa2_fp8_headscale_f16": _shared_wl("gqa2_fp8_headscale_f16", 44, 8, 4, "fp8e4m3", "f16", [70, 150], 3,
                                         head_scales=True),
    "mha_f16_bs32": _shared_wl("mha_f16_bs32", 45, 4, 4, "f16", "f16", [95, 64], 4, bs=32),
    # more groups than one 64-lane slice of group starts
    "many_groups_f16": _shared_wl("many_groups_f16", 46, 4, 4, "f16", "f16", [20 + 9 * (i % 7) for i in range(70)], 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_grouped_matches_oracle(name):
    from gpu_harness import run_gpu
    wl = CASES[name]
    got = run_gpu(wl, grouped=True)
    ref = OracleRun(wl)
    assert np.array_equal(got["k"], ref.pool.k) and np.array_equal(got["v"], ref.pool.v)
    assert np.isfinite(got["out"]).all()
    check_close(got["out"], ref.decode(), wl.kv_dtype)
    sess = got["session"]
    if wl.num_prompts < wl.num_seqs and wl.prompt_lens[0] >= 16:
        assert sess.shared_blocks > 0, "the helper found no shared prefix"


def _raw_grouped(sess, q, wl, group_start, group_shared):
    import paged_kv_cache_449_amd as pk
    dev = q.device
    gs = torch.as_tensor(np.asarray(group_start, dtype=np.int32), device=dev)
    gsh = torch.as_tensor(np.asarray(group_shared, dtype=np.int32), device=dev)
    out = pk.paged_attention_decode_grouped(sess.pool, q, sess.block_tables, sess.context_lens, wl.scale, gs, gsh)
    torch.cuda.synchronize(dev)
    return out.float().cpu().double().numpy()


def test_library_cuts_groups_to_the_row_limit():
    """Groups of 4 candidates with 8 query heads per kv head (32 rows) passed
    uncut: the library runs the first 2 members shared and the others alone."""
    from gpu_harness import run_gpu
    wl = CASES["gqa8_f16_split"]
    got = run_gpu(wl)
    sess, q = got["session"], got["q"]
    import paged_kv_cache_449_amd as pk
    starts, shared = pk.shared_prefix_groups(sess.block_tables.cpu().numpy(), sess.context_lens.cpu().numpy(), 4)
    assert (np.diff(starts) == 4).all() and (shared > 0).all()
    out = _raw_grouped(sess, q, wl, starts, shared)
    check_close(out, OracleRun(wl).decode(), wl.kv_dtype)


@pytest.mark.parametrize("name,shared", [("c4s_cow_f16", 0), ("c4s_aligned_f16", 10_000)])
def test_zero_or_oversized_sharing(name, shared):
    """No sharing decodes every sequence alone.  A stated sharing longer than
    the contexts is cut to whole blocks within every member's context: with
    block-aligned prompts (context = prompt + 1) that cut is exactly the
    prompt's blocks, which the candidates do share."""
    from gpu_harness import run_gpu
    wl = CASES[name]
    got = run_gpu(wl)
    sess, q = got["session"], got["q"]
    starts = list(range(0, wl.num_seqs + 1, 4))
    out = _raw_grouped(sess, q, wl, starts, [shared] * (len(starts) - 1))
    check_close(out, OracleRun(wl).decode(), wl.kv_dtype)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c4_parallel_sampling_f16_p1023", "c4_parallel_sampling_f16_p1024"])
def test_grouped_full_size_every_sequence(name):
    from gpu_harness import run_gpu
    from test_gpu_full import check_all
    wl = W.full_configs()[name]
    got = run_gpu(wl, grouped=True)
    assert got["session"].shared_blocks > 0
    check_all(wl, got)
