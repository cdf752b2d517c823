"""GPU parity at the workloads' stated sizes, in the launch configurations the
benchmark times (library-sized work split; 512-token runs for the GQA
long-context workload, and the library-sized split there too).  The oracle recomputes sampled sequences one by one
(the longest, the shortest and seeded random picks); copy-on-write pools are
compared byte for byte in full."""
import numpy as np
import pytest

import workloads as W
from oracle.run import OracleRun, check_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _sample(wl, k=8):
    n = wl.context_lens
    rng = np.random.default_rng(449)
    pick = {int(np.argmax(n)), int(np.argmin(n)), 0, wl.num_seqs - 1}
    pick |= set(rng.choice(wl.num_seqs, size=min(k, wl.num_seqs), replace=False).tolist())
    return sorted(pick)


def _check_sampled(wl, got):
    seqs = _sample(wl)
    prompts = sorted({wl.parent[s] for s in seqs})
    ref = OracleRun(wl, prompts=prompts)
    check_close(got["out"][seqs], ref.decode(seqs)[seqs], wl.kv_dtype)
    # the sampled sequences' blocks hold the same bytes on both sides
    bb = ref.pool.block_bytes
    for s in seqs:
        for b in ref.tables[s][ref.tables[s] >= 0]:
            sl = slice(int(b) * bb, (int(b) + 1) * bb)
            assert np.array_equal(got["k"][sl], ref.pool.k[sl]), (s, b)
            assert np.array_equal(got["v"][sl], ref.pool.v[sl]), (s, b)


@pytest.mark.parametrize("name", ["c3_llama7b_bf16_bs16", "c3_llama7b_bf16_bs32", "c2_llama13b_f16",
                                  "c5_gqa_long_fp8e4m3", "c5_gqa_long_bf16"])
def test_full_size_sampled(name):
    from gpu_harness import run_gpu
    wl = W.full_configs()[name]
    got = run_gpu(wl)
    assert np.isfinite(got["out"]).all()
    _check_sampled(wl, got)


@pytest.mark.parametrize("name", ["c5_gqa_long_fp8e4m3", "c5_gqa_long_bf16"])
def test_full_size_library_split(name):
    """The GQA long-context workloads with the library-sized split
    (bench.py --partition-tokens 0) instead of their 512-token runs."""
    from gpu_harness import run_gpu
    wl = W.full_configs()[name]
    got = run_gpu(wl, partition_tokens=0)
    assert np.isfinite(got["out"]).all()
    _check_sampled(wl, got)


@pytest.mark.parametrize("name", ["c4_parallel_sampling_f16_p1023", "c4_parallel_sampling_f16_p1024"])
def test_parallel_sampling_full(name):
    from gpu_harness import run_gpu
    wl = W.full_configs()[name]
    got = run_gpu(wl)
    ref = OracleRun(wl)
    expect_pairs = 3 * wl.num_prompts if wl.prompt_lens[0] % wl.block_size else 0
    assert got["pairs"].shape == (expect_pairs, 2)
    np.testing.assert_array_equal(got["pairs"], ref.plan["pairs"])
    assert np.array_equal(got["k"], ref.pool.k) and np.array_equal(got["v"], ref.pool.v)
    seqs = _sample(wl)
    check_close(got["out"][seqs], ref.decode(seqs)[seqs], wl.kv_dtype)
