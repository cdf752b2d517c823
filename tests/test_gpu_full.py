"""GPU parity at the workloads' stated sizes, in the launch configurations the
benchmark times (library-sized work split; 512-token runs for the GQA
long-context workload, and the library-sized split there too).  Every
sequence's output is compared with the oracle, whose sequences are dealt to
the host's cores, and both pools are compared with the oracle's byte for
byte."""
import numpy as np
import pytest

import bench
import workloads as W
from oracle.run import OracleRun, check_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# the oracle of one workload at a time (its pools are up to a few GB)
_REF = {}


def reference(wl):
    """(oracle run, oracle output of every sequence) for a workload."""
    if wl.name not in _REF:
        _REF.clear()
        threads = bench.host_threads()
        ref = OracleRun(wl, threads=threads)
        _REF[wl.name] = (ref, ref.decode_parallel(threads))
    return _REF[wl.name]


def check_all(wl, got, out=None):
    """Whole pools bit-exact and every sequence's output within tolerance."""
    ref, want = reference(wl)
    assert np.array_equal(got["k"], ref.pool.k), "K pool bytes differ"
    assert np.array_equal(got["v"], ref.pool.v), "V pool bytes differ"
    out = got["out"] if out is None else out
    assert np.isfinite(out).all()
    check_close(out, want, wl.kv_dtype)


@pytest.mark.parametrize("name", ["c3_llama7b_bf16_bs16", "c3_llama7b_bf16_bs32", "c2_llama13b_f16",
                                  "c5_gqa_long_fp8e4m3", "c5_gqa_long_bf16"])
def test_full_size_every_sequence(name):
    """The benchmarked split, then (GQA long context) the library-sized split
    on the same pool."""
    from gpu_harness import announce, run_gpu
    import torch
    wl = W.full_configs()[name]
    got = run_gpu(wl)
    check_all(wl, got)
    if wl.partition_tokens:
        announce(f"{name} library split")
        sess = got["session"]
        out = sess.attend(got["q"], partition_tokens=0, scale=wl.scale)
        torch.cuda.synchronize()
        check_all(wl, got, out.float().cpu().double().numpy())


@pytest.mark.parametrize("name", ["c4_parallel_sampling_f16_p1023", "c4_parallel_sampling_f16_p1024"])
def test_parallel_sampling_full(name):
    from gpu_harness import run_gpu
    wl = W.full_configs()[name]
    got = run_gpu(wl)
    ref, _ = reference(wl)
    expect_pairs = 3 * wl.num_prompts if wl.prompt_lens[0] % wl.block_size else 0
    assert got["pairs"].shape == (expect_pairs, 2)
    np.testing.assert_array_equal(got["pairs"], ref.plan["pairs"])
    check_all(wl, got)
