"""A decode step captured in a HIP graph: its launches (copy_blocks, the cache
write, decode attention, and the multi-token attention) allocate nothing and
record no memset once the output and workspace exist, so a captured step can
be replayed.  Each replay, with eager work and synchronisations between the
replays, must reproduce the eager step bit for bit: the pools and the output.
The split-run cases check that every replay leaves the workspace's arrival
counters at zero for the next one."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _captured_step_matches_eager(wl, partition_tokens, multi=False, replays=3):
    import bench
    import paged_kv_cache_449_amd as pk
    from gpu_harness import announce
    announce(f"graph {wl.name} partition={partition_tokens}")
    dev = torch.device("cuda", 0)
    sess, q, kn, vn = bench.build_session(wl, dev)
    pool = sess.pool
    out = torch.empty_like(q)

    def step():
        pk.copy_blocks(pool, sess.pairs)
        pk.reshape_and_cache(pool, kn, vn, sess.slot_mapping)
        if multi:
            pk.paged_attention_prefill(pool, q, sess.block_tables, sess.context_lens, sess.query_start, wl.scale,
                                       out=out)
        else:
            pk.paged_attention_decode(pool, q, sess.block_tables, sess.context_lens, wl.scale, out=out,
                                      partition_tokens=partition_tokens)

    step()
    torch.cuda.synchronize(dev)
    eager, k0, v0 = out.clone(), pool.k_cache.clone(), pool.v_cache.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize(dev)
    for r in range(replays):
        out.zero_()              # eager work between replays
        step()                   # and an eager step on the same workspace
        torch.cuda.synchronize(dev)
        assert torch.equal(out, eager), f"eager step {r}"
        out.zero_()
        torch.cuda.synchronize(dev)
        graph.replay()
        torch.cuda.synchronize(dev)
        assert torch.equal(out, eager), f"replay {r}"
        assert torch.equal(pool.k_cache.view(torch.uint8), k0.view(torch.uint8)), f"replay {r}: K pool"
        assert torch.equal(pool.v_cache.view(torch.uint8), v0.view(torch.uint8)), f"replay {r}: V pool"


@pytest.mark.parametrize("name,partition_tokens", [("c4s_cow_f16", 0), ("c3s_bf16_bs16", 0), ("c3s_bf16_bs16", 16),
                                                   ("c5s_fp8", 512), ("c5s_bf16", 0)])
def test_graph_replay_decode(name, partition_tokens):
    _captured_step_matches_eager(W.small_configs()[name], partition_tokens)


def test_graph_replay_multi_token():
    _captured_step_matches_eager(W.small_multi_token_configs()["p1s_bf16"], 0, multi=True)
