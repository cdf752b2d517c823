"""Pins for the oracle's block-manager emulation, its cache write and block
copy, and the KV footprint formula, against what the pages fix."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from conftest import GOLDEN
from oracle.paging import PagingEmulator, PoolExhausted, internal_waste, plan
from oracle.run import OracleRun


def _golden(name):
    return json.load(open(os.path.join(GOLDEN, name)))


def test_block_table_diagram():
    g = _golden("block_table_example.json")
    bs = g["block_size"]
    # a free list that hands out the diagram's physical blocks in order
    order = g["physical_blocks"] + [b for b in range(8) if b not in g["physical_blocks"]]
    wl = W.custom("diagram", 1, 1, 64, "f32", "f32", bs, [3 * bs], num_blocks=8)
    p = plan(wl, np.asarray(order, np.int32))
    assert p["tables"][0, :3].tolist() == g["physical_blocks"]
    # token positions map to offsets inside the mapped physical block
    slots = np.concatenate([p["prompt_slots"][0], p["new_slots"]])
    for pos in range(3 * bs):
        assert slots[pos] == g["physical_blocks"][pos // bs] * bs + pos % bs


def test_default_block_size_is_16_tokens():
    g = _golden("block_size.json")
    assert W.config_c2().block_size == g["default_tokens"]
    assert {W.config_c3(16).block_size, W.config_c3(32).block_size} == {g["default_tokens"], g["alternative_tokens"]}


@pytest.mark.parametrize("name", ["c1_tiny_f32", "c2s_f16", "c3s_bf16_bs16", "c3s_bf16_bs32", "c5s_fp8"])
def test_internal_waste_bound_and_exact(name):
    """At most one partly filled block per sequence (block_size - 1 unused
    slots at most), measured by counting still-poisoned slots in the blocks
    each sequence owns."""
    wl = W.small_configs()[name]
    run = OracleRun(wl)
    bs = wl.block_size
    eb = oracle.ELEM_BYTES[wl.kv_dtype]
    row = wl.head_dim * eb
    total = 0
    for s in range(wl.num_seqs):
        n = int(wl.context_lens[s])
        blocks = run.tables[s][run.tables[s] >= 0]
        assert len(blocks) == -(-n // bs)
        unused = 0
        for b in blocks:
            for o in range(bs):
                off = ((int(b) * wl.num_kv_heads + 0) * bs + o) * row
                if np.all(run.pool.k[off:off + row] == 0xFF):
                    unused += 1
        assert unused <= bs - 1
        assert (n % bs == 0) == (unused == 0)
        total += unused
    assert total == internal_waste(wl.context_lens, bs)
    assert total <= wl.num_seqs * (bs - 1)


def test_no_block_is_owned_twice_without_sharing():
    wl = W.small_configs()["c3s_bf16_bs16"]
    p = plan(wl, W.free_list_order(wl))
    used = p["tables"][p["tables"] >= 0]
    assert len(np.unique(used)) == len(used)
    assert p["free_left"] == wl.num_blocks - len(used)


def test_parallel_sampling_copy_on_write_full_size():
    g = _golden("parallel_sampling_cow.json")
    wl = W.config_c4()                       # 64 prompts x n=4, prompt 1023 tokens
    p = plan(wl, W.free_list_order(wl))
    assert g["n"] == 4
    pairs = p["pairs"]
    assert pairs.shape == (wl.num_prompts * g["copies_on_first_step"], 2)
    bs = wl.block_size
    nprompt_blocks = -(-wl.prompt_lens[0] // bs)
    for pr in range(wl.num_prompts):
        cands = [s for s, q in enumerate(wl.parent) if q == pr]
        t = p["tables"][cands]
        # the full prompt blocks stay shared by all n candidates
        assert (t[:, :nprompt_blocks - 1] == t[0, :nprompt_blocks - 1]).all()
        for b in t[0, :nprompt_blocks - 1]:
            assert p["refcount"][int(b)] == g["ref_count_after_fork"]
        # the partly filled last block: n-1 candidates got a private copy, the last kept it
        last = t[:, nprompt_blocks - 1]
        assert len(set(last.tolist())) == g["n"]
        assert p["refcount"][int(last[-1])] == 1
        src = {int(a) for a, b in pairs if int(b) in set(last[:-1].tolist())}
        assert src == {int(last[-1])}


def test_block_aligned_prompt_needs_no_copy():
    wl = W.config_c4(prompt_len=1024)
    p = plan(wl, W.free_list_order(wl))
    assert p["pairs"].shape == (0, 2)
    # every candidate appended into a fresh block of its own
    fresh = p["tables"][:, 64]
    assert len(set(fresh.tolist())) == wl.num_seqs


def test_copy_on_write_content_and_candidate_symmetry():
    wl = W.small_configs()["c4s_same_f16"]   # candidates get identical q and new K/V
    run = OracleRun(wl)
    out = run.decode()
    for pr in range(wl.num_prompts):
        cands = [s for s, q in enumerate(wl.parent) if q == pr]
        for s in cands[1:]:
            np.testing.assert_array_equal(out[s], out[cands[0]])
    # copied blocks equal their source on the slots the prompt had filled
    pairs = run.plan["pairs"]
    assert len(pairs) == wl.num_prompts * 3
    bs, row = wl.block_size, wl.head_dim * 2
    filled = wl.prompt_lens[0] % bs
    bb = run.pool.block_bytes
    for a, b in pairs:
        for h in range(wl.num_kv_heads):
            for o in range(filled):
                off = (h * bs + o) * row
                assert np.array_equal(run.pool.k[a * bb + off:a * bb + off + row], run.pool.k[b * bb + off:b * bb + off + row])
                assert np.array_equal(run.pool.v[a * bb + off:a * bb + off + row], run.pool.v[b * bb + off:b * bb + off + row])


def test_pool_exhaustion_raises():
    wl = W.custom("tiny_pool", 1, 1, 64, "f32", "f32", 16, [40, 40], num_blocks=4)
    with pytest.raises(PoolExhausted):
        plan(wl, np.arange(4, dtype=np.int32))


def test_release_returns_blocks_to_free_list():
    em = PagingEmulator(np.arange(3), 16)
    b = em.take()
    em.refcount[b] = 2
    em.give_back(b)
    assert b not in em.free
    em.give_back(b)
    assert list(em.free)[-1] == b


def test_cache_write_round_trip_and_skip():
    wl = W.custom("rt", 3, 3, 64, "bf16", "bf16", 16, [70], num_blocks=9)
    order = np.asarray([5, 2, 8, 0, 7, 1, 3, 4, 6], np.int32)
    p = plan(wl, order)
    k, v = W.prompt_kv(wl, 0)
    pool = oracle.HostPool(wl.num_blocks, 16, 3, 64, "bf16")
    slots = p["prompt_slots"][0].copy()
    slots[5] = -1                              # skipped token
    pool.reshape_and_cache(k, v, "bf16", slots)
    K = pool.k.view(np.uint16).reshape(wl.num_blocks, 3, 16, 64)
    kb = k.view(torch.int16).numpy().view(np.uint16)
    for pos in range(k.shape[0]):
        blk, o = order[pos // 16], pos % 16
        if pos == 5:
            assert (K[blk, :, o, :] == 0xFFFF).all()
        else:
            assert (K[blk, :, o, :] == kb[pos]).all()
    # untouched blocks keep the poison
    owned = set(order[:5].tolist())
    for b in range(wl.num_blocks):
        if b not in owned:
            assert (K[b] == 0xFFFF).all()


def test_cache_write_order_does_not_matter():
    wl = W.small_configs()["c2s_f16"]
    p = plan(wl, W.free_list_order(wl))
    k, v = W.prompt_kv(wl, 1)
    a = oracle.HostPool(wl.num_blocks, 16, wl.num_kv_heads, wl.head_dim, "f16")
    b = oracle.HostPool(wl.num_blocks, 16, wl.num_kv_heads, wl.head_dim, "f16")
    a.reshape_and_cache(k, v, "f16", p["prompt_slots"][1])
    perm = np.random.default_rng(0).permutation(k.shape[0])
    b.reshape_and_cache(k[perm].contiguous(), v[perm].contiguous(), "f16", p["prompt_slots"][1][perm])
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)


def test_copy_blocks_copies_whole_blocks_only():
    pool = oracle.HostPool(6, 16, 2, 64, "f16", fill=0)
    rng = np.random.default_rng(1)
    pool.k[:] = rng.integers(0, 255, pool.k.shape, dtype=np.uint8)
    pool.v[:] = rng.integers(0, 255, pool.v.shape, dtype=np.uint8)
    k0, v0 = pool.k.copy(), pool.v.copy()
    pool.copy_blocks(np.array([[1, 4], [3, 0]], np.int32))
    bb = pool.block_bytes
    K0, K1 = k0.reshape(6, bb), pool.k.reshape(6, bb)
    V0, V1 = v0.reshape(6, bb), pool.v.reshape(6, bb)
    assert np.array_equal(K1[4], K0[1]) and np.array_equal(K1[0], K0[3])
    assert np.array_equal(V1[4], V0[1]) and np.array_equal(V1[0], V0[3])
    for b in (1, 2, 3, 5):
        assert np.array_equal(K1[b], K0[b]) and np.array_equal(V1[b], V0[b])


def test_kv_footprint_formula():
    g = _golden("kv_footprint.json")
    per_tok = oracle.kv_footprint_bytes(g["layers"], g["heads"], g["head_dim"], 1, g["dtype_bytes"])
    assert per_tok == g["bytes_per_token"]
    assert oracle.kv_footprint_bytes(g["layers"], g["heads"], g["head_dim"], 1024, 2) / 2 ** 20 == g["tokens_1024_MiB"]
    assert 16 * oracle.kv_footprint_bytes(40, 40, 128, 1024, 2) / 2 ** 20 == g["concurrent_16_of_1024_MiB"]
    per_seq = oracle.kv_footprint_bytes(40, 40, 128, g["per_sequence_GB_tokens"], 2) / 1e9
    assert abs(per_seq - g["per_sequence_GB_approx"]) < 0.05


def test_footprint_matches_pool_bytes_per_token():
    """One layer of the LLaMA-13B-shaped workload: a pool block holds
    block_size tokens, so K+V bytes per token = 2 * heads * head_dim * bytes."""
    wl = W.config_c2()
    pool_block_bytes = wl.num_kv_heads * wl.block_size * wl.head_dim * 2
    assert 2 * pool_block_bytes / wl.block_size == oracle.kv_footprint_bytes(1, 40, 128, 1, 2) == 20480


def test_swap_out_and_in_moves_whole_blocks():
    """Swap out copies pool blocks to the named host blocks, swap in copies
    host blocks back to the named pool blocks; nothing else changes.  Checked
    against numpy block slicing of the same bytes."""
    pool = oracle.HostPool(6, 16, 2, 64, "bf16", fill=0)
    rng = np.random.default_rng(3)
    pool.k[:] = rng.integers(0, 255, pool.k.shape, dtype=np.uint8)
    pool.v[:] = rng.integers(0, 255, pool.v.shape, dtype=np.uint8)
    bb = pool.block_bytes
    hk = np.zeros(4 * bb, np.uint8)
    hv = np.zeros(4 * bb, np.uint8)
    k0, v0 = pool.k.copy(), pool.v.copy()
    pool.swap(hk, hv, np.array([[5, 0], [1, 3]], np.int32), out=True)
    assert np.array_equal(hk.reshape(4, bb)[0], k0.reshape(6, bb)[5])
    assert np.array_equal(hv.reshape(4, bb)[3], v0.reshape(6, bb)[1])
    assert not hk.reshape(4, bb)[1].any() and not hk.reshape(4, bb)[2].any()
    assert np.array_equal(pool.k, k0) and np.array_equal(pool.v, v0)
    # bring host block 3 back into pool block 2 and host block 0 into pool block 4
    pool.swap(hk, hv, np.array([[3, 2], [0, 4]], np.int32), out=False)
    K, K0 = pool.k.reshape(6, bb), k0.reshape(6, bb)
    V, V0 = pool.v.reshape(6, bb), v0.reshape(6, bb)
    assert np.array_equal(K[2], K0[1]) and np.array_equal(V[2], V0[1])
    assert np.array_equal(K[4], K0[5]) and np.array_equal(V[4], V0[5])
    for b in (0, 1, 3, 5):
        assert np.array_equal(K[b], K0[b]) and np.array_equal(V[b], V0[b])
    with pytest.raises(oracle.OracleError):
        pool.swap(hk, hv, np.array([[0, 4]], np.int32), out=True)   # host has 4 blocks


def test_swap_round_trip_restores_decode():
    """Swapping a sequence's blocks out and back in to other physical blocks,
    with its table rewritten, leaves its decode output bit-identical."""
    wl = W.small_configs()["c2s_f16"]
    run = OracleRun(wl)
    base = run.decode()
    s = int(np.argmin(wl.context_lens))
    blocks = run.tables[s][run.tables[s] >= 0]
    used = set(run.tables[run.tables >= 0].tolist())
    free = [b for b in range(wl.num_blocks) if b not in used][:len(blocks)]
    assert len(free) == len(blocks)
    bb = run.pool.block_bytes
    hk = np.zeros(len(blocks) * bb, np.uint8)
    hv = np.zeros_like(hk)
    run.pool.swap(hk, hv, np.stack([blocks, np.arange(len(blocks))], 1), out=True)
    run.pool.swap(hk, hv, np.stack([np.arange(len(blocks)), free], 1), out=False)
    tables = run.tables.copy()
    tables[s, :len(blocks)] = free
    got = run.pool.decode(run.q, wl.q_dtype, tables, wl.context_lens, wl.scale, wl.num_q_heads)
    np.testing.assert_array_equal(got, base)
