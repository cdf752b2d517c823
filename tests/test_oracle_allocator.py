"""Pins for the oracle's block-manager model (oracle/allocator.py): values
and invariants the pages fix, checked on the model alone.

* Waste bound: a sequence of n tokens holds ceil(n/bs) blocks and wastes
  ceil(n/bs)*bs - n <= bs - 1 slots ("vLLM — 把操作系统的分页搬进 GPU KV
  cache", core mechanism 1; "vLLM 与 KV Cache", how-it-works).
* Parallel sampling (golden fixture): n = 4 candidates share the prompt's
  blocks with ref_count 4; the first step copies 3 blocks; memory grows by
  the copies only.
* Prefix caching (golden fixture): the shared opening's first 16 tokens are
  reused; a different opening, or the same tokens with a different extra
  hash, reuses nothing.
* LRU: cached blocks nobody references are evicted least recently released
  first, never while referenced; an evicted parent makes its descendants
  unreachable.
* Conservation under random operations: every block is free, cached or
  referenced; reference counts equal table entries.
* Without prefix caching the model reproduces the oracle's workload paging
  plan (block tables, slots, copy pairs).
"""
import json
import os

import numpy as np
import pytest

import workloads as W
from conftest import ROOT
from oracle.allocator import AllocatorModel, NoBlocks
from oracle.paging import plan as paging_plan

GOLDEN = os.path.join(ROOT, "tests", "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _pin_waste_bound(Model, bs):
    m = Model(4096, bs)
    for sid, n in enumerate(range(1, 200, 7)):
        m.add_sequence(sid, n)
        assert len(m.table(sid)) == -(-n // bs)
        waste = len(m.table(sid)) * bs - n
        assert 0 <= waste <= bs - 1
        assert waste == (-n) % bs


def _pin_parallel_sampling(Model):
    g = _golden("parallel_sampling_cow.json")
    n, bs, P = g["n"], 16, 1023
    m = Model(256, bs)
    m.add_sequence(0, P)
    kids = list(range(1, n + 1))
    m.fork(0, kids)
    m.release(0)
    last = m.table(1)[-1]
    assert m.ref[last] == g["ref_count_after_fork"]
    used_before = m.stats()["used_blocks"]
    pairs = [m.append(k, 1)[1] for k in kids]
    assert sum(p is not None for p in pairs) == g["copies_on_first_step"]
    assert pairs[-1] is None and m.ref[last] == 1          # the last writer writes in place
    assert m.stats()["used_blocks"] == used_before + g["copies_on_first_step"]
    # all candidates still share every full prompt block
    for b in m.table(1)[:-1]:
        assert m.ref[b] == n


def _pin_prefix_cache(Model):
    g = _golden("prefix_cache_example.json")
    bs = g["block_size"]
    rng = np.random.default_rng(0)
    opening = rng.integers(0, 32000, size=20).tolist()      # 16 <= shared opening < 32
    r0 = opening + rng.integers(0, 32000, size=30).tolist()
    r1 = opening + rng.integers(0, 32000, size=25).tolist()
    r2 = rng.integers(0, 32000, size=40).tolist()
    m = Model(64, bs, prefix_caching=True)
    assert m.add_sequence(0, len(r0), r0)[1] == 0
    s1, c1 = m.add_sequence(1, len(r1), r1)
    assert c1 == g["request1_reused_tokens"]
    assert m.table(1)[0] == m.table(0)[0] and m.table(1)[1] != m.table(0)[1]
    assert s1[:bs] == [m.table(0)[0] * bs + i for i in range(bs)]
    assert m.add_sequence(2, len(r2), r2)[1] == g["request2_reused_tokens"]
    assert "extra" in g["match_inputs"]
    assert m.add_sequence(3, len(r0), r0, extra=7)[1] == 0     # same tokens, other extra input
    assert m.add_sequence(4, len(r0), r0)[1] == (len(r0) // bs) * bs


def _pin_lru(Model):
    bs = 4
    m = Model(7, bs, prefix_caching=True)
    a, b = list(range(8)), list(range(100, 108))            # two prompts of 2 full blocks
    m.add_sequence(0, 8, a)
    m.add_sequence(1, 8, b)
    ta, tb = m.table(0), m.table(1)
    m.release(0)                                            # released last-to-first: ta[1], ta[0]
    m.release(1)                                            # then tb[1], tb[0]
    assert m.lru == [ta[1], ta[0], tb[1], tb[0]] and len(m.free) == 3
    m.add_sequence(2, 16)                                   # 4 blocks: 3 free + 1 eviction
    assert m.evictions == 1 and ta[1] not in m.lru and m.registration[ta[1]] == 0
    assert m.add_sequence(3, 4, a[:4])[1] == 4              # a's first block is still cached
    assert m.add_sequence(4, 8, b)[1] == 8                  # b intact
    assert m.available() == 0
    with pytest.raises(NoBlocks):                           # referenced cached blocks are never evicted
        m.add_sequence(5, 1)


def _pin_evicted_parent(Model):
    bs = 2
    m = Model(3, bs, prefix_caching=True)
    toks = [1, 2, 3, 4]
    m.add_sequence(0, 4, toks)
    t0 = m.table(0)
    m.release(0)                  # LRU: t0[1], t0[0]
    m.add_sequence(1, 2)          # takes the free block
    m.add_sequence(2, 2)          # evicts t0[1] (the child)
    m.release(2)
    m.add_sequence(3, 2)          # takes the free block again (plain free before cached)
    m.add_sequence(4, 2)          # evicts t0[0] (the parent)
    m.release(1), m.release(3), m.release(4)
    assert m.add_sequence(5, 4, toks)[1] == 0


def _pin_conservation(Model):
    rng = np.random.default_rng(3)
    for trial in range(5):
        bs = int(rng.choice([2, 4, 16]))
        N = int(rng.integers(8, 80))
        m = Model(N, bs, free_order=rng.permutation(N).tolist(), prefix_caching=bool(trial % 2))
        live, nid = [], 0
        for _ in range(300):
            op = rng.integers(0, 4)
            try:
                if op == 0 or not live:
                    n = int(rng.integers(0, 3 * bs + 2))
                    toks = rng.integers(0, 3, size=n).tolist()
                    m.add_sequence(nid, n, toks if rng.random() < 0.8 else None)
                    live.append(nid)
                    nid += 1
                elif op == 1:
                    m.fork(live[int(rng.integers(len(live)))], [nid])
                    live.append(nid)
                    nid += 1
                elif op == 2:
                    s = live[int(rng.integers(len(live)))]
                    k = int(rng.integers(1, 2 * bs))
                    m.append(s, k, rng.integers(0, 3, size=k).tolist())
                else:
                    m.release(live.pop(int(rng.integers(len(live)))))
            except NoBlocks:
                pass
            st = m.stats()
            assert st["free_blocks"] + st["cached_blocks"] + st["used_blocks"] == N
            assert sum(m.ref) == st["table_entries"]
            assert set(m.free).isdisjoint(m.lru)
            assert all(m.ref[b] == 0 for b in list(m.free) + m.lru)
            assert all(m.registration[b] for b in m.lru)


def _pin_paging_plan(Model, name):
    wl = W.small_configs()[name]
    order = W.free_list_order(wl)
    ref = paging_plan(wl, order)
    m = Model(wl.num_blocks, wl.block_size, free_order=order)
    for p, L in enumerate(wl.prompt_lens):
        slots, _ = m.add_sequence(("p", p), L)
        np.testing.assert_array_equal(slots, ref["prompt_slots"][p])
    kids = {}
    for s, p in enumerate(wl.parent):
        kids.setdefault(p, []).append(("s", s))
    for p in range(wl.num_prompts):
        m.fork(("p", p), kids.get(p, []))
        m.release(("p", p))
    slots, pairs = [], []
    for s in range(wl.num_seqs):
        got, pair = m.append(("s", s), 1)
        slots += got
        if pair:
            pairs.append(pair)
    np.testing.assert_array_equal(slots, ref["new_slots"])
    np.testing.assert_array_equal(np.asarray(pairs, dtype=np.int32).reshape(-1, 2), ref["pairs"])
    for s in range(wl.num_seqs):
        t = m.table(("s", s))
        np.testing.assert_array_equal(t, ref["tables"][s][:len(t)])


def _pin_parent_is_part_of_the_key(Model):
    """A block whose tokens equal another cached block's tokens but whose
    parent differs is a different prefix: no hit."""
    bs = 4
    m = Model(16, bs, prefix_caching=True)
    b1, b2 = [1, 2, 3, 4], [5, 6, 7, 8]
    m.add_sequence(0, 8, b1 + b2)
    assert m.add_sequence(1, 8, b2 + b1)[1] == 0
    assert m.add_sequence(2, 8, b1 + b1)[1] == 4


def _pin_cow_copies_partial_block_only(Model):
    """Forked candidates sharing a full last block need no copy."""
    m = Model(16, 4)
    m.add_sequence(0, 8)
    m.fork(0, [1, 2])
    assert m.append(1, 1)[1] is None and m.append(2, 1)[1] is None


PINS = [
    *[(_pin_waste_bound, (bs,)) for bs in (8, 16, 32)],
    (_pin_parallel_sampling, ()),
    (_pin_prefix_cache, ()),
    (_pin_lru, ()),
    (_pin_evicted_parent, ()),
    (_pin_conservation, ()),
    *[(_pin_paging_plan, (n,)) for n in ("c1_tiny_f32", "c4s_cow_f16", "c3s_bf16_bs16")],
    (_pin_parent_is_part_of_the_key, ()),
    (_pin_cow_copies_partial_block_only, ()),
]


@pytest.mark.parametrize("pin,args", PINS, ids=[f"{p.__name__[5:]}{a}" for p, a in PINS])
def test_pin(pin, args):
    pin(AllocatorModel, *args)


MUTANTS = {
    "lifo_free_list": ("b = self.free.popleft()", "b = self.free.pop()"),
    "evict_most_recent": ("b = self.lru.pop(0)", "b = self.lru.pop()"),
    "release_first_to_last": ("for b in reversed(s.table):", "for b in s.table:"),
    "cow_keeps_count": ("            self.ref[s.table[-1]] -= 1\n", ""),
    "key_ignores_extra": ("key = (parent, s.extra, tuple(s.pending))", "key = (parent, 0, tuple(s.pending))"),
    "lookup_ignores_extra": ("key = (parent, extra, tuple(", "key = (parent, 0, tuple("),
    "key_ignores_parent": ("key = (parent, s.extra, tuple(s.pending))", "key = (0, s.extra, tuple(s.pending))"),
    "lookup_ignores_parent": ("key = (parent, extra, tuple(", "key = (0, extra, tuple("),
    "evict_referenced": ("if self.ref[b] == 0:\n            if self.registration[b]:",
                         "if self.ref[b] <= 1:\n            if self.registration[b]:"),
    "no_reuse": ("hits.append(self.cache[key])", "break"),
    "cow_always": ("elif self.ref[s.table[-1]] > 1:", "elif self.ref[s.table[-1]] >= 1:"),
    "evict_before_free": ("        if self.free:\n            b = self.free.popleft()",
                          "        if not self.lru and self.free:\n            b = self.free.popleft()"),
}


def test_pins_reject_every_mutant(tmp_path):
    import importlib.util
    import oracle.allocator as A
    src = open(A.__file__).read()
    survivors = []
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, name
        f = tmp_path / f"alloc_{name}.py"
        f.write_text(src.replace(old, new))
        spec = importlib.util.spec_from_file_location(f"alloc_{name}", f)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        caught = False
        for pin, args in PINS:
            try:
                pin(mod.AllocatorModel, *args)
            except (AssertionError, mod.NoBlocks, KeyError, IndexError, ValueError):
                caught = True
                break
        if not caught:
            survivors.append(name)
    assert not survivors, f"mutants not caught by the pins: {survivors}"
