"""CPU model of the decode kernel's work split and merge bookkeeping.

Replays, in Python, the index arithmetic each worker wavefront performs
(which blocks it streams, which partial slot it writes, which arrival counter
it bumps, which records the merging worker reads) for many length mixes, and
checks that every index stays inside its buffer, every block of every
(kv head, sequence) run is streamed exactly once, every run's output is
written exactly once, and the merger reads exactly the records its run's
workers wrote.  This is the host-side check of the grid and indexes before
they run on the device.
"""
import numpy as np
import pytest

COUNTER_SLOTS = 65536
SHARED_SPLIT = 4


def plan(num_seqs, hkv, max_blocks, bs, partition_tokens, num_cus=256, waves_per_cu=16):
    """(chunk or 0, launched workers, record chunks the workspace holds)."""
    units = num_seqs * hkv * max_blocks
    if partition_tokens > 0:
        chunk = partition_tokens // bs
        min_chunk = (units + COUNTER_SLOTS - 9) // (COUNTER_SLOTS - 8)
        chunk = max(chunk, min_chunk)
        workers = -(-units // chunk)
    else:
        chunk = 0
        workers = min(num_cus * waves_per_cu, units)
    workers = max(workers, 1)
    workers = (workers + 7) & ~7
    chunks = workers if partition_tokens > 0 else workers * SHARED_SPLIT
    assert chunks <= COUNTER_SLOTS
    return chunk, workers, chunks


def replay(lens, hkv, max_blocks, bs, partition_tokens, shared=False, **kw):
    S = len(lens)
    max_len = max_blocks * bs
    n = np.clip(lens, 0, max_len)
    nb = -(-n // bs)
    total = int(nb.sum())
    T = total * hkv
    chunk0, W, CH = plan(S, hkv, max_blocks, bs, partition_tokens, **kw)
    rounds = SHARED_SPLIT if (chunk0 == 0 and shared) else 1
    chunk = chunk0 if chunk0 > 0 else max(1, -(-T // (W * rounds)))
    nv = -(-T // chunk)
    per_round = ((nv + 7) & ~7) if rounds == 1 else W
    assert per_round <= W and nv <= rounds * per_round
    pre = np.concatenate([[0], np.cumsum(nb)])
    streamed = np.zeros((hkv, S, max_blocks), dtype=np.int32)
    written = np.zeros((hkv, S), dtype=np.int32)
    records = {}         # (slot) -> (h, s) written
    counters = np.zeros(COUNTER_SLOTS, dtype=np.int32)
    seen_workers = set()
    # chunks in dispatch order; the merge decision depends only on counts,
    # so any completion order gives the same result -- use a shuffled one
    order = [(rd, bid) for rd in range(rounds) for bid in range(W)]
    order = [order[i] for i in np.random.default_rng(0).permutation(len(order))]
    for rd, bid in order:
        if bid >= per_round:
            continue
        w = rd * per_round + (bid & 7) * (per_round >> 3) + (bid >> 3)
        if w >= nv:
            continue
        assert 0 <= w < CH and w not in seen_workers
        seen_workers.add(w)
        start = w * chunk
        if start >= T:
            continue
        end = min(start + chunk, T)
        h = start // total
        r = start - h * total
        s = int(np.searchsorted(pre, r, side="right") - 1)
        while nb[s] == 0:
            s += 1
        off = r - pre[s]
        pos = start
        while True:
            ln = min(nb[s] - off, end - pos)
            assert ln >= 1
            for b in range(off, off + ln):
                assert 0 <= b < max_blocks           # table row bound
                streamed[h, s, b] += 1
            if off == 0 and off + ln == nb[s]:
                written[h, s] += 1
            else:
                k = 0 if pos == start else 1
                slot = 2 * w + k
                assert slot < 2 * CH and slot not in records
                records[slot] = (h, s)
                seg_start = pos - off
                first_w, last_w = seg_start // chunk, (seg_start + nb[s] - 1) // chunk
                assert first_w < last_w < nv and first_w < COUNTER_SLOTS
                counters[first_w] += 1
                if counters[first_w] - 1 == last_w - first_w:
                    got = set()
                    for v in range(first_w, last_w + 1):
                        kk = 0 if v * chunk >= seg_start else 1
                        assert records.get(2 * v + kk) == (h, s), (v, kk)
                        got.add(v)
                    assert len(got) == last_w - first_w + 1
                    written[h, s] += 1
                    counters[first_w] = 0
            pos += ln
            if pos >= end:
                break
            while True:
                s += 1
                if s == S:
                    s = 0
                    h += 1
                    assert h < hkv
                if nb[s] > 0:
                    break
            off = 0
    assert seen_workers == set(range(nv))
    for h in range(hkv):
        for s in range(S):
            assert (streamed[h, s, :nb[s]] == 1).all() and (streamed[h, s, nb[s]:] == 0).all()
            assert written[h, s] == (1 if nb[s] > 0 else 0)
    assert not counters.any()
    return W, chunk


CASES = [
    ([1, 15, 16, 33], 4, 3, 16, 0),
    ([1, 15, 16, 33], 4, 3, 16, 16),
    ([700, 5, 2048, 130, 0, 64], 3, 128, 16, 0),
    ([700, 5, 2048, 130, 0, 64], 3, 128, 16, 16),
    ([700, 5, 2048, 130, 0, 64], 3, 128, 16, 48),
    ([4096] * 3 + [16] * 40, 2, 256, 16, 0),
    ([9000, 3], 1, 64, 16, 0),              # length above the table: clamped
    ([0, 0, 0], 2, 4, 16, 0),
]


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_split_bookkeeping(case, shared):
    lens, hkv, mb, bs, pt = case
    replay(np.asarray(lens), hkv, mb, bs, pt, shared=shared)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("cus", [4, 256])
def test_split_bookkeeping_random(seed, cus):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 300))
    bs = int(rng.choice([8, 16, 32, 64]))
    mb = int(rng.integers(1, 80))
    lens = rng.integers(0, mb * bs + 1, size=S)
    hkv = int(rng.integers(1, 9))
    pt = int(rng.choice([0, bs, 3 * bs, 32 * bs]))
    replay(lens, hkv, mb, bs, pt, shared=bool(seed % 2), num_cus=cus, waves_per_cu=int(rng.integers(1, 20)))


def test_workload_shapes_fit():
    import workloads as W
    for wl in W.full_configs().values():
        shared = len(set(wl.parent)) < wl.num_seqs
        replay(wl.context_lens, wl.num_kv_heads, wl.max_blocks_per_seq, wl.block_size, wl.partition_tokens,
               shared=shared)
