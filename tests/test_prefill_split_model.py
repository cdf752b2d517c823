"""CPU model of the multi-token (prefill) kernel's work split.

Replays the index arithmetic of each worker wavefront: the per-sequence row
tiles (16 / G new tokens x G query heads), the blocks each tile reads (up to
the position of its last token), the flattened (kv head, sequence, tile,
block) stream cut into chunks, partial records, arrival counters and merges.
Checks that every index stays inside its buffer (table rows, q/out rows,
record slots, counters), that every block of every tile is streamed exactly
once, and that every (query row, query head) output is written exactly once,
for consistent and inconsistent query_start arrays.
"""
import numpy as np
import pytest

COUNTER_SLOTS = 65536
WAVES_PER_CU = 8      # one-wave workers, 16-row tiles
GROUPS_PER_CU = 1     # multi-wave work-groups: 128-row blocks (64 for head_dim 256)


def workers_for(num_cus, rows=16):
    w = num_cus * (WAVES_PER_CU if rows == 16 else GROUPS_PER_CU)
    w = max(8, (w + 7) & ~7)
    return min(w, COUNTER_SLOTS)


def lengths(ctx, qs, total_q, max_len):
    """(n, m, q0) per sequence, clamped as the kernel clamps them."""
    out = []
    for s in range(len(ctx)):
        n = min(max(int(ctx[s]), 0), max_len)
        a = min(max(int(qs[s]), 0), total_q)
        b = min(max(int(qs[s + 1]), a), total_q)
        out.append((n, min(b - a, n), a))
    return out


def tile_limit(n, m, Q, r):
    return n - m + min((r + 1) * Q, m)


def tiles_of(n, m, Q, bs):
    """Blocks read by each row tile of a sequence."""
    return [-(-tile_limit(n, m, Q, r) // bs) for r in range(-(-m // Q))]


def replay(ctx, qs, total_q, hkv, G, max_blocks, bs, num_cus=256, rows=16):
    """rows = 16: one-wave 16-row tiles; rows = 64 / 128: work-group row
    blocks (row j of block rb is token rb * (rows / G) + j / G, head j % G)."""
    Q = rows // G
    S = len(ctx)
    max_len = max_blocks * bs
    W = workers_for(num_cus, rows)
    # host bound on a consistent stream
    tiles_bound = -(-total_q * G // 16) + S
    assert tiles_bound * max_blocks * hkv <= (1 << 30)
    L = lengths(ctx, qs, total_q, max_len)
    per_seq = [tiles_of(n, m, Q, bs) for n, m, _ in L]
    nbs = [sum(t) for t in per_seq]
    assert all(x <= (1 << 30) for x in nbs)
    total = sum(nbs)
    if total * hkv > (1 << 30):
        return None            # the kernel computes nothing
    T = total * hkv
    if T == 0:
        return None
    chunk = max(1, -(-T // W))
    nv = -(-T // chunk)
    per_round = (nv + 7) & ~7
    assert per_round <= W
    # the stream, in order: (h, s, r, block offset)
    streamed = {}
    written = np.zeros((total_q, hkv * G), dtype=np.int32)
    records = {}
    counters = np.zeros(COUNTER_SLOTS, dtype=np.int32)
    seen = set()
    order = list(np.random.default_rng(1).permutation(W))
    for bid in order:
        bid = int(bid)
        if bid >= per_round:
            continue
        v = (bid & 7) * (per_round >> 3) + (bid >> 3)
        if v >= nv:
            continue
        assert v not in seen
        seen.add(v)
        start = v * chunk
        end = min(start + chunk, T)
        h, rr = divmod(start, total)
        pre = np.concatenate([[0], np.cumsum(nbs)])
        s = next(i for i in range(S) if nbs[i] > 0 and pre[i] <= rr < pre[i] + nbs[i])
        n, m, q0 = L[s]
        r, off = 0, rr - pre[s]
        while off >= per_seq[s][r]:
            off -= per_seq[s][r]
            r += 1
        pos = start
        while True:
            nb = per_seq[s][r]
            ln = min(nb - off, end - pos)
            assert ln >= 1 and off + ln <= nb <= max_blocks
            for b in range(off, off + ln):
                key = (h, s, r, b)
                streamed[key] = streamed.get(key, 0) + 1
            out_rows = []
            for j in range(rows):
                tok = j // G
                if r * Q + tok < m:
                    row = q0 + r * Q + tok
                    assert 0 <= row < total_q
                    out_rows.append((row, h * G + j % G))
            if off == 0 and off + ln == nb:
                for row in out_rows:
                    written[row] += 1
            else:
                slot = 2 * v + (0 if pos == start else 1)
                assert slot < 2 * W and slot not in records
                records[slot] = (h, s, r)
                seg_start = pos - off
                first_w, last_w = seg_start // chunk, (seg_start + nb - 1) // chunk
                assert first_w < last_w < nv
                counters[first_w] += 1
                if counters[first_w] - 1 == last_w - first_w:
                    for u in range(first_w, last_w + 1):
                        k = 0 if u * chunk >= seg_start else 1
                        assert records.get(2 * u + k) == (h, s, r)
                    for row in out_rows:
                        written[row] += 1
                    counters[first_w] = 0
            pos += ln
            if pos >= end:
                break
            off = 0
            r += 1
            if r * Q < m:
                continue
            r = 0
            while True:
                s += 1
                if s == S:
                    s = 0
                    h += 1
                    assert h < hkv
                n, m, q0 = L[s]
                if m > 0:
                    break
    assert seen == set(range(nv))
    for h in range(hkv):
        for s in range(S):
            for r, nb in enumerate(per_seq[s]):
                for b in range(nb):
                    assert streamed.get((h, s, r, b)) == 1
    assert sum(streamed.values()) == T
    assert not counters.any()
    return written


def _consistent(ctx, m):
    qs = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
    return qs, int(qs[-1])


@pytest.mark.parametrize("rows", [16, 64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("bs", [16, 32])
def test_consistent_rows_written_once(G, bs, rows):
    rng = np.random.default_rng(G * 100 + bs)
    for _ in range(4):
        S = int(rng.integers(1, 12))
        m = rng.integers(0, 70, size=S)
        ctx = m + rng.integers(0, 300, size=S)
        ctx = np.maximum(ctx, 1)
        qs, tq = _consistent(ctx, m)
        mb = int(-(-ctx.max() // bs)) + int(rng.integers(0, 3))
        hkv = int(rng.integers(1, 4))
        for cus in (1, 4, 256):
            written = replay(ctx, qs, tq, hkv, G, mb, bs, num_cus=cus, rows=rows)
            if tq:
                assert written is not None and (written == 1).all()


@pytest.mark.parametrize("rows", [16, 64, 128])
def test_inconsistent_query_start_stays_in_bounds(rows):
    rng = np.random.default_rng(7)
    for _ in range(20):
        S = int(rng.integers(1, 9))
        ctx = rng.integers(-5, 200, size=S)
        qs = rng.integers(-20, 60, size=S + 1)
        tq = int(rng.integers(1, 50))
        replay(ctx, qs, tq, 2, 4, 16, 16, num_cus=2, rows=rows)   # asserts every index in range


@pytest.mark.parametrize("rows", [16, 64, 128])
def test_workload_shapes_fit(rows):
    import workloads as W
    for wl in list(W.multi_token_configs().values()) + list(W.small_multi_token_configs().values()):
        written = replay(wl.context_lens, wl.query_start, wl.total_q, wl.num_kv_heads, wl.group,
                         wl.max_blocks_per_seq, wl.block_size, rows=rows)
        assert (written == 1).all()


RANK_SEQS = 256   # sequences the unit kernel ranks


def replay_units(ctx, qs, total_q, hkv, G, D=128):
    """Unit mode: one work-group per whole row block.  Up to RANK_SEQS
    sequences the list is (rank by context length, longest first; kv head;
    row block last-first), dealt to the XCDs in runs of c units; above it
    the units keep (kv head, sequence, row block) order in contiguous ranges
    per XCD.  Checks the host's grid and that every row block is computed
    exactly once; returns the units each XCD runs, in dispatch order."""
    W = 8 if D <= 128 else 4
    rows = 16 * W
    QB = rows // G
    S = len(ctx)
    L = lengths(ctx, qs, total_q, 1 << 30)
    cnt = [-(-m // QB) for _, m, _ in L]
    per_head = sum(cnt)
    U = per_head * hkv
    bound = (total_q * G // rows + S + 1) * hkv
    grid = (bound + 7) & ~7
    seen = set()
    order = [[] for _ in range(8)]
    if S <= RANK_SEQS:
        c = min(16, max(1, -(-(total_q * G) // (rows * S))))
        grid = 8 * (-(-bound // (8 * c))) * c
        key = [n if m > 0 else -1 for n, m, _ in L]
        ranked = sorted(range(S), key=lambda j: (-key[j], j))
        lst = [(h, s, rb) for s in ranked for h in range(hkv) for rb in reversed(range(cnt[s]))]
        for b in range(grid):
            x, k = b & 7, b >> 3
            i = (k // c) * 8 * c + x * c + k % c
            if i >= len(lst):
                continue
            assert lst[i] not in seen
            seen.add(lst[i])
            order[x].append((k, lst[i]))
    else:
        per_xcd = (U + 7) >> 3
        pre = np.concatenate([[0], np.cumsum(cnt)])
        for b in range(grid):
            k, u = b >> 3, (b & 7) * per_xcd + (b >> 3)
            if k >= per_xcd or u >= U:
                continue
            h, r = divmod(u, per_head)
            s = next(i for i in range(S) if cnt[i] > 0 and pre[i] <= r < pre[i] + cnt[i])
            key = (h, s, r - pre[s])
            assert key not in seen
            seen.add(key)
            order[b & 7].append((k, key))
    return seen, U, [[u for _, u in sorted(o)] for o in order]


@pytest.mark.parametrize("G", [1, 4, 16])
def test_units_cover_every_row_block_once(G):
    rng = np.random.default_rng(G)
    for _ in range(5):
        S = int(rng.integers(1, 40))
        m = rng.integers(0, 700, size=S)
        ctx = m + rng.integers(0, 300, size=S)
        ctx = np.maximum(ctx, 1)
        qs = np.concatenate([[0], np.cumsum(m)])
        for D in (128, 256):
            seen, U, _ = replay_units(ctx, qs, int(qs[-1]), int(rng.integers(1, 9)), G, D)
            assert len(seen) == U


@pytest.mark.parametrize("S", [255, 256, 257, 300])
def test_units_around_the_rank_limit(S):
    """Both orders, at and around the number of sequences the kernel ranks,
    with sequences that have no new rows."""
    rng = np.random.default_rng(S)
    m = rng.integers(0, 300, size=S)
    m[::7] = 0
    ctx = np.maximum(m + rng.integers(0, 200, size=S), 1)
    qs = np.concatenate([[0], np.cumsum(m)])
    for hkv in (1, 3, 8):
        seen, U, _ = replay_units(ctx, qs, int(qs[-1]), hkv, 4)
        assert len(seen) == U


def test_ranked_units_run_longest_first_on_every_xcd():
    """Each XCD receives its units by non-increasing context length of their
    sequence, a sequence's row blocks last (longest) first, and the (sequence,
    kv head) pairs of the chunked-prefill batch stay whole on one XCD."""
    import workloads as W
    for wl in W.multi_token_configs().values():
        if wl.num_seqs > RANK_SEQS:
            continue
        ctx, qs = np.asarray(wl.context_lens), np.asarray(wl.query_start)
        _, _, order = replay_units(ctx, qs, wl.total_q, wl.num_kv_heads, wl.group)
        xcd_of = {}
        for x, units in enumerate(order):
            for (h0, s0, rb0), (h1, s1, rb1) in zip(units, units[1:]):
                assert ctx[s0] >= ctx[s1], f"{wl.name}: XCD {x} not longest first"
                assert (h0, s0) != (h1, s1) or rb0 > rb1
            for h, s, rb in units:
                xcd_of.setdefault((h, s), set()).add(x)
        if wl.name.startswith("p1"):
            assert all(len(v) == 1 for v in xcd_of.values())
