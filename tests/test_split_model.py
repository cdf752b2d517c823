"""CPU model of the decode launch's work plan, work split and merge bookkeeping.

Replays, in Python and with the device code's integer formulas, what the
plan kernel writes (items, per-sequence entries, worker descriptors, record
rows) and what each worker wavefront then does with it: which blocks it
streams, which partial records it writes, which arrival counters it bumps and
which records the merging worker reads.  For many length mixes, tables with
and without shared prefixes, splits and grid sizes it checks that every index
stays inside its buffer, every block of every (kv head, sequence) is
streamed exactly once (a group's shared prefix once for all its members),
every output is written exactly once, and every merge reads exactly the
records its output's pieces wrote.  This is the host-side check of the grid
and indexes before they run on the device.
"""
import numpy as np
import pytest

COUNTER_SLOTS = 65536
SHARED_SPLIT = 4


class Grid:
    """ChunkGrid: spans of `span` blocks, each cut into q chunks of `chunk`."""

    def __init__(self, chunk, span, q):
        self.chunk, self.span, self.q = chunk, span, q

    def of(self, x):
        u, r = divmod(x, self.span)
        return u * self.q + r // self.chunk

    def start(self, v):
        u, r = divmod(v, self.q)
        return u * self.span + r * self.chunk

    def end(self, v, T):
        u, r = divmod(v, self.q)
        return min(u * self.span + (r + 1) * self.chunk, (u + 1) * self.span, T)


def max_pieces(ln, chunk, span, q):
    return -(-ln // chunk) + 1 + (-(-ln // span) if q > 1 else 0)


def host_plan(S, hkv, max_blocks, bs, G, pt, num_cus=256, waves_per_cu=8, groupable=True):
    """make_plan in decode.hip: split, descriptor rounds, grouping limits."""
    units = S * hkv * max_blocks
    workers = num_cus * waves_per_cu
    if pt > 0:
        workers = max(min(workers, units), 1)
        workers = (workers + 7) & ~7
        chunk = pt // bs
        span_max = -(-units // workers)
        max_q = COUNTER_SLOTS // workers
        if -(-span_max // chunk) > max_q:
            chunk = -(-span_max // max_q)
        desc_rounds = max(1, -(-span_max // chunk))
        chunks = workers * desc_rounds
    else:
        chunk = 0
        workers = max(min(workers, units), 1)
        workers = (workers + 7) & ~7
        desc_rounds = SHARED_SPLIT
        chunks = workers * SHARED_SPLIT
    assert chunks <= COUNTER_SLOTS
    grouping = groupable and G <= 8 and bs >= 16 and hkv * S <= COUNTER_SLOTS
    return {"chunk": chunk, "workers": workers, "desc_rounds": desc_rounds, "chunks": chunks,
            "max_members": 16 // G if grouping else 0,
            "grec_rows": (4 * hkv * S * G + 16 * min(chunks if pt > 0 else workers, 8192)) if grouping else 0,
            "flat_rows": 2 * chunks * G}


def device_plan(tables, lens, hkv, bs, num_blocks, G, hp, span_runs=False):
    """paged_decode_plan_kernel, sequentially (its scans give the same values)."""
    S, max_blocks = tables.shape
    max_len = max_blocks * bs
    n = np.clip(lens, 0, max_len).astype(np.int64)
    eq = np.zeros(S, bool)
    for s in range(1, S):
        b0, bp = int(tables[s, 0]), int(tables[s - 1, 0])
        eq[s] = n[s] > 0 and n[s - 1] > 0 and 0 <= b0 < num_blocks and b0 == bp
    M = hp["max_members"]
    grouped = bool(eq.any()) and M >= 2 and hkv * S <= COUNTER_SLOTS
    c = np.zeros(S, np.int64)
    gid = np.arange(S)
    groups = {}
    if grouped:
        for s in range(S):
            if not eq[s]:
                continue
            cap = min(n[s], n[s - 1]) // bs
            k = 0
            while k < cap and tables[s, k] == tables[s - 1, k]:
                k += 1
            c[s] = k
        run_start, g = 0, -1
        for s in range(S):
            if c[s] < 1:
                run_start = s
            lead = (s - run_start) % M == 0
            g += 1 if lead else 0
            gid[s] = g
        for s in range(S):
            if s > 0 and gid[s - 1] == gid[s]:
                continue
            k, m = 2**31 - 1, 1
            for j in range(1, M):
                if s + j >= S or gid[s + j] != gid[s]:
                    break
                k = min(k, int(c[s + j]))
                m += 1
            groups[int(gid[s])] = {"k": k, "m": m, "first": s}
        grouped = any(gr["m"] >= 2 and gr["k"] >= 1 for gr in groups.values())

    def real(s):
        gr = groups.get(int(gid[s]))
        return grouped and gr is not None and gr["m"] >= 2 and gr["k"] >= 1

    def lay_out(grouped_now):
        items, seqs, pos = [], [], 0
        for s in range(S):
            q = {"s_item": -1}
            if n[s] > 0:
                nb = -(-int(n[s]) // bs)
                k = groups[int(gid[s])]["k"] if (grouped_now and real(s)) else 0
                if k and groups[int(gid[s])]["first"] == s:
                    gr = groups[int(gid[s])]
                    gr["item"] = len(items)
                    items.append({"s": s, "off": 0, "len": k, "n": k * bs, "pos": pos, "m": gr["m"]})
                    pos += k
                if nb - k > 0:
                    q["s_item"] = len(items)
                    items.append({"s": s, "off": k, "len": nb - k, "n": int(n[s]), "pos": pos, "m": 0,
                                  "g_len": 0})
                    pos += nb - k
            seqs.append(q)
        return items, seqs, pos

    flags, RH = 0, 0
    for attempt in range(2):
        items, seqs, TB = lay_out(grouped)
        T = TB * hkv
        flags = 2 if grouped else (1 if eq.any() else 0)
        if hp["chunk"] > 0:
            span = max(1, -(-T // hp["workers"]))
            chunk = min(hp["chunk"], span)
            qn = -(-span // chunk)
            rounds = qn
        else:
            rounds = SHARED_SPLIT if flags & 1 else 1
            chunk = max(1, -(-T // (hp["workers"] * rounds)))
            span, qn = chunk, 1
        if not grouped:
            break
        RH = 0
        for s in range(S):
            q = seqs[s]
            if n[s] == 0:
                continue
            gr = groups[int(gid[s])]
            lead = real(s) and gr["first"] == s
            gp = max_pieces(gr["k"], chunk, span, qn) * gr["m"] * G if lead else 0
            if lead:
                items[gr["item"]]["rbase"] = RH
            if q["s_item"] >= 0:
                it = items[q["s_item"]]
                it["rbase"] = RH + gp
                RH += gp + max_pieces(it["len"], chunk, span, qn) * G
            else:
                RH += gp
        for s in range(S):
            q = seqs[s]
            if q["s_item"] >= 0 and real(s):
                gr = groups[int(gid[s])]
                gi = items[gr["item"]]
                si = items[q["s_item"]]
                si.update(member=s - gr["first"], g_pos=gi["pos"], g_len=gi["len"], g_rbase=gi["rbase"],
                          g_m=gi["m"])
        if RH * hkv <= hp["grec_rows"]:
            break
        grouped = False
    g = Grid(chunk, span, qn)
    W = hp["workers"]
    spans = -(-T // span)
    nid = spans * qn
    if qn > 1:
        per_round = (spans + 7) & ~7
        assert per_round <= W
        used_rounds = qn
    else:
        per_round = min(W, (-(-nid // rounds) + 7) & ~7)
        used_rounds = -(-nid // per_round) if nid else 0
        # every worker runs `rounds` or `rounds - 1` chunks
        assert nid == 0 or (used_rounds - 1) * per_round < nid <= used_rounds * per_round
    assert used_rounds <= hp["desc_rounds"] and nid <= hp["chunks"]
    q8 = per_round >> 3

    def slot(v):
        if qn > 1:
            u, rd = divmod(v, qn)
        else:
            rd, u = divmod(v, per_round)
        return rd, (u % q8) * 8 + u // q8

    one_pass = qn > 1 and span_runs and not grouped
    desc = {}
    for i, it in enumerate(items):
        for h in range(hkv):
            a = h * TB + it["pos"]
            e = a + it["len"]
            v = g.of(a)
            if g.start(v) < a:
                v += 1
            while v < nid and g.start(v) < e:
                if one_pass and v % qn:   # only each span's first chunk
                    v += 1
                    continue
                rd, wg = slot(v)
                assert 0 <= rd < used_rounds and 0 <= wg < W
                assert (rd, wg) not in desc
                desc[(rd, wg)] = {"v": v, "h": h, "i": i, "off": g.start(v) - a, "s": it["s"], "n": it["n"],
                                  "len": it["len"]}
                v += 1
    nv = sum(1 for v in range(nid) if g.start(v) < T and not (one_pass and v % qn))
    assert len(desc) == nv
    if qn > 1 and not one_pass:   # equal spans: every worker's share is within one block of the others'
        shares = {}
        for (rd, wg), d in desc.items():
            shares[wg] = shares.get(wg, 0) + g.end(d["v"], T) - g.start(d["v"])
        short = [x for x in shares.values() if x != span]
        assert len(shares) == spans and short in ([], [T - (spans - 1) * span])
    got = walk_descs(items, TB, hkv, g, rounds, W, one_pass=one_pass)
    keys = ("v", "h", "i", "off") if grouped else ("v", "h", "i", "off", "s", "len", "n")
    assert got.keys() == desc.keys()
    assert all(all(got[k][f] == desc[k][f] for f in keys) for k in desc)
    return {"items": items, "seqs": seqs, "desc": desc, "T": T, "TB": TB, "NI": len(items), "chunk": chunk,
            "span": span, "q": qn, "grid": g, "rounds": 1 if one_pass else used_rounds, "flags": flags, "RH": RH, "n": n,
            "groups": groups, "gid": gid, "grouped": grouped}


def walk_descs(items, TB, hkv, g, rounds, W, threads=1024, one_pass=False):
    """plan_write_descs as the device runs it: thread t takes worker slots
    t, t + threads, ... (stepping slot and round without divisions), and
    each slot with a chunk binary-searches its first item."""
    pos = [it["pos"] for it in items]
    NI = len(items)
    T = TB * hkv
    C, SP, Q = g.chunk, g.span, g.q
    spans = -(-T // SP)
    nid = spans * Q
    if Q > 1:
        per_round = (spans + 7) & ~7
        n_rounds = Q
    else:
        per_round = min(W, (-(-nid // rounds) + 7) & ~7)
        n_rounds = -(-nid // per_round) if nid else 0
    q8 = per_round >> 3

    def find(r):
        lo, hi = 0, NI
        while hi - lo > 1:
            mid = (lo + hi) >> 1
            if pos[mid] <= r:
                lo = mid
            else:
                hi = mid
        return lo

    out = {}
    n_slots = W if one_pass else max(n_rounds, 1) * W
    db, drd = threads % W, threads // W
    for t in range(threads):
        b, rd = t % W, t // W
        for k in range(t, n_slots, threads):
            assert (rd, b) == divmod(k, W)
            u = (b & 7) * q8 + (b >> 3)
            v = u * Q + rd if Q > 1 else rd * per_round + u
            st = u * SP + rd * C if Q > 1 else v * C
            if b < per_round and v < nid and st < T:
                assert g.start(v) == st
                h, r = divmod(st, TB)
                i = find(r)
                out[(rd, b)] = {"v": v, "h": h, "i": i, "off": r - pos[i], "s": items[i]["s"],
                                "len": items[i]["len"], "n": items[i]["n"]}
            b += db
            rd += drd
            if b >= W:
                b -= W
                rd += 1
    return out


def walk(pl, hkv, bs, G, hp, max_blocks, span_runs=False):
    """Every worker's chunks (decode_chunk / grouped_chunk) and merges.

    span_runs: flat plans with partitions as the matrix-core runs take them:
    a worker streams its whole span from its first round's chunk, and a run
    that crosses chunk boundaries leaves one record per chunk."""
    items, T, TB, NI, g = pl["items"], pl["T"], pl["TB"], pl["NI"], pl["grid"]
    n = pl["n"]
    S = len(n)
    nb = -(-n // bs)
    streamed = np.zeros((hkv, S, max(max_blocks, 1)), np.int32)
    shared_reads = {}
    written = np.zeros((hkv, S), np.int32)
    counters = {}
    recs = {}
    grouped = pl["flags"] & 2
    cap_rows = max(hp["grec_rows"], hp["flat_rows"])

    def pieces(h, ipos, ilen):
        a = h * TB + ipos
        return g.of(a + ilen - 1) - g.of(a) + 1

    order = sorted(pl["desc"].items(), key=lambda kv: np.random.default_rng(kv[1]["v"]).random())
    span_runs = span_runs and g.q > 1 and not grouped
    for (rd, wg), d in order:
        if span_runs and rd > 0:
            continue
        start, end = g.start(d["v"]), g.end(d["v"], T)
        if span_runs:
            end = min((d["v"] // g.q + 1) * g.span, T)
        h, i, off, pos = d["h"], d["i"], d["off"], start
        while True:
            it = items[i]
            ln = min(it["len"] - off, end - pos)
            assert ln >= 1 and 0 <= h < hkv
            s = it["s"]
            blocks = range(it["off"] + off, it["off"] + off + ln)
            assert blocks.stop <= nb[s] <= max_blocks
            if it["m"] > 0:   # G-item piece: members' rows
                assert grouped and it["m"] * G <= 16
                for b in blocks:
                    for j in range(it["m"]):
                        assert b < n[s + j] // bs   # inside every member's full blocks
                        shared_reads[(h, s + j, b)] = shared_reads.get((h, s + j, b), 0) + 1
                pg = pieces(h, it["pos"], it["len"])
                k = d["v"] - g.of(h * TB + it["pos"])
                assert 0 <= k < pg <= max_pieces(it["len"], g.chunk, g.span, g.q)
                rows = it["m"] * G
                row0 = h * pl["RH"] + it["rbase"] + k * rows
                for j in range(it["m"]):
                    for r in range(G):
                        key = row0 + j * G + r
                        assert key not in recs and 0 <= key < hkv * pl["RH"] <= cap_rows
                        recs[key] = (h, s + j, "g", k)
                for j in range(it["m"]):
                    counters[(h, s + j)] = counters.get((h, s + j), 0) + 1
            else:
                for b in blocks:
                    streamed[h, s, b] += 1
                ps = pieces(h, it["pos"], it["len"])
                pg = pieces(h, it["g_pos"], it["g_len"]) if grouped and it.get("g_len", 0) > 0 else 0
                whole = ps + pg == 1
                if not grouped:
                    whole = off == 0 and off + ln == it["len"] and g.of(pos) == g.of(pos + ln - 1)
                if whole:
                    written[h, s] += 1
                elif grouped:
                    k = d["v"] - g.of(h * TB + it["pos"])
                    assert k < max_pieces(it["len"], g.chunk, g.span, g.q)
                    row0 = h * pl["RH"] + it["rbase"] + k * G
                    for r in range(G):
                        key = row0 + r
                        assert key not in recs and 0 <= key < hkv * pl["RH"] <= cap_rows
                        recs[key] = (h, s, "s", k)
                    counters[(h, s)] = counters.get((h, s), 0) + 1
                else:   # flat: slot 0/1 of each chunk, counter of the run's first chunk
                    w = g.of(pos)
                    wstart = g.start(w)
                    assert span_runs or (w == d["v"] and wstart == start)
                    nparts = g.of(pos + ln - 1) - w + 1
                    assert span_runs or nparts == 1
                    for k in range(nparts):
                        kk = (0 if pos == wstart else 1) if k == 0 else 0
                        key = ("flat", 2 * (w + k) + kk)
                        assert key not in recs and 2 * (w + k) + kk < 2 * hp["chunks"]
                        recs[key] = (h, s)
                    seg = pos - off
                    fw, lw = g.of(seg), g.of(seg + it["len"] - 1)
                    assert fw < lw and fw < COUNTER_SLOTS
                    counters[("flat", fw)] = counters.get(("flat", fw), 0) + nparts
                    if counters[("flat", fw)] == lw - fw + 1:
                        for v in range(fw, lw + 1):
                            kk2 = 0 if g.start(v) >= seg else 1
                            assert recs.get(("flat", 2 * v + kk2)) == (h, s)
                        written[h, s] += 1
                        counters[("flat", fw)] = 0
            pos += ln
            if pos >= end:
                break
            i += 1
            if i == NI:
                i, h = 0, h + 1
            off = 0
    if grouped:   # merges: each output's records, G-item pieces then S-item pieces
        for (h, s), got in counters.items():
            it_s = items[pl["seqs"][s]["s_item"]] if pl["seqs"][s]["s_item"] >= 0 else None
            gr = pl["groups"].get(int(pl["gid"][s]))
            pg = pieces(h, items[gr["item"]]["pos"], items[gr["item"]]["len"]) if (
                gr and "item" in gr and gr["m"] >= 2 and gr["k"] >= 1) else 0
            ps = pieces(h, it_s["pos"], it_s["len"]) if it_s else 0
            assert got == pg + ps and h * S + s < COUNTER_SLOTS
            for c in range(pg):
                gi = items[gr["item"]]
                mem = s - gr["first"]
                for r in range(G):
                    key = h * pl["RH"] + gi["rbase"] + c * gi["m"] * G + mem * G + r
                    assert recs[key] == (h, s, "g", c)
            for c in range(ps):
                for r in range(G):
                    key = h * pl["RH"] + it_s["rbase"] + c * G + r
                    assert recs[key] == (h, s, "s", c)
            written[h, s] += 1
    else:
        assert all(v == 0 for v in counters.values())
    # every block of every (kv head, sequence) is read exactly once: by the
    # sequence's own items, or by its group's G-item for all members
    for h in range(hkv):
        for s in range(S):
            for b in range(nb[s]):
                assert streamed[h, s, b] + shared_reads.get((h, s, b), 0) == 1, (h, s, b)
            assert not streamed[h, s, nb[s]:].any()
            assert written[h, s] == (1 if nb[s] > 0 else 0), (h, s)


def replay(tables, lens, hkv, bs, pt, G=1, num_blocks=None, **kw):
    tables = np.asarray(tables, np.int64)
    S, mb = tables.shape
    num_blocks = num_blocks if num_blocks is not None else int(tables.max(initial=0)) + 1
    hp = host_plan(S, hkv, mb, bs, G, pt, **kw)
    pl = device_plan(tables, np.asarray(lens), hkv, bs, num_blocks, G, hp)
    walk(pl, hkv, bs, G, hp, mb)
    if pl["q"] > 1 and not pl["grouped"]:   # matrix-core runs: one descriptor and one pass per span
        one = device_plan(tables, np.asarray(lens), hkv, bs, num_blocks, G, hp, span_runs=True)
        walk(one, hkv, bs, G, hp, mb, span_runs=True)
    return pl


def private_tables(lens, bs, mb, rng):
    """Tables with every sequence on its own blocks, in random places."""
    S = len(lens)
    ids = rng.permutation(S * mb)
    t = -np.ones((S, mb), np.int64)
    for s in range(S):
        k = -(-int(min(lens[s], mb * bs)) // bs)
        t[s, :k] = ids[s * mb:s * mb + k]
    return t


def forked_tables(prompt_lens, n, extra, bs, rng, mb=None):
    """n candidates per prompt sharing its full blocks; the partial last block
    and `extra` further tokens on blocks of their own (copy-on-write)."""
    S = len(prompt_lens) * n
    lens = np.array([p + extra for p in prompt_lens for _ in range(n)])
    mb = mb or int(max(-(-lens // bs)))
    t = -np.ones((S, mb), np.int64)
    nxt = 0
    for pi, p in enumerate(prompt_lens):
        full = p // bs
        shared_ids = list(range(nxt, nxt + full))
        nxt += full
        for j in range(n):
            s = pi * n + j
            t[s, :full] = shared_ids
            k = -(-int(lens[s]) // bs)
            for b in range(full, k):
                t[s, b] = nxt
                nxt += 1
    perm = rng.permutation(nxt)
    return np.where(t >= 0, perm[np.maximum(t, 0)], -1), lens


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


@pytest.mark.parametrize("case", CASES)
def test_flat_bookkeeping(case):
    lens, hkv, mb, bs, pt = case
    t = private_tables(lens, bs, mb, np.random.default_rng(1))
    pl = replay(t, lens, hkv, bs, pt)
    assert pl["flags"] == 0


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("pt", [0, 16, 64])
@pytest.mark.parametrize("shape", [([1023] * 3, 4, 1), ([95, 80, 130], 4, 5), ([1024] * 2, 4, 1),
                                   ([47], 4, 1), ([200, 31], 8, 40), ([16, 16], 3, 0)])
def test_grouped_bookkeeping(shape, pt, G):
    prompts, n, extra = shape
    rng = np.random.default_rng(7)
    t, lens = forked_tables(prompts, n, extra, 16, rng)
    pl = replay(t, lens, 2, 16, pt, G=G)
    if G <= 8 and min(prompts) >= 16:
        assert pl["flags"] == 2, "forked candidates should be grouped"


def test_shared_first_block_without_a_full_shared_block_stays_flat():
    """Candidates that share only a partial first block have nothing to read
    once: the plan stays flat (the L2-sharing mode)."""
    t = np.array([[5, -1]] * 4 + [[7, 8]] * 2, np.int64)   # 10 tokens on one shared block; 20 on two
    lens = np.array([10, 10, 10, 10, 20, 20])
    t[5, 0] = 9
    pl = replay(t, lens, 2, 16, 0, num_blocks=10)
    assert pl["flags"] == 1


def test_grouping_is_off_for_small_blocks_and_wide_groups():
    t, lens = forked_tables([100, 64], 4, 3, 8, np.random.default_rng(4))
    assert replay(t, lens, 2, 8, 0)["flags"] == 1           # block size 8: no 16-token tiles
    t, lens = forked_tables([100, 64], 4, 3, 16, np.random.default_rng(4))
    assert replay(t, lens, 1, 16, 0, G=16)["flags"] == 1    # 16 query rows: one member per group


def test_group_records_fall_back_to_flat_when_short():
    t, lens = forked_tables([400] * 4, 4, 2, 16, np.random.default_rng(5))
    hp = host_plan(t.shape[0], 2, t.shape[1], 16, 1, 0)
    hp["grec_rows"] = 3   # far too few rows: the plan is laid out flat
    pl = device_plan(t, lens, 2, 16, int(t.max()) + 1, 1, hp)
    assert pl["flags"] == 1
    walk(pl, 2, 16, 1, hp, t.shape[1])


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("cus", [4, 256])
def test_random_bookkeeping(seed, cus):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([8, 16, 32, 64]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.integers(1, 9))
    if seed % 2:
        prompts = rng.integers(0, 300, size=int(rng.integers(1, 40))).tolist()
        t, lens = forked_tables(prompts, int(rng.integers(1, 9)), int(rng.integers(0, 40)), bs, rng)
        # shuffle some rows so runs of candidates are broken up
        if seed % 3 == 0:
            perm = rng.permutation(len(lens))
            t, lens = t[perm], lens[perm]
    else:
        S = int(rng.integers(1, 300))
        mb = int(rng.integers(1, 80))
        lens = rng.integers(0, mb * bs + 1, size=S)
        t = private_tables(lens, bs, mb, rng)
    pt = int(rng.choice([0, bs, 3 * bs, 32 * bs]))
    replay(t, lens, hkv, bs, pt, G=G, num_cus=cus, waves_per_cu=int(rng.integers(1, 20)))


def test_workload_shapes_fit():
    import workloads as W
    from oracle.paging import plan
    for wl in W.full_configs().values():
        tables = plan(wl, W.free_list_order(wl))["tables"]
        pl = replay(tables, wl.context_lens, wl.num_kv_heads, wl.block_size, wl.partition_tokens,
                    G=wl.group, num_blocks=wl.num_blocks)
        shared = len(set(wl.parent)) < wl.num_seqs
        assert bool(pl["flags"] & 2) == shared, wl.name
        if wl.partition_tokens:   # equal spans per worker, each cut into whole partitions and a rest
            assert pl["chunk"] == wl.partition_tokens // wl.block_size and pl["q"] > 1, wl.name
