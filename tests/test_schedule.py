"""Host work lists of the decode launcher (CPU only).

A decode of context c in partitions of pt tokens has ceil(c / pt) partitions
(polomodov.tech, split-context partitions; the partition results are merged
by their log-sum-exp).  The work list must cover every (sequence, partition)
once, and a shared-prefix group item may only cover tokens whose physical
blocks are the same for all its members (comfyai.app 6.4.2-6.4.3: forked
samples point at the parent's blocks until they write).
"""
import numpy as np
import pytest

import oracle
import synth


def _pk():
    import paged_kv_cache_write_amd as pk
    return pk


def test_decode_schedule_order():
    """Full partitions first, then partial ones longest first, then empty rows."""
    pk = _pk()
    ctx = np.array([0, 300, 256, 1000, 5, 512], dtype=np.int32)
    items, pt, mx = pk.decode_schedule(ctx, 40, 128, 16, 1, 256)
    assert (pt, mx) == (256, 1000)
    assert items[:, :2].tolist() == [[1, 0], [2, 0], [3, 0], [3, 1], [3, 2], [5, 0], [5, 1],
                                     [3, 3], [1, 1], [4, 0], [0, 0]]
    # (first token, tokens, partitions of the row)
    assert items[:, 2:].tolist() == [[0, 256, 2], [0, 256, 1], [0, 256, 4], [256, 256, 4],
                                     [512, 256, 4], [0, 256, 2], [256, 256, 2], [768, 232, 4],
                                     [256, 44, 2], [0, 5, 1], [0, 0, 0]]
    rng = np.random.default_rng(0)
    for _ in range(20):
        ctx = rng.integers(0, 5000, size=int(rng.integers(1, 50))).astype(np.int32)
        items, pt, mx = pk.decode_schedule(ctx, 40, 128, 16, 1, 512)
        want = sorted([(s, p) for s, c in enumerate(ctx) for p in range(-(-int(c) // pt))] +
                      [(s, 0) for s, c in enumerate(ctx) if c == 0])
        assert sorted(map(tuple, items[:, :2].tolist())) == want
        sizes = items[:, 3].tolist()
        assert sizes == sorted(sizes, reverse=True)
        for s, p, t0, n, npart in items.tolist():
            assert t0 == p * pt and n == min(pt, int(ctx[s]) - t0) or ctx[s] == 0
            assert npart == -(-int(ctx[s]) // pt)


# waves the automatic partition size aims for (one round of wave slots)
TARGET_WAVES = 2048


@pytest.mark.parametrize("bs", [8, 16, 32, 64, 128])
def test_automatic_partitions_are_balanced(bs):
    """Automatic partitions: each row is cut into ceil(ctx / pt) partitions that
    start on whole units of max(32, bs) tokens, cover the row once, are at most pt
    long and differ by at most one unit (the last may end early at the context);
    pt is the smallest size from 256 up whose launch fits the wave target, else the
    largest; the work list runs longest first."""
    pk = _pk()
    rng = np.random.default_rng(bs)
    q = max(32, bs)
    max_pt = min(64 * bs, 1024)
    for trial in range(25):
        H = int(rng.choice([1, 8, 40]))
        ctx = rng.integers(0, 6000, size=int(rng.integers(1, 60))).astype(np.int32)
        if trial % 5 == 0:
            ctx[:] = 2048
        items, pt, mx = pk.decode_schedule(ctx, H, 128, bs, 1, 0)
        assert mx == int(ctx.max())
        assert 256 <= pt <= max_pt or pt == max_pt
        waves = lambda t: H * sum(-(-int(c) // t) for c in ctx)
        if pt > min(256, max_pt):
            assert waves(pt - q) > TARGET_WAVES          # a smaller size would not fit
        assert waves(pt) <= TARGET_WAVES or pt == max_pt
        sizes = items[:, 3].tolist()
        assert sizes == sorted(sizes, reverse=True)
        rows = {}
        for s, p, t0, n, npart in items.tolist():
            rows.setdefault(s, []).append((p, t0, n, npart))
        assert sorted(rows) == list(range(ctx.size))
        for s, parts in rows.items():
            c = int(ctx[s])
            if c == 0:
                assert parts == [(0, 0, 0, 0)]
                continue
            parts.sort()
            n_parts = -(-c // pt)
            assert [p for p, *_ in parts] == list(range(n_parts))
            assert all(npart == n_parts for *_, npart in parts)
            t = 0
            for p, t0, n, _ in parts:
                assert t0 == t and t0 % q == 0 and 0 < n <= pt
                t += n
            assert t == c
            lens = [n for _, _, n, _ in parts]
            assert max(lens[:-1] or [0]) - min(lens[:-1] or [0]) <= q
            assert lens[-1] <= max(lens)


def _tables_after_step(wl):
    """Replay a workload's op script on the pool model; tables and contexts of the
    decode step's sequences after their slots were appended."""
    m = oracle.BlockPoolModel(wl.NB, wl.bs, wl.free_order)
    seqs = None
    for op in wl.ops:
        if op[0] == "add":
            m.add_seq(op[1], op[2])
        elif op[0] == "fork":
            m.fork(op[1], op[2])
        elif op[0] == "extend":
            for _ in range(op[2]):
                m.append_slot(op[1])
        else:
            seqs = list(op[1])
            for s in seqs:
                m.append_slot(int(s))
    tables = np.asarray(m.table_array(seqs, wl.max_blocks_per_seq, wl.poison_block), np.int32)
    ctx = np.array([m.lens[s] for s in seqs], np.int32)
    return tables, ctx


def check_shared_schedule(d, tables, ctx, bs, max_members=16):
    """Every (sequence, token) covered once; partition indices 0..n-1 once per row with
    one agreed n; group items only over blocks that all members share, with 2 to
    max_members members (16 on the matrix cores, 8 for float32)."""
    pt = d["partition_tokens"]
    S = ctx.size
    cover = {s: [] for s in range(S)}      # (t0, ntok, part, nparts)
    for s, p, t0, n, npart in d["items"].tolist():
        if ctx[s] == 0:
            assert (p, t0, n, npart) == (0, 0, 0, 0)
            continue
        assert 0 < n <= pt
        cover[s].append((t0, n, p, npart))
    for moff, cnt, p, t0, n in d["groups"].tolist():
        assert 2 <= cnt <= max_members and n == 256 and t0 == 256 * p
        mem = d["members"][moff:moff + cnt]
        b0, b1 = t0 // bs, (t0 + n + bs - 1) // bs
        lead = tables[mem[0, 0], b0:b1]
        for s, npart in mem.tolist():
            assert np.array_equal(tables[s, b0:b1], lead), "group over unshared blocks"
            cover[s].append((t0, n, p, npart))
    grouped = {int(s) for s in d["members"][:, 0]} if len(d["members"]) else set()
    for s in range(S):
        if ctx[s] == 0:
            assert not cover[s]
            continue
        if s in grouped:   # the row's last partition is a single item
            assert max(cover[s])[0] + max(cover[s])[1] == ctx[s]
            last = max(cover[s])
            assert any(it[0] == s and it[2] == last[0] for it in d["items"].tolist())
        segs = sorted(cover[s])
        nparts = {c[3] for c in segs}
        assert nparts == {len(segs)}, (s, segs)
        assert sorted(c[2] for c in segs) == list(range(len(segs)))
        pos = 0
        for t0, n, p, _ in segs:
            assert t0 == pos
            pos += n
        assert pos == ctx[s]
        # partition index grows with the first token (the merge is order-free, but the
        # index is the row's slot in the workspace)
        assert [c[2] for c in segs] == list(range(len(segs)))
    return cover


@pytest.mark.parametrize("cow", [False, True])
def test_shared_schedule_config4(cow):
    """8 prompts x 8 samples of 1024-token shared prompts: each prompt's samples form one
    group over the shared 1024 tokens (4 group items of 256 tokens, 8 members)."""
    pk = _pk()
    wl = synth.make_workload(4, cow=cow, values=False)
    tables, ctx = _tables_after_step(wl)
    d = pk.decode_schedule_shared(ctx, tables, wl.H, wl.D, wl.bs, 1, 0)
    check_shared_schedule(d, tables, ctx, wl.bs)
    assert len(d["members"]) == 64
    assert len(d["groups"]) == 8 * 4
    assert sorted(d["members"][:, 0].tolist()) == list(range(64))
    # the single items are ordered longest first
    sizes = d["items"][:, 3].tolist()
    assert sizes == sorted(sizes, reverse=True)
    ws = pk.decode_workspace_size(len(ctx), wl.H, wl.D, wl.bs, int(ctx.max()), 1, 256)
    assert d["workspace_bytes"] >= ws


def test_shared_schedule_without_sharing_is_plain():
    """No two tables start alike: the shared schedule is the plain one."""
    pk = _pk()
    for cfg in (1, 2):
        wl = synth.make_workload(cfg, values=False)
        tables, ctx = _tables_after_step(wl)
        d = pk.decode_schedule_shared(ctx, tables, wl.H, wl.D, wl.bs, 1, 0)
        items, pt, mx = pk.decode_schedule(ctx, wl.H, wl.D, wl.bs, 1, 0)
        assert len(d["groups"]) == 0 and len(d["members"]) == 0
        assert (d["partition_tokens"], d["max_context_len"]) == (pt, mx)
        assert np.array_equal(d["items"], items)


def test_shared_schedule_random_forks():
    """Random fork trees over a small pool: tables diverge at random blocks, some members
    share less than one group partition, contexts include zero."""
    pk = _pk()
    rng = np.random.default_rng(7)
    for trial in range(30):
        bs = int(rng.choice([8, 16, 32, 64]))
        NB = 4096
        m = oracle.BlockPoolModel(NB, bs, list(range(NB)))
        seqs = []
        roots = int(rng.integers(1, 4))
        for r in range(roots):
            m.add_seq(r, int(rng.integers(0, 1400)))
            seqs.append(r)
        nxt = roots
        for _ in range(int(rng.integers(0, 12))):
            parent = int(rng.choice(seqs))
            m.fork(parent, nxt)
            for _ in range(int(rng.integers(0, 300))):
                m.append_slot(nxt)
            seqs.append(nxt)
            nxt += 1
        for s in seqs:
            m.append_slot(s)
        W = max(-(-m.lens[s] // bs) for s in seqs) + 1
        tables = np.asarray(m.table_array(seqs, W, NB - 1), np.int32)
        ctx = np.array([m.lens[s] for s in seqs], np.int32)
        d = pk.decode_schedule_shared(ctx, tables, 40, 128, bs, 1, int(rng.choice([0, 256, 512])))
        check_shared_schedule(d, tables, ctx, bs)


def test_shared_schedule_groups_of_more_than_eight():
    """20 forks of one prompt: members are cut into balanced chunks of at most 8
    (float32) or 16 (16-bit storage, matrix cores)."""
    pk = _pk()
    bs = 16
    m = oracle.BlockPoolModel(2048, bs, list(range(2048)))
    m.add_seq(0, 777)
    for c in range(1, 20):
        m.fork(0, c)
    seqs = list(range(20))
    for s in seqs:
        m.append_slot(s)
    tables = np.asarray(m.table_array(seqs, 64, 2047), np.int32)
    ctx = np.array([m.lens[s] for s in seqs], np.int32)
    d = pk.decode_schedule_shared(ctx, tables, 8, 64, bs, 0, 0)      # float32: 8 per chunk
    check_shared_schedule(d, tables, ctx, bs, max_members=8)
    cnts = sorted({tuple(g[:2]) for g in d["groups"].tolist()})
    assert [c for _, c in cnts] == [6, 7, 7]
    assert len(d["groups"]) == 3 * 3     # 768 shared tokens = 3 group partitions
    d = pk.decode_schedule_shared(ctx, tables, 8, 64, bs, 2, 0)      # bfloat16: 16 per chunk
    check_shared_schedule(d, tables, ctx, bs)
    cnts = sorted({tuple(g[:2]) for g in d["groups"].tolist()})
    assert [c for _, c in cnts] == [10, 10]


def test_shared_schedule_errors():
    pk = _pk()
    ctx = np.array([300, -1], np.int32)
    tables = np.zeros((2, 40), np.int32)
    with pytest.raises(pk.PAError):
        pk.decode_schedule_shared(ctx, tables, 8, 128, 16, 1, 0)
    with pytest.raises(pk.PAError):
        pk.decode_schedule_shared(np.array([300], np.int32), tables[:1], 8, 96, 16, 1, 0)


@pytest.mark.parametrize("bs", [8, 16, 32, 128])
def test_automatic_partition_size(bs):
    """The automatic partition size is the smallest of 256, 256 + q, ... tokens
    (q = max(32, bs); at most 64 blocks and 1024 tokens) whose work list fits 2048
    waves, or the largest when none does: checked as properties of the chosen size
    on random batches, from a handful of sequences to hundreds."""
    pk = _pk()
    H = 40
    rng = np.random.default_rng(bs)
    cap = min(1024, 64 * bs)
    q = max(32, bs)
    seen = set()
    for i in range(40):
        S = int(rng.integers(1, 12)) if i % 2 else int(rng.integers(12, 300))
        ctx = rng.integers(1, 4000, size=S).astype(np.int32)
        items, pt, _ = pk.decode_schedule(ctx, H, 128, bs, 1, 0)
        seen.add(pt)
        waves = lambda p: int((-(-ctx.astype(np.int64) // p)).sum()) * H
        assert min(256, cap) <= pt <= cap and (pt - min(256, cap)) % q == 0 and pt % bs == 0
        assert len(items) * H == waves(pt)
        assert waves(pt) <= TARGET_WAVES or pt == cap
        if pt > min(256, cap):
            assert waves(pt - q) > TARGET_WAVES, "a smaller partition also fitted"
    assert len(seen) > 1
