"""The C++ block manager (libpa.so, host code) against the oracle's BlockPoolModel.

No GPU: the block manager never touches device memory.  Tables, slots,
copy-on-write pairs, refcounts and the free list must match bit for bit.
"""
import copy
import numpy as np
import pytest

import oracle
import synth


def _bm(*a, **k):
    import paged_kv_cache_write_amd as pk
    return pk.BlockManager(*a, **k)


def _same_state(bm, model):
    assert bm.num_free == len(model.free)
    assert bm.free_list() == list(model.free)
    assert bm.refcounts() == model.ref
    assert bm.num_seqs == len(model.tables) + len(model.swapped)
    for s, tab in model.tables.items():
        assert bm.block_table(s) == tab
        assert bm.seq_len(s) == model.lens[s]


def test_cow_example_comfyai_643(golden):
    g = golden("cow_example.json")
    bm = _bm(g["num_blocks"], g["block_size"])
    ids = {"A1": 0, "A2": 1, "B": 2}
    bm.add_seq(0, 6)
    bm.add_seq(2, 3)
    bm.fork(0, 1)
    a = g["after_fork"]
    assert bm.block_table(0) == a["A1"] and bm.block_table(1) == a["A2"]
    slot, cow = bm.append_slot(ids["A1"])
    a = g["after_A1_append"]
    assert (slot, list(cow)) == (a["A1_slot"], a["cow"])
    assert bm.block_table(0) == a["A1"] and bm.block_table(1) == a["A2"]
    assert {str(b): r for b, r in enumerate(bm.refcounts()) if r} == a["refcount"]
    slot, cow = bm.append_slot(ids["A2"])
    assert (slot, cow) == (g["after_A2_append"]["A2_slot"], None)


def test_alloc_timeline_slide11(golden):
    g = golden("alloc_timeline.json")
    bm = _bm(len(g["free_order"]), g["block_size"], g["free_order"])
    bm.add_seq(0, g["prompt_tokens"])
    assert bm.block_table(0) == g["after_prefill"]["table"]
    for key in ("step1", "step2"):
        slot, cow = bm.append_slot(0)
        assert cow is None and slot == g[key]["slot"] and bm.block_table(0) == g[key]["table"]
        assert bm.num_free == g[key]["num_free"]


def test_random_ops_match_model():
    import paged_kv_cache_write_amd as pk
    rng = np.random.default_rng(11)
    for trial in range(30):
        bs = int(rng.choice([2, 4, 8, 16]))
        NB = int(rng.integers(4, 80))
        order = rng.permutation(NB)[: int(rng.integers(1, NB + 1))]
        bm, model = _bm(NB, bs, order), oracle.BlockPoolModel(NB, bs, order)
        live, nxt = [], 100
        for _ in range(250):
            op = int(rng.integers(0, 5))
            if op == 0 or not live:
                n = int(rng.integers(0, 3 * bs))
                try:
                    model.add_seq(nxt, n)
                    ok = True
                except oracle.BlockPoolModel.NoBlocks:
                    ok = False
                if ok:
                    bm.add_seq(nxt, n)
                    live.append(nxt)
                else:
                    with pytest.raises(pk.PAError) as e:
                        bm.add_seq(nxt, n)
                    assert e.value.status == -4
                nxt += 1
            elif op == 1:
                p = live[int(rng.integers(len(live)))]
                model.fork(p, nxt)
                bm.fork(p, nxt)
                live.append(nxt)
                nxt += 1
            elif op == 2:
                s = live[int(rng.integers(len(live)))]
                try:
                    want = model.append_slot(s)
                except oracle.BlockPoolModel.NoBlocks:
                    want = None
                if want is None:
                    with pytest.raises(pk.PAError):
                        bm.append_slot(s)
                else:
                    got = bm.append_slot(s)
                    assert got == want
            elif op == 3:
                batch = [live[int(i)] for i in rng.integers(0, len(live), size=int(rng.integers(1, 6)))]
                snapshot_ok = True
                want_slots, want_cows = [], []
                saved = copy.deepcopy(model)
                try:
                    for s in batch:
                        slot, cow = model.append_slot(s)
                        want_slots.append(slot)
                        if cow:
                            want_cows.append(cow)
                except oracle.BlockPoolModel.NoBlocks:
                    snapshot_ok = False
                if snapshot_ok:
                    slots, cows = bm.append_slots(batch)
                    assert slots.tolist() == want_slots
                    assert [tuple(c) for c in cows.tolist()] == want_cows
                else:
                    with pytest.raises(pk.PAError) as e:
                        bm.append_slots(batch)
                    assert e.value.status == -4
                    model = saved        # all or nothing: the batch changed nothing
            else:
                s = live.pop(int(rng.integers(len(live))))
                model.free_seq(s)
                bm.free_seq(s)
            _same_state(bm, model)


def test_workload_scripts_match_model():
    """Execute each config's op script on both managers (no K/V data)."""
    cases = [synth.make_workload(cfg, values=False, **kw) for cfg, kw in
             ((1, {}), (2, {}), (4, {}), (4, {"cow": True}), (5, {"bs": 8, "S": 40}))]
    cases += [synth.make_fork_tree(seed, 1, 8, "f32", bs, forks=12, max_prompt=200,
                                   max_extend=50) for seed, bs in ((510, 8), (511, 16))]
    cases += [synth.make_beam_search(seed, 1, 8, "f32", bs, prompt=p, width=w, steps=15)
              for seed, bs, p, w in ((512, 8, 37, 4), (513, 16, 300, 8))]
    cases += [synth.make_preemption(seed, 1, 8, "f32", bs) for seed, bs in ((514, 8), (515, 16))]
    for wl in cases:
        bm, model = _bm(wl.NB, wl.bs, wl.free_order), oracle.BlockPoolModel(wl.NB, wl.bs, wl.free_order)
        for op in wl.ops:
            if op[0] == "add":
                model.add_seq(op[1], op[2])
                bm.add_seq(op[1], op[2])
                assert bm.slots(op[1], 0, op[2]).tolist() == model.slots(op[1], 0, op[2])
            elif op[0] == "fork":
                model.fork(op[1], op[2])
                bm.fork(op[1], op[2])
            elif op[0] == "free":
                model.free_seq(op[1])
                bm.free_seq(op[1])
            elif op[0] == "select":
                for p, c in op[1]:
                    model.fork(p, c)
                for r in op[2]:
                    model.free_seq(r)
                bm.select(op[1], op[2])
                _same_state(bm, model)
            elif op[0] == "host_pool":
                model.set_host_pool(op[1])
                bm.set_host_pool(op[1])
            elif op[0] in ("swap_out", "swap_in"):
                want = getattr(model, op[0])(op[1])
                got = getattr(bm, op[0])(op[1])
                assert [tuple(p) for p in got.tolist()] == want
                _same_state(bm, model)
            elif op[0] == "extend":
                want = [model.append_slot(op[1]) for _ in range(op[2])]
                slots, cows = bm.append_slots([op[1]] * op[2])
                assert slots.tolist() == [w[0] for w in want]
                assert [tuple(c) for c in cows.tolist()] == [w[1] for w in want if w[1]]
            else:
                seqs = np.array(op[1], dtype=np.int64)
                want = [model.append_slot(int(s)) for s in seqs]
                S, W = seqs.size, wl.max_blocks_per_seq
                slots = np.empty(S, np.int64)
                cows = np.empty(2 * S, np.int32)
                tables = np.empty((S, W), np.int32)
                ctx = np.empty(S, np.int32)
                ncow = bm.step_into(seqs, slots, cows, tables, wl.poison_block, ctx)
                assert slots.tolist() == [w[0] for w in want]
                assert [tuple(c) for c in cows[:2 * ncow].reshape(-1, 2).tolist()] == \
                    [w[1] for w in want if w[1]]
                assert np.array_equal(tables, model.table_array(list(seqs), W, wl.poison_block))
                assert ctx.tolist() == [model.lens[int(s)] for s in seqs]
                assert ctx.tolist() == wl.ctx.tolist()
        _same_state(bm, model)


def test_cow_subcase_counts():
    """Config-4 CoW variant: 7 of 8 siblings copy the shared last block, the last writes in place."""
    wl = synth.make_workload(4, cow=True, values=False)
    model = oracle.BlockPoolModel(wl.NB, wl.bs, wl.free_order)
    cows = 0
    for op in wl.ops:
        if op[0] == "add":
            model.add_seq(op[1], op[2])
        elif op[0] == "fork":
            model.fork(op[1], op[2])
        elif op[0] == "extend":
            cows += sum(model.append_slot(op[1])[1] is not None for _ in range(op[2]))
        else:
            cows += sum(model.append_slot(int(s))[1] is not None for s in op[1])
    assert cows == 7 * 8


def test_errors():
    import paged_kv_cache_write_amd as pk
    bm = _bm(4, 4)
    bm.add_seq(1, 4)
    with pytest.raises(pk.PAError) as e:
        bm.add_seq(1, 1)
    assert e.value.status == -7
    with pytest.raises(pk.PAError) as e:
        bm.fork(9, 10)
    assert e.value.status == -6
    with pytest.raises(pk.PAError) as e:
        bm.add_seq(2, 17)
    assert e.value.status == -4
    assert bm.num_free == 3              # failed add changed nothing
    with pytest.raises(pk.PAError) as e:
        pk.BlockManager(4, 4, [0, 0])
    assert e.value.status == -1
    tables, ctx = bm.block_tables([1], 1, -1)
    assert tables.tolist() == [[bm.block_table(1)[0]]] and ctx.tolist() == [4]
    bm.append_slot(1)
    with pytest.raises(pk.PAError) as e:
        bm.block_tables([1], 1, -1)
    assert e.value.status == -8


def test_select_checks_before_changing():
    """A beam selection with any bad argument changes nothing; a good one forks, then
    frees (blocks held only by retired beams go back to the free list in order)."""
    import paged_kv_cache_write_amd as pk
    bm, model = _bm(16, 4), oracle.BlockPoolModel(16, 4)
    for x in (bm, model):
        x.add_seq(1, 6)
        x.add_seq(2, 3)
    before = (bm.free_list(), bm.refcounts())
    for pairs, retire, status in (([(9, 5)], [], -6),           # unknown parent
                                  ([(1, 2)], [], -7),           # child exists
                                  ([(1, 5), (2, 5)], [], -7),   # child twice
                                  ([(1, 5)], [9], -6),          # unknown retired
                                  ([(1, 5)], [2, 2], -1)):      # retired twice
        with pytest.raises(pk.PAError) as e:
            bm.select(pairs, retire)
        assert e.value.status == status
        assert (bm.free_list(), bm.refcounts()) == before
    bm.select([(1, 5), (1, 6), (2, 7)], [1, 2])
    for p, c in ((1, 5), (1, 6), (2, 7)):
        model.fork(p, c)
    model.free_seq(1)
    model.free_seq(2)
    _same_state(bm, model)
    assert bm.seq_len(5) == 6 and bm.refcount(bm.block_table(5)[0]) == 2

def test_failed_batch_changes_nothing():
    """A batch of appends that runs out of blocks part way (after a new block and a
    copy on write) is undone: lengths, tables, refcounts and the free list's order
    are as before, and the same batch succeeds once a sequence is freed."""
    import paged_kv_cache_write_amd as pk
    bm = _bm(5, 4, [4, 3, 2, 1, 0])
    bm.add_seq(1, 4)          # one full block: the next append takes a new block
    bm.add_seq(2, 2)
    bm.fork(2, 3)             # 2 and 3 share a partly filled block: copy on write
    bm.add_seq(4, 5)          # two blocks; 1 block left free
    state = (bm.free_list(), bm.refcounts(), [bm.block_table(s) for s in (1, 2, 3, 4)],
             [bm.seq_len(s) for s in (1, 2, 3, 4)])
    assert len(state[0]) == 1
    with pytest.raises(pk.PAError) as e:
        bm.append_slots([1, 2, 4])        # 1 takes the last free block, 2 would copy
    assert e.value.status == -4
    assert (bm.free_list(), bm.refcounts(), [bm.block_table(s) for s in (1, 2, 3, 4)],
            [bm.seq_len(s) for s in (1, 2, 3, 4)]) == state
    bm.free_seq(4)
    slots, cows = bm.append_slots([1, 2, 3])
    assert cows.shape == (1, 2) and bm.seq_len(1) == 5


def _same_host_state(bm, model):
    assert bm.host_free_list() == list(model.host_free)
    assert bm.host_refcounts() == model.host_ref
    for s, t in model.swapped.items():
        assert bm.is_swapped(s) and bm.block_table(s) == t


@pytest.mark.parametrize("seed,bs", [(516, 8), (517, 16), (518, 32)])
def test_preemption_swap_round_trip(seed, bs):
    """The newest request is swapped out as a group, the others reuse its device
    blocks, and it comes back into other blocks; both managers agree throughout."""
    wl = synth.make_preemption(seed, 1, 8, "f32", bs)
    bm, model = _bm(wl.NB, wl.bs, wl.free_order), oracle.BlockPoolModel(wl.NB, wl.bs, wl.free_order)
    out_blocks, reused = None, False
    for op in wl.ops:
        if op[0] == "add":
            model.add_seq(op[1], op[2]); bm.add_seq(op[1], op[2])
        elif op[0] == "fork":
            model.fork(op[1], op[2]); bm.fork(op[1], op[2])
        elif op[0] == "extend":
            model.append_slot(op[1]); bm.append_slot(op[1])
            if out_blocks and set(model.tables[op[1]]) & out_blocks:
                reused = True
        elif op[0] == "free":
            model.free_seq(op[1]); bm.free_seq(op[1])
        elif op[0] == "host_pool":
            model.set_host_pool(op[1]); bm.set_host_pool(op[1])
        elif op[0] == "swap_out":
            pairs = bm.swap_out(op[1])
            assert [tuple(p) for p in pairs.tolist()] == model.swap_out(op[1])
            out_blocks = {int(p[0]) for p in pairs}
            with pytest.raises(Exception):
                bm.append_slot(op[1][0])            # a swapped-out sequence cannot grow
        elif op[0] == "swap_in":
            pairs = bm.swap_in(op[1])
            assert [tuple(p) for p in pairs.tolist()] == model.swap_in(op[1])
        elif op[0] == "step":
            for s in op[1]:
                model.append_slot(s); bm.append_slot(s)
        _same_state(bm, model)
        _same_host_state(bm, model)
    assert reused, "the other requests should take the blocks the preempted group gave back"


def test_swap_checks_before_changing():
    """Swapping part of a group, unknown or repeated sequences, a short pool or a
    short pairs buffer change nothing; blocks_needed matches the model's count."""
    import paged_kv_cache_write_amd as pk
    bm, model = _bm(10, 4), oracle.BlockPoolModel(10, 4)
    for x in (bm, model):
        x.add_seq(1, 6)
        x.fork(1, 2)
        x.add_seq(3, 9)
        x.set_host_pool(2)
    before = (bm.free_list(), bm.refcounts(), bm.host_free_list())
    for seqs, status in (([1], -1), ([9], -6), ([1, 1, 2], -1), ([3], -4)):
        with pytest.raises(pk.PAError) as e:
            bm.swap_out(seqs)
        assert e.value.status == status
        assert (bm.free_list(), bm.refcounts(), bm.host_free_list()) == before
    with pytest.raises(pk.PAError):
        bm.swap_in([1])                               # not swapped out
    for seqs in ([1, 2, 3, 1], [3, 3, 3, 3], [2, 1], [3]):
        assert bm.blocks_needed(seqs) == model.blocks_needed(seqs)
    assert bm.blocks_needed([1, 2]) == 1              # the first writer copies, the last writes in place
    assert [tuple(p) for p in bm.swap_out([2, 1]).tolist()] == model.swap_out([2, 1])
    with pytest.raises(pk.PAError) as e:
        bm.fork(2, 4)                                 # swapped out: no fork
    assert e.value.status == -6
    bm.free_seq(2)                                    # frees host references
    model.free_seq(2)
    _same_host_state(bm, model)
    assert [tuple(p) for p in bm.swap_in([1]).tolist()] == model.swap_in([1])
    _same_state(bm, model)
    _same_host_state(bm, model)