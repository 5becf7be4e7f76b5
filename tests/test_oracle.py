"""Pins for the oracle, checked against what the pages and the mathematics fix.

No GPU.  Each pin names the passage or the closed form it comes from.  The last
group plants plausible mistakes into the oracle (on the CPU) and checks that
some pin here catches each of them.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from gpu_harness import contiguous_kv
import synth
from oracle import paged_attention as pa


# ---------------------------------------------------------------- helpers
def _pool(NB, H, bs, D, fill=np.nan):
    return np.full((NB, H, bs, D), fill, dtype=np.float64)


def _scatter(K, table, NB, bs):
    """Place contiguous [L, H, D] tokens into a fresh NaN pool through ``table``
    by explicit loops (an independent placement, not oracle_cache_write)."""
    L, H, D = K.shape
    pool = _pool(NB, H, bs, D)
    for t in range(L):
        for h in range(H):
            pool[table[t // bs], h, t % bs, :] = K[t, h, :]
    return pool


def _decode_one(q, K, V, scale, bs=4, NB=None, seed=0):
    """Run oracle_decode for one sequence whose K/V are scattered at random."""
    L, H, D = K.shape
    nblk = -(-L // bs)
    NB = NB or nblk + 3
    table = np.random.default_rng(seed).permutation(NB)[:nblk]
    kp, vp = _scatter(K, table, NB, bs), _scatter(V, table, NB, bs)
    row = np.concatenate([table, [10**9] * 2])      # entries past ceil(L/bs) are invalid
    out = oracle.oracle_decode(q[None], kp, vp, row[None], [L], scale, "f32")
    return out[0]


# ------------------------------------------------------ printed numbers
def test_kv_bytes_per_token_13b(golden):
    g = golden("kv_sizes.json")
    m = g["model"]
    per_tok = oracle.kv_bytes_per_token(m["layers"], m["heads"], m["head_dim"], m["elem_bytes"])
    assert per_tok == math.prod(g["per_token_bytes_factors"]) == 819200
    assert per_tok == g["per_token_printed_KB"] * 1024           # "800 KB" are KiB
    assert m["heads"] * m["head_dim"] == m["d_model"]


def test_kv_cache_worked_example(golden):
    g = golden("kv_sizes.json")
    m, ex = g["model"], g["worked_example"]
    b = oracle.kv_cache_bytes(ex["batch"], ex["seq_len"], m["layers"], m["d_model"], m["elem_bytes"])
    assert b == 3355443200
    assert float(f"{b:.{ex['printed_sig_figs'] - 1}e}") == ex["printed_bytes"]
    assert round(b / 2**30, 1) == ex["printed_GB_approx"]       # "about 3.1 GB" is GiB
    r = g["request_2048"]
    b2 = oracle.kv_cache_bytes(1, r["seq_len"], m["layers"], m["d_model"], m["elem_bytes"])
    assert round(b2 / 2**30, 1) == r["printed_GB_slide5"]       # 1.5625 GiB -> "1.6 GB"
    assert round(b2 / 1e9, 1) == r["printed_GB_comfyai"]        # 1.678e9 B -> "1.7 GB"


def test_workload_shape_matches_13b_layer():
    wl = synth.make_workload(2, values=False)
    per_layer = wl.H * wl.D * 2 * wl.elem_bytes
    assert per_layer * 40 == 819200


# ----------------------------------------------------- structural examples
def test_block_table_example_slide10(golden):
    g = golden("block_table_example.json")
    bs, NB, L = g["block_size"], g["num_blocks"], g["context_len"]
    table = [10**9 if p is None else p for p in g["logical_to_physical"]]
    cache = np.zeros((NB, 1, bs, 1))
    for b in range(NB):
        cache[b, 0, :, 0] = 100 * b + np.arange(bs)             # value = 100*block + offset
    got = pa.oracle_gather(cache, table, L)[:, 0, 0]
    want = [100 * table[t // bs] + t % bs for t in range(L)]
    assert got.tolist() == want
    # the unallocated 4th entry is never read: an out-of-range id there is harmless
    assert -(-L // bs) == 3


def test_alloc_timeline_slide11(golden):
    g = golden("alloc_timeline.json")
    bm = oracle.BlockPoolModel(len(g["free_order"]), g["block_size"], g["free_order"])
    bm.add_seq(0, g["prompt_tokens"])
    assert bm.tables[0] == g["after_prefill"]["table"]
    assert len(bm.free) == g["after_prefill"]["num_free"]
    for key in ("step1", "step2"):
        slot, cow = bm.append_slot(0)
        assert cow is None
        assert slot == g[key]["slot"] and bm.tables[0] == g[key]["table"]
        assert len(bm.free) == g[key]["num_free"]


def test_cow_example_comfyai_643(golden):
    g = golden("cow_example.json")
    bm = oracle.BlockPoolModel(g["num_blocks"], g["block_size"])
    ids = {"A1": 0, "A2": 1, "B": 2}
    res = {}
    for op in g["ops"]:
        if op[0] == "add":
            bm.add_seq(ids[op[1]], op[2])
        elif op[0] == "fork":
            bm.fork(ids[op[1]], ids[op[2]])
            res["fork"] = None
        else:
            res[op[1]] = bm.append_slot(ids[op[1]])
            if op[1] == "A1":
                a = g["after_A1_append"]
                assert bm.tables[0] == a["A1"] and bm.tables[1] == a["A2"]
                assert list(res["A1"][1]) == a["cow"] and res["A1"][0] == a["A1_slot"]
                assert {str(b): r for b, r in enumerate(bm.ref) if r} == a["refcount"]
        if op[0] == "fork":
            a = g["after_fork"]
            assert bm.tables[0] == a["A1"] and bm.tables[1] == a["A2"]
            assert {str(b): r for b, r in enumerate(bm.ref) if r} == a["refcount"]
    a = g["after_A2_append"]
    assert bm.tables[1] == a["A2"] and res["A2"] == (a["A2_slot"], None)


# ------------------------------------------------------------ closed forms
def test_ctx1_returns_v0():
    rng = np.random.default_rng(1)
    q, K, V = rng.normal(size=(3, 8)), rng.normal(size=(1, 3, 8)), rng.normal(size=(1, 3, 8))
    assert np.array_equal(_decode_one(q, K, V, 0.3), V[0])


def test_zero_query_and_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(2)
    L, H, D = 37, 2, 6
    K, V = rng.normal(size=(L, H, D)), rng.normal(size=(L, H, D))
    out = _decode_one(np.zeros((H, D)), K, V, 0.5)
    np.testing.assert_allclose(out, V.mean(axis=0), rtol=0, atol=1e-14)
    Keq = np.broadcast_to(rng.normal(size=(1, H, D)), (L, H, D)).copy()
    out = _decode_one(rng.normal(size=(H, D)), Keq, V, 0.5)
    np.testing.assert_allclose(out, V.mean(axis=0), rtol=0, atol=1e-14)


def test_two_token_closed_form_fixes_scale_and_sign():
    # q=(1,0), K0=(0,0), K1=(2,0), scale 1/2: logits (0, 1), so w1 = e/(1+e)
    q = np.array([[1.0, 0.0]])
    K = np.array([[[0.0, 0.0]], [[2.0, 0.0]]])
    V = np.array([[[1.0, -3.0]], [[5.0, 7.0]]])
    w1 = math.e / (1 + math.e)
    want = (1 - w1) * V[0, 0] + w1 * V[1, 0]
    np.testing.assert_allclose(_decode_one(q, K, V, 0.5)[0], want, rtol=0, atol=1e-15)


def test_one_hot_index_probe_decodes_position():
    rng = np.random.default_rng(3)
    L, H, D, bs = 300, 3, 8, 16
    scale = 1 / math.sqrt(D)
    for trial in range(3):
        tstar = rng.integers(0, L, size=H)
        K = np.zeros((L, H, D))
        V = np.zeros((L, H, D))
        t = np.arange(L)
        V[:, :, 0] = (t // 64)[:, None]
        V[:, :, 1] = (t % 64)[:, None]
        for h in range(H):
            K[tstar[h], h, 0] = 200 / scale
        q = np.zeros((H, D))
        q[:, 0] = 1.0
        out = _decode_one(q, K, V, scale, bs=bs, seed=trial)
        dec = np.rint(out[:, 0]) * 64 + np.rint(out[:, 1])
        assert dec.tolist() == tstar.tolist()
        assert np.all(np.abs(out[:, :2] - V[tstar, np.arange(H), :2]) < 1e-80)


# ------------------------------------------------------------- invariants
def test_softmax_weights_sum_to_one_and_match_library():
    wl = synth.make_workload(1)
    r = oracle.run_workload(wl, decode=False)
    out, w = oracle.oracle_decode(wl.q, r["k_cache"], r["v_cache"], r["tables"], r["ctx"],
                                  wl.scale, wl.dtype, return_weights=True)
    assert len(w) == wl.S * wl.H
    for (s, h), ws in w.items():
        assert ws.shape == (int(r["ctx"][s]),)
        assert abs(ws.sum() - 1) < 1e-12 and np.all(ws >= 0)
        k, _ = wl.kv(s, 0, int(r["ctx"][s]))
        logits = wl.scale * (k[:, h, :].astype(np.float64) @ wl.q[s, h].astype(np.float64))
        np.testing.assert_allclose(ws, scipy.special.softmax(logits), rtol=1e-13, atol=1e-16)


def test_brute_force_tiny():
    rng = np.random.default_rng(4)
    for trial in range(40):
        D = int(rng.integers(1, 3))
        L = int(rng.integers(1, 4))
        q = rng.normal(size=(1, D))
        K = rng.normal(size=(L, 1, D)) * 3
        V = rng.normal(size=(L, 1, D))
        scale = float(rng.uniform(0.1, 2.0))
        got = _decode_one(q, K, V, scale, bs=2, seed=trial)[0]
        want = oracle.attention_brute_force(q[0].tolist(), K[:, 0, :].tolist(),
                                            V[:, 0, :].tolist(), scale)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("cfg", [1, 2])
def test_decode_equals_unpaged_attention(cfg):
    """Paged decode on the pool == attention on the contiguous K/V as drawn
    (bit-identical: the gather is exact and the arithmetic the same)."""
    wl = synth.make_workload(cfg)
    seqs = list(range(wl.S)) if cfg == 1 else [0, 7, 29]
    r = oracle.run_workload(wl, decode_seqs=seqs)
    for s in seqs:
        L = int(r["ctx"][s])
        k, v = wl.kv(s, 0, L)
        kf, vf, qf = (oracle.widen(a, wl.dtype) for a in (k, v, wl.q[s]))
        for h in range(wl.H):
            logits = wl.scale * (kf[:, h, :] @ qf[h])
            e = np.exp(logits - logits.max())
            want = (e / e.sum()) @ vf[:, h, :]
            assert np.array_equal(r["out"][s, h], want)


@pytest.mark.parametrize("kind,seed,bs", [("tree", 500, 16), ("tree", 501, 8), ("tree", 502, 32),
                                          ("beam", 503, 8), ("beam", 504, 16),
                                          ("preempt", 505, 8), ("preempt", 506, 16)])
def test_fork_tree_decode_equals_unpaged_attention(kind, seed, bs):
    """Random fork trees (forks of forks, parents extended after forking, copy on
    write of half-full shared blocks) and beam searches (selection with repeats,
    retired beams freed): each decode row equals attention over the sequence's
    logical K/V as drawn, so the script's sharing never leaks one branch's tokens
    into another."""
    if kind == "tree":
        wl = synth.make_fork_tree(seed, 2, 16, "f32", bs, roots=2, forks=8, max_prompt=120,
                                  max_extend=40)
    elif kind == "beam":
        wl = synth.make_beam_search(seed, 2, 16, "f32", bs, prompt=45, width=4, steps=9)
    else:   # swapped out to the host pool and back in to other blocks
        wl = synth.make_preemption(seed, 2, 16, "f32", bs, rounds_before=6, rounds_out=12)
    r = oracle.run_workload(wl)
    step = [op for op in wl.ops if op[0] == "step"][-1][1]
    assert r["all_cows"].shape[0] > 0 or kind == "preempt"
    for row, s in enumerate(step):
        L = int(r["ctx"][row])
        k, v = wl.kv(s, 0, L)
        for h in range(wl.H):
            logits = wl.scale * (k[:, h, :].astype(np.float64) @ wl.q[row, h].astype(np.float64))
            e = np.exp(logits - logits.max())
            want = (e / e.sum()) @ v[:, h, :].astype(np.float64)
            assert np.array_equal(r["out"][row, h], want)


@pytest.mark.parametrize("layout", ["SLHD", "SHLD"])
def test_contiguous_decode_equals_paged(layout):
    """Non-paged decode on the K/V as drawn == the paged decode on the pool built
    by the op script, bit for bit (the gather is exact, the arithmetic the same)."""
    wl = synth.make_workload(1)
    r = oracle.run_workload(wl)
    k, v = contiguous_kv(wl, r["ctx"], layout)
    got = oracle.oracle_decode_contiguous(wl.q, k, v, r["ctx"], wl.scale, wl.dtype, layout)
    assert np.array_equal(got, r["out"])


def test_contiguous_decode_closed_forms():
    """ctx = 1 gives V_0 exactly; q = 0 gives the mean of V; ctx = 0 a zero row;
    both layouts agree bit for bit."""
    rng = np.random.default_rng(5)
    S, L, H, D = 3, 7, 2, 4
    k = rng.normal(size=(S, L, H, D)).astype(np.float32)
    v = rng.normal(size=(S, L, H, D)).astype(np.float32)
    q = rng.normal(size=(S, H, D)).astype(np.float32)
    q[2] = 0.0
    ctx = np.array([1, 0, 7])
    a = oracle.oracle_decode_contiguous(q, k, v, ctx, 0.5, "f32", "SLHD")
    b = oracle.oracle_decode_contiguous(q, np.ascontiguousarray(k.transpose(0, 2, 1, 3)),
                                        np.ascontiguousarray(v.transpose(0, 2, 1, 3)), ctx, 0.5,
                                        "f32", "SHLD")
    assert np.array_equal(a, b)
    assert np.array_equal(a[0], v[0, 0].astype(np.float64))
    assert np.array_equal(a[1], np.zeros((H, D)))
    np.testing.assert_allclose(a[2], v[2].astype(np.float64).mean(axis=0), rtol=0, atol=1e-15)


def _prefill_oracle(wl, q, cu_q):
    r = oracle.run_workload(wl, decode=False)
    return r, oracle.oracle_prefill(q, r["k_cache"], r["v_cache"], r["tables"], cu_q, r["ctx"],
                                    wl.scale, wl.dtype)


def test_prefill_equals_per_position_attention():
    """Each prefill row equals attention of that query over the logical K/V as
    drawn, up to and including its own position (bit-identical), for a chunk
    after a cached prefix, a whole prompt, and a one-token chunk."""
    wl, q, cu_q = synth.make_prefill(600, 2, 16, "f32", 4, [5, 0, 9], [7, 6, 1])
    r, out = _prefill_oracle(wl, q, cu_q)
    for s in range(3):
        L, ql = int(r["ctx"][s]), int(cu_q[s + 1] - cu_q[s])
        k, v = wl.kv(s, 0, L)
        for i in range(ql):
            pos, row = L - ql + i, int(cu_q[s]) + i
            for h in range(wl.H):
                logits = wl.scale * (k[:pos + 1, h].astype(np.float64) @ q[row, h].astype(np.float64))
                e = np.exp(logits - logits.max())
                want = (e / e.sum()) @ v[:pos + 1, h].astype(np.float64)
                assert np.array_equal(out[row, h], want)


def test_prefill_closed_forms_and_causality():
    """Position 0 attends to itself only (out = V_0 exactly); the last row of a
    chunk equals the decode of that position (bit-identical); changing K/V after
    a query's position leaves its row unchanged."""
    wl, q, cu_q = synth.make_prefill(601, 2, 8, "f32", 4, [0, 3], [5, 4])
    r, out = _prefill_oracle(wl, q, cu_q)
    k0, v0 = wl.kv(0, 0, 1)
    assert np.array_equal(out[0], v0[0].astype(np.float64))
    dec = oracle.oracle_decode(q[cu_q[1:] - 1], r["k_cache"], r["v_cache"], r["tables"],
                               r["ctx"], wl.scale, wl.dtype)
    assert np.array_equal(out[cu_q[1:] - 1], dec)
    # causality: poison every cached slot after sequence 1's first query position
    kc, vc = r["k_cache"].copy(), r["v_cache"].copy()
    pos = int(r["ctx"][1]) - 4
    for t in range(pos + 1, int(r["ctx"][1])):
        b, o = r["tables"][1][t // wl.bs], t % wl.bs
        kc[b, :, o] = 1e3
        vc[b, :, o] = -1e3
    out2 = oracle.oracle_prefill(q, kc, vc, r["tables"], cu_q, r["ctx"], wl.scale, wl.dtype)
    assert np.array_equal(out2[cu_q[1]], out[cu_q[1]])
    assert not np.array_equal(out2[cu_q[1] + 1], out[cu_q[1] + 1])


def test_cache_write_places_every_token():
    """After the script, every token t of every sequence sits at
    pool[table[t//bs], :, t%bs, :], and nothing else was written."""
    for cfg, kw in ((1, {}), (4, {"cow": True})):
        wl = synth.make_workload(cfg, **kw)
        r = oracle.run_workload(wl, decode=False)
        kc, vc, tables = r["k_cache"], r["v_cache"], r["tables"]
        written = np.zeros((wl.NB, wl.bs), dtype=bool)
        for s in range(wl.S):
            L = int(r["ctx"][s])
            k, v = wl.kv(s, 0, L)
            t = np.arange(L)
            b, o = tables[s, t // wl.bs], t % wl.bs
            assert np.array_equal(kc[b, :, o, :], k) and np.array_equal(vc[b, :, o, :], v)
            written[b, o] = True
        probe = kc[:, :, :, 0] if cfg == 1 else kc[:, :1, :, 0]     # all heads on the small case
        nan_rows = np.isnan(oracle.widen(probe, wl.dtype)).all(axis=1)  # [NB, bs]
        assert np.array_equal(~nan_rows, written)


def test_permutation_invariance():
    wl = synth.make_workload(1)
    r = oracle.run_workload(wl)
    perm = np.random.default_rng(5).permutation(wl.NB)
    kc = np.empty_like(r["k_cache"])
    vc = np.empty_like(r["v_cache"])
    kc[perm] = r["k_cache"]
    vc[perm] = r["v_cache"]
    tables = perm[r["tables"]]
    out = oracle.oracle_decode(wl.q, kc, vc, tables, r["ctx"], wl.scale, wl.dtype)
    assert np.array_equal(out, r["out"])


def test_block_size_invariance():
    outs = []
    for bs in synth.SWEEP_BLOCK_SIZES:
        wl = synth.make_workload(5, bs=bs, S=3)
        outs.append(oracle.run_workload(wl)["out"])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_ctx_zero_row_is_zero():
    q = np.ones((1, 2, 4), dtype=np.float32)
    cache = np.full((2, 2, 4, 4), np.nan, dtype=np.float32)
    out = oracle.oracle_decode(q, cache, cache, np.array([[10**9]]), [0], 1.0, "f32")
    assert np.array_equal(out, np.zeros((1, 2, 4)))


def test_bf16_widening_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 65280.0, 2.0**-126], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)          # these values fit bf16 exactly
    assert np.array_equal(oracle.widen(bits, "bf16"), x.astype(np.float64))


# ------------------------------------------------------------ block manager
def _check_pool_invariants(bm):
    ref = [0] * bm.NB
    for tab in bm.tables.values():
        for b in tab:
            ref[b] += 1
    assert ref == bm.ref
    assert len(bm.free) + sum(1 for r in ref if r) == bm.NB
    assert set(bm.free).isdisjoint(b for b, r in enumerate(ref) if r)
    for s, tab in bm.tables.items():
        L = bm.lens[s]
        assert len(tab) == -(-L // bm.bs)
        assert len(tab) * bm.bs - L <= bm.bs - 1            # waste of at most bs-1 tokens


def test_block_pool_random_ops_keep_invariants():
    rng = np.random.default_rng(6)
    for trial in range(20):
        bs = int(rng.choice([2, 4, 16]))
        NB = int(rng.integers(8, 64))
        bm = oracle.BlockPoolModel(NB, bs, rng.permutation(NB))
        live, nxt = [], 0
        for _ in range(300):
            op = rng.integers(0, 4)
            try:
                if op == 0 or not live:
                    bm.add_seq(nxt, int(rng.integers(0, 3 * bs)))
                    live.append(nxt)
                    nxt += 1
                elif op == 1:
                    p = live[rng.integers(len(live))]
                    bm.fork(p, nxt)
                    live.append(nxt)
                    nxt += 1
                elif op == 2:
                    s = live[rng.integers(len(live))]
                    slot, cow = bm.append_slot(s)
                    b = slot // bs
                    assert bm.ref[b] == 1                   # never a write into a shared block
                    if cow is not None:
                        assert cow[1] == b and bm.ref[cow[0]] >= 1
                else:
                    s = live.pop(rng.integers(len(live)))
                    bm.free_seq(s)
            except oracle.BlockPoolModel.NoBlocks:
                pass
            _check_pool_invariants(bm)


def test_pool_exhaustion_raises():
    bm = oracle.BlockPoolModel(2, 4)
    bm.add_seq(0, 8)
    with pytest.raises(oracle.BlockPoolModel.NoBlocks):
        bm.append_slot(0)
    with pytest.raises(oracle.BlockPoolModel.NoBlocks):
        bm.add_seq(1, 1)


def test_useful_kv_waste_bounded():
    ctx = synth.config5_ctx()
    for bs in synth.SWEEP_BLOCK_SIZES:
        f = oracle.useful_kv_fraction(ctx, bs)
        # only each sequence's last block may hold empty slots, at most bs - 1 of them
        # (comfyai.app 6.4.1; brentwoodlivery "5.3.18" waste card)
        waste_slots = sum(ctx) / f - sum(ctx)
        assert -1e-6 <= waste_slots <= len(ctx) * (bs - 1) + 1e-6
        assert 0 < f <= 1


def test_useful_kv_fraction_hand_worked():
    """Values worked out by hand: ctx 17, 16 and 40 at block size 16 occupy 2 + 1 + 3
    blocks = 96 slots for 73 tokens; one token at block size 128 uses 1 of 128 slots;
    whole blocks waste nothing; block size 1 never wastes."""
    assert oracle.useful_kv_fraction([17, 16, 40], 16) == 73 / 96
    assert oracle.useful_kv_fraction([1], 128) == 1 / 128
    assert oracle.useful_kv_fraction([16, 32, 4096], 16) == 1.0
    assert oracle.useful_kv_fraction([3, 5, 999], 1) == 1.0
    # one token past a block boundary opens a whole block: 17 tokens in 32 slots
    assert oracle.useful_kv_fraction([17], 16) == 17 / 32


def test_useful_kv_fraction_matches_block_pool():
    """The fraction equals tokens held / slots of the blocks BlockPoolModel actually
    allocated, after random adds and appends (an independent count of the same
    allocation rule)."""
    rng = np.random.default_rng(12)
    for bs in (8, 16, 32):
        bm = oracle.BlockPoolModel(4096, bs)
        lens = {}
        for s in range(40):
            n = int(rng.integers(1, 300))
            bm.add_seq(s, n)
            lens[s] = n
        for _ in range(500):
            s = int(rng.integers(40))
            bm.append_slot(s)
            lens[s] += 1
        ctx = [lens[s] for s in range(40)]
        slots = sum(len(bm.tables[s]) for s in range(40)) * bs
        assert oracle.useful_kv_fraction(ctx, bs) == sum(ctx) / slots


# ------------------------------------------------------- planted mistakes
def _pins_pass():
    """Run the attention pins on tiny inputs; return False if one fails."""
    checks = [test_ctx1_returns_v0, test_zero_query_and_equal_keys_give_mean_of_v,
              test_two_token_closed_form_fixes_scale_and_sign,
              test_one_hot_index_probe_decodes_position, test_brute_force_tiny,
              test_block_table_example_slide10, test_permutation_invariance]
    import json
    import os
    from conftest import GOLDEN

    def golden(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)
    for c in checks:
        try:
            c(golden) if c is test_block_table_example_slide10 else c()
        except AssertionError:
            return False
    return True


def _attn_wrong_scale(q, K, V, scale):
    return _ATTN(q, K, V, scale * 1.01)


def _attn_swapped_kv(q, K, V, scale):
    return _ATTN(q, V, K, scale)


def _attn_no_normalise(q, K, V, scale):
    logits = scale * (K @ q)
    w = np.exp(logits - logits.max())
    return w @ V, w


def _attn_drop_last(q, K, V, scale):
    if K.shape[0] > 1:
        K, V = K[:-1], V[:-1]
    return _ATTN(q, K, V, scale)


_ATTN = pa.attention_one


def _gather_off_by_one(cache, table_row, ctx):
    NB, H, bs, D = cache.shape
    nblk = -(-int(ctx) // bs)
    blocks = [cache[int(table_row[j])] for j in range(nblk)]
    tokens = np.concatenate([b.transpose(1, 0, 2) for b in blocks], axis=0)
    return np.roll(tokens, 1, axis=0)[:ctx]


def _gather_head_token_swap(cache, table_row, ctx):
    NB, H, bs, D = cache.shape
    nblk = -(-int(ctx) // bs)
    blocks = [cache[int(table_row[j])] for j in range(nblk)]
    tokens = np.concatenate([b.reshape(bs, H, D) for b in blocks], axis=0)
    return tokens[:ctx]


@pytest.mark.parametrize("name,attr,fn", [
    ("wrong scale", "attention_one", _attn_wrong_scale),
    ("K and V swapped", "attention_one", _attn_swapped_kv),
    ("missing normalisation", "attention_one", _attn_no_normalise),
    ("dropped last token", "attention_one", _attn_drop_last),
    ("gather off by one", "oracle_gather", _gather_off_by_one),
    ("gather layout confusion", "oracle_gather", _gather_head_token_swap),
])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fn):
    assert _pins_pass()
    monkeypatch.setattr(pa, attr, fn)
    assert not _pins_pass(), f"no pin catches: {name}"
