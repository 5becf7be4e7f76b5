"""GPU parity: the HIP path (through the C ABI) against the oracle.

Pools, tables, slot mappings and copy-on-write pairs must be bit-exact;
attention outputs within 2e-3 absolute of the float64 oracle, finite, with
never-written pool slots and unused table entries poisoned with NaN.
"""
import math
import time

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import TOL, bits, compare_outputs, log, oracle_bits, run_gpu, to_dev
from gpu_harness import check_workload as _check_workload
from gpu_harness import same_storage as _same_storage

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


# ------------------------------------------------------------ the 5 configs
def test_config1_tiny_fp32():
    wl = synth.make_workload(1)
    g, r, _ = _check_workload(wl)
    # ctx = 1: softmax weight exactly 1, so out == V of the only token, bit for bit
    s0 = int(np.argmin(wl.ctx))
    assert wl.ctx[s0] == 1
    _, v = wl.kv(s0, 0, 1)
    assert np.array_equal(bits(g["out"][s0]), oracle_bits(v[0], "f32"))


def test_config2_llama13b_layer():
    _check_workload(synth.make_workload(2))


def test_mapped_staging_available():
    """The engine's host-written device staging (large PCIe BAR) is there on this
    GPU, so the steps above ran the decode that writes the new tokens itself."""
    from paged_kv_cache_write_amd.engine import PagedKVEngine
    eng = PagedKVEngine(8, 2, 64, 16, torch.float16, 4, 2)
    if not eng.has_mapped_staging:
        pytest.skip("device memory is not mapped for the host here: the engine uses the "
                    "prologue kernel")
    eng.set_mapped_staging(False)
    eng.set_mapped_staging(True)


@pytest.mark.parametrize("dtype,D,bs", [("f16", 128, 16), ("bf16", 64, 8), ("f32", 128, 128),
                                        ("f16", 64, 32)])
def test_new_tokens_written_by_the_decode(dtype, D, bs):
    """The decode launch that writes the step's new tokens itself (mapped
    staging) against the prologue kernel's write followed by the decode: the
    same pools and the same output bits.  The contexts put the new token at
    every place in a partition's last chunk, on a full last chunk, and alone
    in a partition; the oracle checks the mapped run."""
    synth.cache_draws(False)
    ctx = [1, 2, 31, 32, 33, 63, 64, 65, 96, 97, 256, 257, 1024, 1025, 2 * 64 * bs + 32,
           2 * 64 * bs + 33]
    wl = synth.make_custom(900 + D + bs, 5, D, dtype, bs, ctx)
    g, r, _ = _check_workload(wl, cast_bound=True)
    if not g["engine"].has_mapped_staging:
        pytest.skip("no mapped staging on this device")
    g2 = run_gpu(wl, mapped=False)
    assert np.array_equal(bits(g["out"]), bits(g2["out"])), "output bits differ between the paths"
    assert torch.equal(g["engine"].k_cache.view(torch.uint8), g2["engine"].k_cache.view(torch.uint8))
    assert torch.equal(g["engine"].v_cache.view(torch.uint8), g2["engine"].v_cache.view(torch.uint8))
    pt = max(32, bs)  # short partitions: many rows end in a partition of their own
    g3 = run_gpu(wl, partition_tokens=pt)
    g4 = run_gpu(wl, partition_tokens=pt, mapped=False)
    assert np.array_equal(bits(g3["out"]), bits(g4["out"])), "split: output bits differ"
    compare_outputs(g3["out"], r["out"], what=f"{wl.name} split pt={pt}", cast_dtype=dtype)


def test_config2_prologue_staging():
    """Config 2 with mapped staging off: the prologue kernel reads the pinned host
    slot and writes the new tokens, then the decode."""
    _check_workload(synth.make_workload(2), mapped=False)


def test_config3_long_context_split():
    wl = synth.make_workload(3)
    _check_workload(wl, partition_tokens=wl.partition_tokens)


@pytest.mark.parametrize("cow", [False, True])
def test_config4_shared_prefix(cow):
    """With shared-prefix group items (32: 8 groups x 4 partitions of 256 tokens)
    and without: within tolerance of the oracle, pools bit-exact.  With mapped
    staging the shared-prefix decode launch writes the new tokens itself
    (after the step's copies on write); the prologue path gives the same bits."""
    wl = synth.make_workload(4, cow=cow)
    g, r, _ = _check_workload(wl)
    if cow:
        assert r["all_cows"].shape[0] == 7 * 8
    assert g["engine"].last_step["num_group_items"] == 32
    g_off = run_gpu(wl, sharing=False)
    assert g_off["engine"].last_step["num_group_items"] == 0
    compare_outputs(g_off["out"], r["out"], what=wl.name + " no sharing")
    _same_storage(g_off["engine"].k_cache, r["k_cache"], wl.dtype, "k_cache, no sharing")
    _same_storage(g_off["engine"].v_cache, r["v_cache"], wl.dtype, "v_cache, no sharing")
    if g["engine"].has_mapped_staging:
        for sharing, ref in ((True, g), (False, g_off)):
            gp = run_gpu(wl, sharing=sharing, mapped=False)
            assert np.array_equal(bits(gp["out"]), bits(ref["out"])), f"sharing={sharing}: bits"
            _same_storage(gp["engine"].k_cache, r["k_cache"], wl.dtype, "k_cache, prologue path")
            _same_storage(gp["engine"].v_cache, r["v_cache"], wl.dtype, "v_cache, prologue path")


@pytest.mark.parametrize("bs", synth.SWEEP_BLOCK_SIZES)
def test_config5_block_size_sweep(bs):
    """All 256 sequences x 40 heads compared with the oracle at every block size,
    through the launch the engine makes for them (4-head workgroups at this size)."""
    synth.cache_draws(True)
    wl = synth.make_workload(5, bs=bs)
    _check_workload(wl)


# ------------------------------------------------- every kernel instance
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [8, 16, 32, 64, 128])
def test_kernel_instances(dtype, D, bs):
    synth.cache_draws(False)
    # ragged: single token, block boundaries +-1, several partitions with a tail
    ctx = [1, bs - 1, bs, bs + 1, 3 * bs + 5, 1000, 2 * 64 * bs + 17]
    seed = 100 + {"f32": 0, "f16": 1, "bf16": 2}[dtype] * 100 + D + bs
    wl = synth.make_custom(seed, 3, D, dtype, bs, ctx)
    g, r, _ = _check_workload(wl, partition_tokens=0, cast_bound=True)
    # forced short partitions: the split path on every sequence longer than one
    pt = max(32, bs)
    g2 = run_gpu(wl, partition_tokens=pt)
    compare_outputs(g2["out"], r["out"], what=f"{wl.name} split pt={pt}", cast_dtype=dtype)


# ------------------------------------------------------------ size extremes
def test_long_context_many_partitions():
    """One ~100k-token context next to short ones (automatic partitions: ~98 of
    1024 tokens, the merge's path for more partitions than lanes) and a 16k one."""
    synth.cache_draws(False)
    wl = synth.make_custom(700, 2, 128, "f16", 16, [100003, 1, 16384, 77])
    _check_workload(wl, cast_bound=True)


def test_many_sequences():
    """4096 sequences of 1 to 40 tokens: 8192 rows, ragged tails, the work list
    longest first."""
    synth.cache_draws(False)
    ctx = (np.arange(4096) % 40) + 1
    wl = synth.make_custom(701, 2, 64, "bf16", 8, ctx)
    _check_workload(wl, cast_bound=True)


# ---------------------------------------------------------- exact probes
def _scatter_direct(ks, vs, H, D, dtype, bs, NB, free_order, poison, fill=float("nan")):
    """Build a pool with the library from contiguous per-sequence K/V (host arrays)."""
    from paged_kv_cache_write_amd.engine import PagedKVEngine
    maxB = max(-(-k.shape[0] // bs) for k in ks)
    eng = PagedKVEngine(NB, H, D, bs, {"f16": torch.float16, "bf16": torch.bfloat16,
                                       "f32": torch.float32}[dtype], maxB, len(ks),
                        free_order=free_order, pad_block=poison, fill=fill)
    for s, (k, v) in enumerate(zip(ks, vs)):
        eng.add_sequence(s, to_dev(k, dtype), to_dev(v, dtype))
    tables, ctx = eng.bm.block_tables(np.arange(len(ks)), maxB, poison)
    return eng, torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(), int(ctx.max())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_one_hot_index_probe(dtype):
    """q = e0 and one key 200/scale make the softmax a one-hot at t*; V encodes
    position t as (t // 64, t % 64), exact in fp16/bf16: out decodes t* exactly."""
    import paged_kv_cache_write_amd as pk
    rng = np.random.default_rng(7)
    S, H, D, bs = 12, 8, 128, 16
    scale = 1 / math.sqrt(D)
    ctx = rng.integers(1, 3000, size=S)
    ctx[0], ctx[1] = 1, 2048
    ks, vs, tstar = [], [], rng.integers(0, 1 << 30, size=(S, H)) % ctx[:, None]
    for s in range(S):
        L = int(ctx[s])
        k = np.zeros((L, H, D), np.float32)
        v = np.zeros((L, H, D), np.float32)
        t = np.arange(L)
        v[:, :, 0] = (t // 64)[:, None]
        v[:, :, 1] = (t % 64)[:, None]
        for h in range(H):
            k[tstar[s, h], h, 0] = 200 / scale
        ks.append(synth.to_storage(k, dtype))
        vs.append(synth.to_storage(v, dtype))
    NB = int(sum(-(-c // bs) for c in ctx)) + 5
    order = rng.permutation(NB).astype(np.int32)
    eng, tables, cl, mx = _scatter_direct(ks, vs, H, D, dtype, bs, NB, order[:-1], int(order[-1]))
    q = np.zeros((S, H, D), np.float32)
    q[:, :, 0] = 1
    qd = to_dev(synth.to_storage(q, dtype), dtype)
    for pt in (0, 32, 256):
        out = pk.decode(qd, eng.k_cache, eng.v_cache, tables, cl, scale, mx, partition_tokens=pt)
        o = out.float().cpu().numpy()
        dec = o[:, :, 0] * 64 + o[:, :, 1]
        assert np.array_equal(dec, tstar.astype(np.float32)), f"pt={pt}"
        assert np.all(o[:, :, 2:] == 0)
    log(f"one-hot probe {dtype}: {S * H} positions decoded exactly")


def test_permutation_invariance_bit_exact():
    """Same logical K/V at a different physical placement: identical output bits."""
    import paged_kv_cache_write_amd as pk
    wl = synth.make_custom(400, 4, 128, "f16", 16, [700, 33, 1500, 2048, 1])
    ks = [wl.kv(s, 0, int(wl.ctx[s]))[0] for s in range(wl.S)]
    vs = [wl.kv(s, 0, int(wl.ctx[s]))[1] for s in range(wl.S)]
    outs = []
    for seed in (1, 2):
        order = np.random.default_rng(seed).permutation(wl.NB).astype(np.int32)
        eng, tables, cl, mx = _scatter_direct(ks, vs, wl.H, wl.D, "f16", 16, wl.NB, order[:-1],
                                              int(order[-1]))
        q = to_dev(wl.q, "f16")
        outs.append(bits(pk.decode(q, eng.k_cache, eng.v_cache, tables, cl, wl.scale, mx)))
    assert np.array_equal(outs[0], outs[1])


def test_split_matches_single_pass():
    import paged_kv_cache_write_amd as pk
    wl = synth.make_custom(401, 8, 128, "f16", 16, [1024, 777, 1, 1000, 513, 64])
    r = oracle.run_workload(wl)
    g = run_gpu(wl, partition_tokens=1024)          # one partition per sequence
    e1 = compare_outputs(g["out"], r["out"], what="single pass")
    for pt in (32, 64, 256, 512):
        g2 = run_gpu(wl, partition_tokens=pt)
        e2 = compare_outputs(g2["out"], r["out"], what=f"split pt={pt}")
        diff = (g2["out"].float() - g["out"].float()).abs().max().item()
        assert diff <= 2 * TOL
    assert pk.decode_plan(wl.S, wl.H, wl.D, 16, 1024, 1, 1024)[1] == 1
    del e1, e2


def test_context_zero_and_negative_slots():
    import paged_kv_cache_write_amd as pk
    H, D, bs, NB = 2, 64, 16, 8
    kc = torch.full((NB, H, bs, D), float("nan"), dtype=torch.float16, device="cuda")
    vc = kc.clone()
    slot_list = [3, -1, 0, 17, -5, 1, 40, 2]
    k = torch.randn(len(slot_list), H, D, device="cuda").half()
    v = torch.randn(len(slot_list), H, D, device="cuda").half()
    slots = torch.tensor(slot_list, dtype=torch.int64, device="cuda")
    before = bits(kc)
    pk.cache_write(k, v, slots, kc, vc)
    after = bits(kc)
    written = np.zeros((NB, bs), bool)
    for n, s in enumerate(slot_list):
        if s >= 0:
            written[s // bs, s % bs] = True
            assert np.array_equal(after[s // bs, :, s % bs, :], bits(k[n]))
            assert np.array_equal(bits(vc)[s // bs, :, s % bs, :], bits(v[n]))
    a, b = after.transpose(0, 2, 1, 3), before.transpose(0, 2, 1, 3)   # [NB, bs, H, D]
    assert np.array_equal(a[~written], b[~written])                   # untouched slots
    # ctx = 0 rows are zero; their tables point at a NaN block
    q = torch.randn(3, H, D, device="cuda").half()
    tables = torch.tensor([[7, 7], [0, 7], [7, 7]], dtype=torch.int32, device="cuda")
    cl = torch.tensor([0, 4, 0], dtype=torch.int32, device="cuda")
    out = pk.decode(q, kc, vc, tables, cl, 0.125, 4)
    o = out.float().cpu().numpy()
    assert np.all(o[0] == 0) and np.all(o[2] == 0) and np.isfinite(o[1]).all()
    # empty launches are no-ops
    pk.cache_write(k[:0], v[:0], slots[:0], kc, vc)
    pk.copy_blocks(kc, vc, torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()


def test_copy_blocks_direct():
    import paged_kv_cache_write_amd as pk
    for dtype, H, D, bs in (("bf16", 40, 128, 16), ("f32", 3, 64, 128)):
        NB = 64
        rng = np.random.default_rng(3)
        k = synth.to_storage(rng.standard_normal((NB, H, bs, D), dtype=np.float32), dtype)
        v = synth.to_storage(rng.standard_normal((NB, H, bs, D), dtype=np.float32), dtype)
        perm = rng.permutation(NB)
        pairs = np.stack([perm[:20], perm[20:40]], axis=1).astype(np.int32)
        kd, vd = to_dev(k, dtype), to_dev(v, dtype)
        pk.copy_blocks(kd, vd, torch.from_numpy(pairs).cuda())
        oracle.oracle_copy_blocks(k, v, pairs)
        _same_storage(kd, k, dtype, "k after copy")
        _same_storage(vd, v, dtype, "v after copy")


def test_two_launch_and_counter_reuse():
    """pa_decode (one launch, counters) and pa_decode_partitions + pa_decode_reduce
    agree bit for bit, and the counters are left at zero call after call."""
    import paged_kv_cache_write_amd as pk
    wl = synth.make_custom(402, 8, 128, "bf16", 16, [1, 100, 700, 1500, 2048, 3000, 257, 31])
    r = oracle.run_workload(wl)
    g = run_gpu(wl, partition_tokens=128)
    eng = g["engine"]
    tables, ctx = eng.bm.block_tables(np.arange(wl.S), wl.max_blocks_per_seq, wl.poison_block)
    dt_, dc = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    q = to_dev(wl.q, "bf16")
    mx = int(ctx.max())
    ws = torch.zeros(pk.decode_workspace_size(wl.S, wl.H, wl.D, 16, mx, 2, 128), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for _ in range(3):
        outs.append(bits(pk.decode(q, eng.k_cache, eng.v_cache, dt_, dc, wl.scale, mx,
                                   workspace=ws, partition_tokens=128)))
        assert int(ws[: wl.S * wl.H * 4].view(torch.int32).abs().sum().item()) == 0
    assert all(np.array_equal(o, outs[0]) for o in outs)
    o2 = torch.empty_like(q)
    ws2 = torch.full_like(ws, 0x55)          # the two-launch form needs no zero fill
    pk.decode_partitions(q, eng.k_cache, eng.v_cache, dt_, dc, wl.scale, mx, o2, ws2, 128)
    pk.decode_reduce(q, eng.k_cache, eng.v_cache, dt_, dc, wl.scale, mx, o2, ws2, 128)
    assert np.array_equal(bits(o2), outs[0])
    compare_outputs(o2, r["out"], what="two launches", cast_dtype="bf16")


def test_fused_merge_repeatable():
    """The one-launch merge (counters + agent-scope partial exchange) gives the
    same bits as the two-launch merge on every one of many repeated calls at the
    13B-layer shape, with short partitions so that most rows are merged."""
    import paged_kv_cache_write_amd as pk
    wl = synth.make_workload(2)
    g = run_gpu(wl)
    eng = g["engine"]
    tables, ctx = eng.bm.block_tables(np.arange(wl.S), wl.max_blocks_per_seq, wl.poison_block)
    dt_, dc = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    q = to_dev(wl.q, wl.dtype)
    mx = int(ctx.max())
    for pt in (64, 256):
        ws = torch.zeros(pk.decode_workspace_size(wl.S, wl.H, wl.D, 16, mx, 1, pt),
                         dtype=torch.uint8, device="cuda")
        ref = torch.empty_like(q)
        pk.decode_partitions(q, eng.k_cache, eng.v_cache, dt_, dc, wl.scale, mx, ref, ws, pt)
        pk.decode_reduce(q, eng.k_cache, eng.v_cache, dt_, dc, wl.scale, mx, ref, ws, pt)
        ws.zero_()
        want = bits(ref)
        outs = [torch.empty_like(q) for _ in range(50)]
        for o in outs:
            pk.decode(q, eng.k_cache, eng.v_cache, dt_, dc, wl.scale, mx, out=o, workspace=ws,
                      partition_tokens=pt)
        torch.cuda.synchronize()
        bad = sum(not np.array_equal(bits(o), want) for o in outs)
        assert bad == 0, f"pt={pt}: {bad} of {len(outs)} fused calls differ from the two-launch merge"
        assert int(ws[: wl.S * wl.H * 4].view(torch.int32).abs().sum().item()) == 0
        log(f"fused merge pt={pt}: 50 calls bit-identical to the two-launch merge")


@pytest.mark.parametrize("ring,mapped,sharing", [(16, None, True), (4, None, True),
                                                 (3, None, True), (16, None, False),
                                                 (4, False, True)])
def test_engine_steps_in_flight(ring, mapped, sharing):
    """Forty engine steps enqueued behind a long GPU wait, so that the host wraps
    the staging ring several times (16 or 4 slots: one guard event per
    half; 3 slots: one event per step) while earlier steps have not run:
    every step's output, pool write and
    copy-on-write must match the oracle replaying the same steps in order.
    The staging is the engine's default (mapped device slots where the host
    can write them: the host rewrites a device slot only after its guard
    event), or the pinned host slots (mapped off); without sharing the decode
    writes the new tokens itself.
    Twice a beam-style selection (one fork, one retired sequence) happens on
    the host between in-flight steps, so later steps copy on write and reuse
    freed blocks; each step has its own q and new-token K/V."""
    import dataclasses
    wl = synth.make_fork_tree(733, 4, 128, "f16", 16, roots=2, forks=6, max_prompt=500,
                              max_extend=120)
    nsteps = 40
    S = int(wl.ctx.size)
    extra = S * (-(-(nsteps + 2) // wl.bs) + 2)
    wl2 = dataclasses.replace(
        wl, NB=wl.NB + extra,
        free_order=np.concatenate([wl.free_order,
                                   np.arange(wl.NB, wl.NB + extra, dtype=np.int32)]),
        max_blocks_per_seq=wl.max_blocks_per_seq + -(-nsteps // wl.bs) + 1)
    r = oracle.run_workload(wl2, decode=False)     # through the workload's own step
    bm, kc, vc = r["model"], r["k_cache"], r["v_cache"]
    seqs = [int(s) for s in wl.ops[-1][1]]
    g = run_gpu(wl2, ring=ring, mapped=mapped, sharing=sharing)
    eng = g["engine"]
    assert eng.ring == ring
    rng = np.random.default_rng(np.random.SeedSequence([733, 77]))
    qs, ks, vs = [], [], []
    for _ in range(nsteps):
        qs.append(synth.to_storage(rng.standard_normal((S, wl.H, wl.D)), "f16"))
        ks.append(synth.to_storage(rng.standard_normal((S, wl.H, wl.D)), "f16"))
        vs.append(synth.to_storage(rng.standard_normal((S, wl.H, wl.D)), "f16"))
    qd = [to_dev(x, "f16") for x in qs]
    kd = [to_dev(x, "f16") for x in ks]
    vd = [to_dev(x, "f16") for x in vs]
    outs = [torch.empty_like(qd[0]) for _ in range(nsteps)]
    # before step i: fork row p's sequence into a new id that takes row r's place
    selections = {12: (2, 5, 1000), 27: (0, 3, 1001)}
    gseqs = list(seqs)
    torch.cuda.synchronize()
    # the GPU stays busy (400 writes of 1 GiB, ~60 ms) while the host runs ahead
    filler = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for j in range(400):
        filler.fill_(j & 0xFF)
    f1.record()
    ahead = None
    t0 = time.perf_counter()
    for i in range(nsteps):
        if i == eng.ring // 2:  # half the ring enqueued; the wrap below waits for a guard event
            ahead = not f1.query()
            host_ms = (time.perf_counter() - t0) * 1e3
        if i in selections:
            p, rr, child = selections[i]
            eng.select([(gseqs[p], child)], [gseqs[rr]])
            gseqs[rr] = child
        eng.step(np.array(gseqs, dtype=np.int64), qd[i], kd[i], vd[i], wl.scale, out=outs[i])
    torch.cuda.synchronize()
    ncow = 0
    for i in range(nsteps):
        if i in selections:
            p, rr, child = selections[i]
            bm.fork(seqs[p], child)
            bm.free_seq(seqs[rr])
            seqs[rr] = child
        slots, cows = [], []
        for s in seqs:
            slot, cow = bm.append_slot(s)
            slots.append(slot)
            if cow is not None:
                cows.append(cow)
        ncow += len(cows)
        oracle.oracle_copy_blocks(kc, vc, cows)
        oracle.oracle_cache_write(ks[i], vs[i], slots, kc, vc)
        tables = bm.table_array(seqs, wl2.max_blocks_per_seq, wl.poison_block)
        ctx = np.array([bm.lens[s] for s in seqs], dtype=np.int64)
        ref = oracle.oracle_decode(qs[i], kc, vc, tables, ctx, wl.scale, "f16")
        compare_outputs(outs[i], ref, what=f"engine step {i + 1} of {nsteps}", cast_dtype="f16")
    _same_storage(eng.k_cache, kc, "f16", "k pool after the steps")
    _same_storage(eng.v_cache, vc, "f16", "v pool after the steps")
    log(f"ring {ring}: host enqueued {eng.ring // 2} steps in {host_ms:.2f} ms; the GPU filler took "
        f"{f0.elapsed_time(f1):.2f} ms")
    assert ahead, "the host should have filled the staging ring while the GPU was busy"
    assert ncow >= 2, "the selections should make later steps copy on write"
    log(f"{nsteps} engine steps in flight: outputs and pools match ({ncow} copies on write)")


@pytest.mark.parametrize("dtype,D,H,bs", [("bf16", 128, 40, 16), ("f32", 64, 10, 8),
                                          ("f16", 64, 12, 32)])
def test_wide_workgroup_launch(dtype, D, H, bs):
    """Work lists of 8192 waves or more run with workgroups of 4 consecutive heads
    (head counts that 4 does not divide included): pools bit-exact, every output
    within tolerance, ragged contexts that also split into several partitions."""
    rng = np.random.default_rng(np.random.SeedSequence([741, D, H]))
    S = -(-8400 // H)
    ctx = rng.integers(1, 1400, size=S)
    ctx[:7] = [1, 2, 15, 16, 17, 1023, 1399]
    wl = synth.make_custom(741 + H, H, D, dtype, bs, ctx)
    g, _, _ = _check_workload(wl, cast_bound=True)
    info = g["engine"].last_info
    assert info.num_items * H >= 8192, "the launch should be wide"
    log(f"wide launch: {info.num_items} items x {H} heads, partitions of "
        f"{info.partition_tokens} tokens")


def test_engine_batch_grows_between_steps():
    """Steps over 3, then 8, then 5, then 8 sequences of long (split) contexts on
    one engine and one workspace.  The engine reserves its workspace counters for
    its largest batch, so the partials a small step leaves never sit where a
    larger step's counters are.  Each step's output is compared with the oracle's
    decode of the engine's own pool and tables after that step."""
    from paged_kv_cache_write_amd.engine import PagedKVEngine
    synth.cache_draws(False)
    ctx0 = [1500, 2900, 700, 2200, 3000, 1800, 999, 2500]
    wl = synth.make_custom(781, 40, 128, "f16", 16, ctx0)
    extra = 4
    NB = wl.NB + len(ctx0) * extra
    free_order = np.concatenate([wl.free_order, np.arange(wl.NB, NB, dtype=np.int32)])
    eng = PagedKVEngine(NB, wl.H, wl.D, wl.bs, torch.float16, wl.max_blocks_per_seq + extra,
                        len(ctx0), free_order=free_order, pad_block=wl.poison_block,
                        fill=float("nan"))
    for op in wl.ops:
        if op[0] == "add":
            k, v = wl.kv(op[1], 0, op[2])
            eng.add_sequence(op[1], to_dev(k, wl.dtype), to_dev(v, wl.dtype))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(781)
    for step, seqs in enumerate([[0, 1, 2], list(range(8)), [3, 4, 5, 6, 7], list(range(8))]):
        log(f"case growing batch: step {step}, {len(seqs)} sequences")
        n = len(seqs)
        q = torch.randn(n, wl.H, wl.D, device="cuda", generator=gen).half()
        k_new = torch.randn(n, wl.H, wl.D, device="cuda", generator=gen).half()
        v_new = torch.randn(n, wl.H, wl.D, device="cuda", generator=gen).half()
        out = eng.step(np.array(seqs, dtype=np.int64), q, k_new, v_new, wl.scale)
        torch.cuda.synchronize()
        assert eng.last_info.partition_tokens < 3000        # the long rows are split
        tables, ctx = eng.bm.block_tables(np.array(seqs), eng.maxB, wl.poison_block)
        ref = oracle.oracle_decode(q.cpu().numpy(), eng.k_cache.cpu().numpy(),
                                   eng.v_cache.cpu().numpy(), tables, ctx, wl.scale, "f16")
        compare_outputs(out, ref, what=f"growing batch step {step}")
