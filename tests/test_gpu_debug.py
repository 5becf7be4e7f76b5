"""Device-side index checks of the PA_DEBUG build (libpa_debug.so) and
pa_debug_status.

Table entries, slots and copy pairs are caller-supplied indices into the block
pool (comfyai.app "6.4 PagedAttention" 6.4.1-6.4.2: block tables map logical
to physical blocks; polomodov.tech "vLLM and PagedAttention" slide 11: new
tokens go to slots).  A release build trusts them.  The debug build checks
each one before it becomes an address: a bad one sets a bit that
pa_debug_status returns, and is not used (a table entry reads block 0, a slot
or pair skips its write or copy), so nothing outside the pools is touched and
every other result is unchanged.  Entries of a table row past a sequence's
context are never used and never flagged.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bits, compare_outputs, log, oracle_bits, run_gpu, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


@pytest.fixture
def pk_debug():
    import paged_kv_cache_write_amd as pk
    prev = pk.use_debug_library(True)
    assert pk.lib().pa_debug_enabled() == 1
    pk.debug_status()  # start from a clear error word
    yield pk
    pk.use_debug_library(prev)


def _case(dtype="f16", H=4, D=128, bs=16, ctx=(100, 700, 1500), seed=770):
    rng = np.random.default_rng(seed)
    nbs = [-(-c // bs) for c in ctx]
    NB = sum(nbs) + 8
    perm = rng.permutation(NB).astype(np.int32)
    W = max(nbs) + 3
    tables = np.full((len(ctx), W), -7, np.int32)  # entries past the context: never used
    pos = 0
    for i, n in enumerate(nbs):
        tables[i, :n] = perm[pos:pos + n]
        pos += n
    shape = (NB, H, bs, D)
    kc = synth.to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)
    vc = synth.to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)
    q = synth.to_storage(rng.standard_normal((len(ctx), H, D), dtype=np.float32), dtype)
    return kc, vc, q, tables, np.array(ctx, np.int32)


@pytest.mark.parametrize("partition_tokens", [0, 256])
def test_release_library_reports_nothing(partition_tokens):
    import paged_kv_cache_write_amd as pk
    assert pk.lib().pa_debug_enabled() == 0
    kc, vc, q, tables, ctx = _case()
    kd, vd, qd = to_dev(kc, "f16"), to_dev(vc, "f16"), to_dev(q, "f16")
    out = pk.decode(qd, kd, vd, torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(),
                    1 / np.sqrt(128), int(ctx.max()), partition_tokens=partition_tokens)
    assert pk.debug_status() == 0
    ref = oracle.oracle_decode(q, kc, vc, tables, ctx, 1 / np.sqrt(128), "f16")
    compare_outputs(out, ref, what="release", cast_dtype="f16")


@pytest.mark.parametrize("dtype,partition_tokens", [("f16", 0), ("bf16", 256), ("f32", 512)])
def test_debug_decode_valid_and_bad_table_entries(pk_debug, dtype, partition_tokens):
    """Valid tables (with garbage past each context): no bit, oracle outputs.
    One entry inside sequence 1's context out of the pool: the TABLE bit, and
    sequences 0 and 2 still match the oracle."""
    pk = pk_debug
    kc, vc, q, tables, ctx = _case(dtype)
    scale = 1 / np.sqrt(q.shape[2])
    kd, vd, qd = to_dev(kc, dtype), to_dev(vc, dtype), to_dev(q, dtype)
    cd = torch.from_numpy(ctx).cuda()
    ref = oracle.oracle_decode(q, kc, vc, tables, ctx, scale, dtype)
    out = pk.decode(qd, kd, vd, torch.from_numpy(tables).cuda(), cd, scale, int(ctx.max()),
                    partition_tokens=partition_tokens)
    assert pk.debug_status() == 0
    compare_outputs(out, ref, what=f"debug valid {dtype}", cast_dtype=dtype)
    bad = tables.copy()
    bad[1, 3] = kc.shape[0] + 5  # tokens 48..63 of a 700-token context
    log(f"case debug bad table entry {dtype} partition={partition_tokens}")
    out = pk.decode(qd, kd, vd, torch.from_numpy(bad).cuda(), cd, scale, int(ctx.max()),
                    partition_tokens=partition_tokens)
    assert pk.debug_status() == pk.PA_DEBUG_TABLE
    assert pk.debug_status() == 0  # read and cleared
    compare_outputs(out, ref, seqs=[0, 2], what=f"debug bad table {dtype}", cast_dtype=dtype)


def test_debug_shared_prefix_group_table_entry(pk_debug):
    """The group (shared-prefix) kernel checks the shared blocks' entries."""
    pk = pk_debug
    kc, vc, q, tables, ctx = _case("f16", ctx=(1100, 1100, 1300))
    tables[1, :64] = tables[0, :64]  # sequences 0 and 1 share 1024 tokens
    d = pk.decode_schedule_shared(ctx, tables, 4, 128, 16, 1, 0)
    assert len(d["groups"]) > 0
    kd, vd, qd = to_dev(kc, "f16"), to_dev(vc, "f16"), to_dev(q, "f16")
    ws = torch.zeros(max(d["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")
    args = dict(items=torch.from_numpy(d["items"]).cuda(),
                groups=torch.from_numpy(d["groups"]).cuda(),
                members=torch.from_numpy(d["members"]).cuda())
    cd = torch.from_numpy(ctx).cuda()
    ref = oracle.oracle_decode(q, kc, vc, tables, ctx, 0.1, "f16")
    out = pk.decode_scheduled_shared(qd, kd, vd, torch.from_numpy(tables).cuda(), cd, 0.1,
                                     d["max_context_len"], args["items"], args["groups"],
                                     args["members"], d["partition_tokens"], workspace=ws)
    assert pk.debug_status() == 0
    compare_outputs(out, ref, what="debug shared valid", cast_dtype="f16")
    bad = tables.copy()
    bad[:2, 5] = -3  # a shared block (the group reads it through its first member's row)
    out = pk.decode_scheduled_shared(qd, kd, vd, torch.from_numpy(bad).cuda(), cd, 0.1,
                                     d["max_context_len"], args["items"], args["groups"],
                                     args["members"], d["partition_tokens"], workspace=ws)
    assert pk.debug_status() & pk.PA_DEBUG_TABLE
    compare_outputs(out, ref, seqs=[2], what="debug shared bad", cast_dtype="f16")


def test_debug_cache_write_and_copies(pk_debug):
    """A slot past the pool sets the SLOT bit and is skipped; copy pairs out of
    their pools set the PAIR bit and are skipped; everything else lands
    bit-exactly where the oracle puts it."""
    pk = pk_debug
    rng = np.random.default_rng(771)
    NB, H, bs, D, N = 24, 4, 16, 64, 6
    kc = synth.to_storage(rng.standard_normal((NB, H, bs, D), dtype=np.float32), "f16")
    vc = synth.to_storage(rng.standard_normal((NB, H, bs, D), dtype=np.float32), "f16")
    k = synth.to_storage(rng.standard_normal((N, H, D), dtype=np.float32), "f16")
    v = synth.to_storage(rng.standard_normal((N, H, D), dtype=np.float32), "f16")
    slots = np.array([5, 40, -1, NB * bs + 3, 100, 383], np.int64)
    kd, vd = to_dev(kc, "f16"), to_dev(vc, "f16")
    pk.cache_write(to_dev(k, "f16"), to_dev(v, "f16"), torch.from_numpy(slots).cuda(), kd, vd)
    assert pk.debug_status() == pk.PA_DEBUG_SLOT
    ok = slots.copy()
    ok[3] = -1  # the bad slot is skipped
    ko, vo = kc.copy(), vc.copy()
    oracle.oracle_cache_write(k, v, ok, ko, vo)
    assert np.array_equal(bits(kd), oracle_bits(ko, "f16"))
    assert np.array_equal(bits(vd), oracle_bits(vo, "f16"))
    pairs = np.array([[1, 7], [NB + 1, 2], [3, -1], [4, 9]], np.int32)
    pk.copy_blocks(kd, vd, torch.from_numpy(pairs).cuda())
    assert pk.debug_status() == pk.PA_DEBUG_PAIR
    oracle.oracle_copy_blocks(ko, vo, pairs[[0, 3]])
    assert np.array_equal(bits(kd), oracle_bits(ko, "f16"))
    assert np.array_equal(bits(vd), oracle_bits(vo, "f16"))
    hk = torch.zeros((4, H, bs, D), dtype=torch.float16, pin_memory=True)
    hv = torch.zeros((4, H, bs, D), dtype=torch.float16, pin_memory=True)
    out_pairs = torch.tensor([[2, 0], [3, 4]], dtype=torch.int32).cuda()  # dst 4 >= 4 host blocks
    pk.copy_blocks_between(kd, vd, hk, hv, out_pairs)
    assert pk.debug_status() == pk.PA_DEBUG_PAIR
    assert np.array_equal(hk[0].view(torch.int16).numpy(), oracle_bits(ko[2], "f16"))
    assert int(hk[1:].view(torch.int16).abs().sum()) == 0


def test_debug_prefill_table_entry(pk_debug):
    """pa_prefill's block ids: a bad entry inside sequence 1's context sets the
    TABLE bit; sequence 0's rows still match the oracle."""
    pk = pk_debug
    synth.cache_draws(False)
    wl, q, cu_q = synth.make_prefill(772, 4, 128, "f16", 16, [300, 0], [90, 200])
    eng = run_gpu(wl)["engine"]
    tables, ctx = eng.bm.block_tables(np.arange(2), wl.max_blocks_per_seq, wl.poison_block)
    r = oracle.run_workload(wl, decode=False)
    assert np.array_equal(tables, r["tables"]) and np.array_equal(ctx, r["ctx"])
    ref = oracle.oracle_prefill(q, r["k_cache"], r["v_cache"], r["tables"], cu_q, r["ctx"],
                                wl.scale, wl.dtype)
    assert pk.debug_status() == 0
    args = (to_dev(q, "f16"), eng.k_cache, eng.v_cache)
    extra = (torch.from_numpy(cu_q).cuda(), torch.from_numpy(ctx).cuda(), wl.scale,
             int(np.diff(cu_q).max()))
    out = pk.prefill(*args, torch.from_numpy(tables).cuda(), *extra)
    assert pk.debug_status() == 0
    compare_outputs(out, ref, what="debug prefill valid", cast_dtype="f16")
    bad = tables.copy()
    bad[1, 2] = eng.NB + 11  # tokens 32..47 of a 200-token prompt
    out = pk.prefill(*args, torch.from_numpy(bad).cuda(), *extra)
    assert pk.debug_status() == pk.PA_DEBUG_TABLE
    rows0 = torch.arange(int(cu_q[0]), int(cu_q[1]), device="cuda")
    compare_outputs(out[rows0], ref[cu_q[0]:cu_q[1]], what="debug prefill bad",
                    cast_dtype="f16")


@pytest.mark.parametrize("debug", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_malformed_group_item_keeps_counters(debug, dtype):
    """A shared-prefix group item whose token count is not one whole 256-token
    partition streams nothing: each member gets a partial of weight zero at the
    item's partition, every row still completes, and the row counters return to
    zero, so the next call with the builder's lists on the same workspace gives
    the bits of a call on a fresh one.  The debug build also reports
    PA_DEBUG_ITEM; every kernel exits normally in both builds."""
    import paged_kv_cache_write_amd as pk
    from test_gpu_shared import _direct_case
    prev = pk.use_debug_library(debug)
    try:
        pk.debug_status()
        codes = {"f32": 0, "f16": 1, "bf16": 2}
        kc, vc, q, tables, ctx, poison = _direct_case(dtype, 16)
        H, D = q.shape[1], q.shape[2]
        scale = 1.0 / np.sqrt(D)
        d = pk.decode_schedule_shared(ctx, tables, H, D, 16, codes[dtype], 0)
        assert len(d["groups"]) > 1
        log(f"case malformed group item {dtype} debug={debug}: {len(d['groups'])} group items")
        kd, vd, qd = to_dev(kc, dtype), to_dev(vc, dtype), to_dev(q, dtype)
        td, cd = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
        items = torch.from_numpy(d["items"]).cuda()
        members = torch.from_numpy(d["members"]).cuda()
        good = torch.from_numpy(d["groups"]).cuda()
        bad_h = d["groups"].copy()
        bad_h[0, 4] = 128                       # half a shared partition
        bad = torch.from_numpy(bad_h).cuda()
        run = lambda groups, ws: pk.decode_scheduled_shared(
            qd, kd, vd, td, cd, scale, d["max_context_len"], items, groups, members,
            d["partition_tokens"], workspace=ws)
        nbytes = max(d["workspace_bytes"], 16)
        fresh = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        ref = bits(run(good, fresh))
        torch.cuda.synchronize()
        assert pk.debug_status() == 0
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        o = run(bad, ws)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o.float()).all())
        assert int(ws[: len(ctx) * H * 4].view(torch.int32).abs().sum().item()) == 0
        assert pk.debug_status() == (pk.PA_DEBUG_ITEM if debug else 0)
        again = bits(run(good, ws))
        torch.cuda.synchronize()
        assert np.array_equal(again, ref)
        assert pk.debug_status() == 0
    finally:
        pk.use_debug_library(prev)


def test_debug_flags_single_item_outside_workspace(pk_debug):
    """Debug build: a single work item whose partition index lies past the
    workspace does nothing (no store) and sets PA_DEBUG_ITEM; after the workspace
    is zero-filled again, the builder's list gives the reference bits.  (A release
    build trusts the list: this case runs on the debug build only.)"""
    pk = pk_debug
    kc, vc, q, tables, ctx = _case()
    scale = 1 / np.sqrt(q.shape[2])
    items_h, pt, mx = pk.decode_schedule(ctx, 4, 128, 16, 1, 256)
    kd, vd, qd = to_dev(kc, "f16"), to_dev(vc, "f16"), to_dev(q, "f16")
    td, cd = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    nbytes = max(pk.decode_workspace_size(len(ctx), 4, 128, 16, mx, 1, pt), 16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    items = torch.from_numpy(items_h).cuda()
    ref = bits(pk.decode_scheduled(qd, kd, vd, td, cd, scale, mx, items, pt, workspace=ws))
    torch.cuda.synchronize()
    assert pk.debug_status() == 0
    bad_h = items_h.copy()
    bad_h[0, 1] = 1 << 20                        # partition index far past the workspace
    pk.decode_scheduled(qd, kd, vd, td, cd, scale, mx, torch.from_numpy(bad_h).cuda(), pt,
                        workspace=ws)
    assert pk.debug_status() == pk.PA_DEBUG_ITEM
    ws.zero_()
    again = bits(pk.decode_scheduled(qd, kd, vd, td, cd, scale, mx, items, pt, workspace=ws))
    torch.cuda.synchronize()
    assert np.array_equal(again, ref)
