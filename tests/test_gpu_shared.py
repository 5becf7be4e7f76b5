"""GPU parity of the shared-prefix decode (group items) against the oracle.

Sequences forked from one prompt point at the same physical blocks until they
write (comfyai.app "6.4 PagedAttention" 6.4.2-6.4.3; polomodov.tech "vLLM and
PagedAttention" slides 13-14).  The launcher streams such blocks once per
group of sequences; the result must still be each sequence's own attention:
within 2e-3 of the float64 oracle, with sharing on or off.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bits, check_workload, compare_outputs, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


@pytest.mark.parametrize("dtype,bs,D", [("f16", 16, 128), ("bf16", 8, 128), ("f32", 32, 64),
                                        ("f16", 64, 64), ("bf16", 128, 128)])
def test_fork_tree(dtype, bs, D):
    """Random fork trees with long prompts: forks of forks, parents extended after
    forking, copies on write; groups of every size up to 8 and beyond."""
    seed = 520 + bs
    wl = synth.make_fork_tree(seed, 4, D, dtype, bs, roots=3, forks=14, max_extend=300,
                              prompt_lens=[1100, 700, 300])
    g, r, _ = check_workload(wl, cast_bound=True)
    info = g["engine"].last_step
    log(f"  group items {info['num_group_items']}, single items {info['num_items']}")
    assert info["num_group_items"] > 0


@pytest.mark.parametrize("dtype,bs,width", [("f16", 16, 4), ("bf16", 8, 8), ("f32", 32, 4)])
def test_beam_search(dtype, bs, width):
    """Beam search as a block tree: 20 rounds of appends and selections (repeated
    parents, retired beams freed, children copying their parent's shared last
    block on write), then a decode of every beam; the 600-token prompt is shared
    by all beams, so the decode uses group items."""
    wl = synth.make_beam_search(560 + bs, 4, 128, dtype, bs, prompt=600, width=width, steps=20)
    g, r, _ = check_workload(wl, cast_bound=True)
    assert r["all_cows"].shape[0] > 0
    assert g["engine"].last_step["num_group_items"] > 0


@pytest.mark.parametrize("dtype,bs", [("f16", 16), ("bf16", 8), ("f32", 32)])
def test_preemption_swap(dtype, bs):
    """The newest request (a group of 2 samples) is swapped out to the pinned host
    pool, the others reuse its device blocks, it is swapped back into other
    blocks: pools bit-exact with the oracle and every sequence decodes correctly."""
    wl = synth.make_preemption(930 + bs, 4, 128, dtype, bs)
    check_workload(wl, cast_bound=True)


def test_fork_tree_forced_short_partitions():
    """Group items of 256 tokens next to single items of 64: the workspace stride
    and partition indices of both kinds interleave in one row."""
    wl = synth.make_fork_tree(530, 8, 128, "f16", 16, roots=2, forks=10, max_extend=400,
                              prompt_lens=[1300, 520])
    g, r, _ = check_workload(wl, partition_tokens=64)
    assert g["engine"].last_step["num_group_items"] > 0


def _direct_case(dtype, bs, H=4, D=128, seed=540):
    """Hand-built tables: pairs with identical rows (the shared run stops one
    token short of the context: 256 gives no group, 512 one group partition and a
    single item of 256 tokens), a pair that diverges inside a block, a group of 11
    and a loner."""
    rng = np.random.default_rng(seed)
    spec = [(256, "A"), (256, "A"), (512, "B"), (512, "B"), (1000, "C"), (300, "C"),
            (777, None), (0, None)] + [(600 + 37 * i, "D") for i in range(11)]
    nbt = {k: 0 for k in "ABCD"}
    for n, k in spec:
        if k:
            nbt[k] = max(nbt[k], -(-n // bs))
    need = sum(-(-n // bs) for n, _ in spec) + sum(nbt.values())
    NB = need + 4
    perm = rng.permutation(NB).astype(np.int32)
    pos = [0]

    def take(n):
        out = perm[pos[0]:pos[0] + n]
        pos[0] += n
        return out
    prefix = {k: take(v) for k, v in nbt.items()}
    W = max(-(-n // bs) for n, _ in spec)
    poison = int(perm[-1])
    tables = np.full((len(spec), W), poison, np.int32)
    for i, (n, k) in enumerate(spec):
        nb = -(-n // bs)
        if k is None:
            tables[i, :nb] = take(nb)
            continue
        row = prefix[k][:nb].copy()
        if k == "C" and i == 5:            # diverges at token 290: own blocks from there
            cut = 290 // bs
            row[cut:] = take(nb - cut)
        if k == "D":                       # members keep 600 shared tokens, own tails
            cut = 600 // bs
            row[cut:] = take(nb - cut)
        tables[i, :nb] = row
    ctx = np.array([n for n, _ in spec], np.int32)
    shape = (NB, H, bs, D)
    kc = synth.to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)
    vc = synth.to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)
    q = synth.to_storage(rng.standard_normal((len(spec), H, D), dtype=np.float32), dtype)
    return kc, vc, q, tables, ctx, poison


@pytest.mark.parametrize("dtype,bs,D", [("f16", 16, 128), ("bf16", 32, 128), ("f32", 8, 128),
                                        ("bf16", 16, 64), ("f16", 8, 64)])
def test_direct_shared_entry_points(dtype, bs, D):
    """pa_decode_schedule_shared + pa_decode_scheduled_shared through the C ABI on
    hand-built tables, against the oracle; called eight times (counters return
    to zero, bits repeat whichever wave merges a row) and against pa_decode
    without groups."""
    import paged_kv_cache_write_amd as pk
    codes = {"f32": 0, "f16": 1, "bf16": 2}
    kc, vc, q, tables, ctx, poison = _direct_case(dtype, bs, D=D)
    H, D = q.shape[1], q.shape[2]
    scale = 1.0 / np.sqrt(D)
    log(f"case direct-shared {dtype} bs={bs} D={D} S={len(ctx)}")
    d = pk.decode_schedule_shared(ctx, tables, H, D, bs, codes[dtype], 0)
    assert len(d["groups"]) > 0
    cnts = sorted(set(map(tuple, d["groups"][:, :2].tolist())))
    log(f"  groups (member offset, count): {cnts}")
    ref = oracle.oracle_decode(q, kc, vc, tables, ctx, scale, dtype)
    kd, vd, qd = to_dev(kc, dtype), to_dev(vc, dtype), to_dev(q, dtype)
    # poison the block that pads every table row
    kd[poison] = float("nan")
    vd[poison] = float("nan")
    td, cd = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    items = torch.from_numpy(d["items"]).cuda()
    groups = torch.from_numpy(d["groups"]).cuda()
    members = torch.from_numpy(d["members"]).cuda()
    ws = torch.zeros(max(d["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(8):
        o = pk.decode_scheduled_shared(qd, kd, vd, td, cd, scale, d["max_context_len"], items,
                                       groups, members, d["partition_tokens"], workspace=ws)
        torch.cuda.synchronize()
        outs.append(bits(o))
        assert int(ws[: len(ctx) * H * 4].view(torch.int32).abs().sum().item()) == 0
    assert all(np.array_equal(x, outs[0]) for x in outs)
    compare_outputs(o, ref, what=f"direct shared {dtype}", cast_dtype=dtype)
    plain = pk.decode(qd, kd, vd, td, cd, scale, int(ctx.max()))
    compare_outputs(plain, ref, what=f"direct plain {dtype}", cast_dtype=dtype)


def test_shared_entry_point_errors():
    """Groups without members, or no work at all, are rejected before any launch."""
    import paged_kv_cache_write_amd as pk
    kc, vc, q, tables, ctx, _ = _direct_case("f16", 16)
    d = pk.decode_schedule_shared(ctx, tables, 4, 128, 16, 1, 0)
    qd, kd, vd = to_dev(q, "f16"), to_dev(kc, "f16"), to_dev(vc, "f16")
    td, cd = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    groups = torch.from_numpy(d["groups"]).cuda()
    ws = torch.zeros(d["workspace_bytes"], dtype=torch.uint8, device="cuda")
    L = pk.lib()
    args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), td.data_ptr(), tables.shape[1],
            cd.data_ptr(), len(ctx), 4, 128, 16, kd.shape[0], 0.1, int(ctx.max()), 1,
            torch.empty_like(qd).data_ptr(), ws.data_ptr(), ws.numel(),
            d["partition_tokens"], None)
    assert L.pa_decode_scheduled_shared(*args, None, 0, groups.data_ptr(), len(groups),
                                        None) == -1
    assert L.pa_decode_scheduled_shared(*args, None, 0, None, 0, None) == -1
    torch.cuda.synchronize()


def test_config4_merges_repeat_bit_for_bit():
    """Shared-prefix workload at full size (64 sequences in 8 groups, bf16): a
    row's partials are merged by whichever wave finishes it last, a group wave
    (several rows at once) or a single wave (one row), so thirty calls in a row
    must give the same bits, leave the counters at zero and match the oracle."""
    import paged_kv_cache_write_amd as pk
    from gpu_harness import run_gpu
    wl = synth.make_workload(4)
    g = run_gpu(wl)
    eng = g["engine"]
    step = np.array([op for op in wl.ops if op[0] == "step"][-1][1], dtype=np.int64)
    tables, ctx = eng.bm.block_tables(step, wl.max_blocks_per_seq, wl.poison_block)
    d = pk.decode_schedule_shared(ctx, tables, wl.H, wl.D, wl.bs, 2, 0)
    assert len(d["groups"]) > 0
    q = to_dev(wl.q, wl.dtype)
    td, cd = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    items = torch.from_numpy(d["items"]).cuda()
    groups = torch.from_numpy(d["groups"]).cuda()
    members = torch.from_numpy(d["members"]).cuda()
    ws = torch.zeros(max(d["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(q) for _ in range(30)]
    for o in outs:
        pk.decode_scheduled_shared(q, eng.k_cache, eng.v_cache, td, cd, wl.scale,
                                   d["max_context_len"], items, groups, members,
                                   d["partition_tokens"], out=o, workspace=ws)
    torch.cuda.synchronize()
    want = bits(outs[0])
    bad = sum(not np.array_equal(bits(o), want) for o in outs)
    assert bad == 0, f"{bad} of {len(outs)} calls differ"
    assert int(ws[: len(ctx) * wl.H * 4].view(torch.int32).abs().sum().item()) == 0
    compare_outputs(g["out"], oracle.run_workload(wl)["out"], what="config 4 engine step")
    assert np.array_equal(bits(g["out"]), want), "the engine step's own decode differs"
    log(f"config 4: {len(outs)} calls bit-identical, {len(d['groups'])} group items")
