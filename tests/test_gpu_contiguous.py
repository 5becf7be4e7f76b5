"""GPU parity of the non-paged decode (pa_decode_contiguous) against the oracle.

polomodov.tech "vLLM and PagedAttention" slide 19 compares the paged kernel
with attention over contiguous K/V.  The contiguous entry point computes the
same attention with token rows addressed by strides; with the same partitions
it runs the same arithmetic in the same order as the paged decode, so on
identical data the two agree bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bits, compare_outputs, contiguous_kv, log, run_gpu, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

CODES = {"f32": 0, "f16": 1, "bf16": 2}


@pytest.mark.parametrize("layout", ["SLHD", "SHLD"])
@pytest.mark.parametrize("dtype,D", [("f16", 128), ("bf16", 64), ("f32", 128)])
def test_contiguous_vs_oracle(dtype, D, layout):
    """Ragged contexts (0, 1, chunk and partition boundaries +-1, several
    partitions), grid order and a work list, automatic and forced-short partitions."""
    synth.cache_draws(False)
    ctx = np.array([1, 31, 32, 33, 1000, 2100, 1024, 5])
    wl = synth.make_custom(800 + D + CODES[dtype], 3, D, dtype, 16, ctx)
    k, v = contiguous_kv(wl, ctx, layout)
    ctx0 = ctx.copy()
    ctx0[-1] = 0                                   # a zero context row
    ref = oracle.oracle_decode_contiguous(wl.q, k, v, ctx0, wl.scale, dtype, layout)
    kd, vd, qd = to_dev(k, dtype), to_dev(v, dtype), to_dev(wl.q, dtype)
    cd = torch.from_numpy(ctx0.astype(np.int32)).cuda()
    mx = int(ctx0.max())
    log(f"case contiguous {dtype} D={D} {layout} ctx={ctx0.tolist()}")
    for pt in (0, 64):
        o = pk().decode_contiguous(qd, kd, vd, cd, wl.scale, mx, layout=layout,
                                   partition_tokens=pt)
        compare_outputs(o, ref, what=f"contiguous {layout} pt={pt} grid", cast_dtype=dtype)
        items, pt2, mx2 = pk().decode_schedule(ctx0.astype(np.int32), wl.H, D, 16, CODES[dtype], pt)
        o2 = pk().decode_contiguous(qd, kd, vd, cd, wl.scale, mx2, layout=layout,
                                    partition_tokens=pt2, items=torch.from_numpy(items).cuda())
        compare_outputs(o2, ref, what=f"contiguous {layout} pt={pt2} scheduled", cast_dtype=dtype)


def pk():
    import paged_kv_cache_write_amd as m
    return m


def test_contiguous_bit_identical_to_paged():
    """The 13B-layer workload: paged decode (through the engine) and contiguous
    decode of the same logical K/V with the same work list give the same bits."""
    synth.cache_draws(False)
    wl = synth.make_workload(2)
    g = run_gpu(wl)
    eng = g["engine"]
    step = np.array([op for op in wl.ops if op[0] == "step"][-1][1], dtype=np.int64)
    tables, ctx = eng.bm.block_tables(step, wl.max_blocks_per_seq, wl.poison_block)
    pt = eng.last_step["partition_tokens"]
    # the engine's own (automatic) work list, rebuilt from the same contexts
    items, pt2, mx = pk().decode_schedule(ctx, wl.H, wl.D, wl.bs, CODES[wl.dtype], 0)
    assert pt2 == pt
    k, v = contiguous_kv(wl, ctx, "SLHD")
    qd = to_dev(wl.q, wl.dtype)
    o = pk().decode_contiguous(qd, to_dev(k, wl.dtype), to_dev(v, wl.dtype),
                               torch.from_numpy(ctx).cuda(), wl.scale, mx, layout="SLHD",
                               partition_tokens=pt, items=torch.from_numpy(items).cuda())
    torch.cuda.synchronize()
    same = np.array_equal(bits(o), bits(g["out"]))
    log(f"contiguous vs paged (engine) bit-identical: {same}")
    assert same


def test_contiguous_rejects_bad_strides():
    L = pk().lib()
    q = torch.zeros(2, 2, 64, dtype=torch.float16, device="cuda")
    k = torch.zeros(2, 8, 2, 64, dtype=torch.float16, device="cuda")
    c = torch.ones(2, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    args = [q.data_ptr(), k.data_ptr(), k.data_ptr(), c.data_ptr(), 2, 2, 64, 8 * 2 * 64, 2 * 64,
            64, 8, 0.1, 1, 1, o.data_ptr(), None, 0, 0, None, None, 0]
    assert L.pa_decode_contiguous(*args) == 0
    bad = list(args)
    bad[8] = 2 * 64 + 3                            # token stride not 16-byte aligned
    assert L.pa_decode_contiguous(*bad) == -1
    bad = list(args)
    bad[12] = 9                                    # max_context_len beyond max_tokens
    assert L.pa_decode_contiguous(*bad) == -1
    torch.cuda.synchronize()
