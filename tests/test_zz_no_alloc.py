"""pa_decode_noalloc, the decode whose scratch (row counters and partials) is the
library's own device array, for callers that cannot allocate device memory.
Through the C ABI it must give pa_decode's bits (same kernels, same plan) on
calls in a row, the second with a smaller input, and refuse a call that needs
more scratch than the array holds before any launch."""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bits, compare_outputs, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

CODES = {"f32": 0, "f16": 1, "bf16": 2}


def _case(seed, S, H, D, bs, lo, hi, dtype):
    """Seeded scattered pool, tables padded with a NaN block, q/K/V ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(lo, hi + 1, S).astype(np.int32)
    nbs = -(-ctx // bs)
    NB = int(nbs.sum()) + 1
    perm = rng.permutation(NB).astype(np.int32)
    poison = int(perm[-1])
    tables = np.full((S, int(nbs.max())), poison, np.int32)
    pos = 0
    for i, n in enumerate(nbs):
        tables[i, :n] = perm[pos:pos + n]
        pos += n
    shape = (NB, H, bs, D)
    kc = synth.to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)
    vc = synth.to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)
    q = synth.to_storage(rng.standard_normal((S, H, D), dtype=np.float32), dtype)
    return q, kc, vc, tables, ctx, poison


def _run_both(pk, q, kc, vc, tables, ctx, poison, dtype, pt):
    """pa_decode (torch-allocated zeroed workspace) and pa_decode_noalloc on the same
    inputs; returns both outputs."""
    S, H, D = q.shape
    NB, _, bs, _ = kc.shape
    kd, vd, qd = to_dev(kc, dtype), to_dev(vc, dtype), to_dev(q, dtype)
    kd[poison] = float("nan")
    vd[poison] = float("nan")
    td, cd = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    mx = int(ctx.max())
    scale = 1.0 / np.sqrt(D)
    need = pk.decode_workspace_size(S, H, D, bs, mx, CODES[dtype], pt)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    o_ref, o_na = torch.empty_like(qd), torch.empty_like(qd)
    st = torch.cuda.current_stream().cuda_stream
    L = pk.lib()
    rc = L.pa_decode(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), td.data_ptr(), tables.shape[1],
                     cd.data_ptr(), S, H, D, bs, NB, scale, mx, CODES[dtype], o_ref.data_ptr(),
                     ws.data_ptr(), ws.numel(), pt, st)
    assert rc == 0, rc
    rc = L.pa_decode_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), td.data_ptr(),
                             tables.shape[1], cd.data_ptr(), S, H, D, bs, NB, scale, mx,
                             CODES[dtype], o_na.data_ptr(), pt, st)
    assert rc == 0, rc
    torch.cuda.synchronize()
    log(f"  workspace the call needs: {need} bytes")
    return o_ref, o_na


def test_noalloc_matches_pa_decode():
    import paged_kv_cache_write_amd as pk
    cases = [  # (seed, S, H, D, bs, ctx lo, ctx hi, dtype, partition_tokens)
        (9101, 30, 40, 128, 16, 256, 2048, "f16", 0),     # the 13B-layer batch shape
        (9102, 5, 8, 64, 32, 1, 900, "bf16", 64),         # smaller, many short partitions
        (9103, 30, 40, 128, 16, 256, 2048, "f16", 0),     # the first shape again
    ]
    for seed, S, H, D, bs, lo, hi, dtype, pt in cases:
        log(f"case noalloc seed={seed} S={S} H={H} D={D} bs={bs} {dtype} pt={pt}")
        q, kc, vc, tables, ctx, poison = _case(seed, S, H, D, bs, lo, hi, dtype)
        o_ref, o_na = _run_both(pk, q, kc, vc, tables, ctx, poison, dtype, pt)
        assert np.array_equal(bits(o_na), bits(o_ref)), "pa_decode_noalloc differs from pa_decode"
        ref = oracle.oracle_decode(q, kc, vc, tables, ctx, 1.0 / np.sqrt(D), dtype)
        compare_outputs(o_na, ref, what=f"noalloc seed {seed}", cast_dtype=dtype)


def test_noalloc_refuses_more_than_its_scratch():
    """256 sequences x 40 heads of 4096 tokens in 32-token partitions need ~680 MB of
    partials: PA_ERR_WORKSPACE before any pointer is used (null pointers here)."""
    import paged_kv_cache_write_amd as pk
    need = pk.decode_workspace_size(256, 40, 128, 16, 4096, 1, 32)
    assert need > 32 << 20
    rc = pk.lib().pa_decode_noalloc(None, None, None, None, 256, None, 256, 40, 128, 16, 4096,
                                    0.1, 4096, 1, None, 32, None)
    assert rc == -5                  # PA_ERR_WORKSPACE
