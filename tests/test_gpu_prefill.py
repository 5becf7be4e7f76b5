"""GPU parity of the paged prefill attention (pa_prefill) against the oracle.

A chunk of new tokens per sequence (after a cached prefix, or a whole prompt)
is written through the slot mapping, then attends causally over the paged
cache (brentwoodlivery "5.3.18", the prefill/decode cards; comfyai.app
6.4.3).  Outputs within 2e-3 of the float64 oracle (plus the final cast's
half ulp: early positions attend to few tokens, so |out| is near 1).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_harness import compare_outputs, log, run_gpu, same_storage, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _pk():
    import paged_kv_cache_write_amd as pk
    return pk


def _run(wl, q, cu_q):
    log(f"case {wl.name}: S={len(cu_q) - 1} H={wl.H} D={wl.D} bs={wl.bs} "
        f"ctx={wl.ctx.tolist()} q_lens={np.diff(cu_q).tolist()}")
    g = run_gpu(wl)
    eng = g["engine"]
    S = len(cu_q) - 1
    tables, ctx = eng.bm.block_tables(np.arange(S), wl.max_blocks_per_seq, wl.poison_block)
    r = oracle.run_workload(wl, decode=False)
    assert np.array_equal(tables, r["tables"]) and np.array_equal(ctx, r["ctx"])
    same_storage(eng.k_cache, r["k_cache"], wl.dtype, "k_cache")
    same_storage(eng.v_cache, r["v_cache"], wl.dtype, "v_cache")
    ref = oracle.oracle_prefill(q, r["k_cache"], r["v_cache"], r["tables"], cu_q, r["ctx"],
                                wl.scale, wl.dtype)
    out = _pk().prefill(to_dev(q, wl.dtype), eng.k_cache, eng.v_cache,
                        torch.from_numpy(tables).cuda(), torch.from_numpy(cu_q).cuda(),
                        torch.from_numpy(ctx).cuda(), wl.scale, int(np.diff(cu_q).max()))
    torch.cuda.synchronize()
    compare_outputs(out, ref, what=wl.name, cast_dtype=wl.dtype)
    return eng, tables, ctx, out


@pytest.mark.parametrize("dtype,D,bs", [("f16", 128, 16), ("bf16", 128, 8), ("f16", 64, 32),
                                        ("bf16", 64, 128)])
def test_prefill_chunks(dtype, D, bs):
    """Prefixes 0 .. ~1000 tokens with chunks of 1 .. 250 tokens: whole prompts,
    chunks after a cached prefix, partial 16-query tiles, a one-token chunk."""
    synth.cache_draws(False)
    wl, q, cu_q = synth.make_prefill(620 + bs + D, 3, D, dtype, bs, [0, 17, 300, 1000, 0, 64],
                                     [33, 1, 64, 250, 200, 16])
    _run(wl, q, cu_q)


def test_prefill_long_prefix_and_empty_chunk():
    """A 3000-token cached prefix with a 100-token chunk, next to a sequence with
    no new token (its rows are absent) and a 512-token prompt."""
    synth.cache_draws(False)
    wl, q, cu_q = synth.make_prefill(640, 4, 128, "bf16", 16, [3000, 50, 0], [100, 0, 512])
    _run(wl, q, cu_q)


@pytest.mark.parametrize("dtype,D", [("f16", 128), ("bf16", 64)])
def test_prefill_prefix_past_the_table_window(dtype, D):
    """Contexts of more than 1024 blocks (bs 8): the kernel's block-table window
    in LDS (1024 entries) moves along the context; chunk lengths that leave
    partial 16-query sets and one to three steps after the last full pass."""
    synth.cache_draws(False)
    wl, q, cu_q = synth.make_prefill(650 + D, 2, D, dtype, 8, [8500, 8200, 130],
                                     [70, 33, 5])
    _run(wl, q, cu_q)


@pytest.mark.parametrize("q_len", [1, 31, 32, 33, 95, 96, 97, 129, 256, 300])
def test_prefill_step_counts(q_len):
    """Whole prompts whose key ranges end on and around step (32-key) and
    tile (256-query) boundaries: every count of steps after the last pass of
    four, and tiles with partial sets."""
    synth.cache_draws(False)
    wl, q, cu_q = synth.make_prefill(660 + q_len, 2, 128, "f16", 16, [0, 7], [q_len, q_len])
    _run(wl, q, cu_q)


def test_prefill_last_row_matches_decode():
    """A chunk's last query is the decode of that position: pa_prefill's last rows
    agree with pa_decode on the same cache within the tolerance."""
    synth.cache_draws(False)
    wl, q, cu_q = synth.make_prefill(641, 4, 128, "f16", 16, [700, 20, 1500], [90, 7, 33])
    eng, tables, ctx, out = _run(wl, q, cu_q)
    last = cu_q[1:] - 1
    qd = to_dev(q[last], "f16")
    dec = _pk().decode(qd, eng.k_cache, eng.v_cache, torch.from_numpy(tables).cuda(),
                       torch.from_numpy(ctx).cuda(), wl.scale, int(ctx.max()))
    d = (dec.float() - out[torch.from_numpy(last.astype(np.int64)).cuda()].float()).abs().max()
    log(f"prefill last rows vs decode: max diff {float(d):.2e}")
    assert float(d) <= 4e-3


def test_prefill_rejects_fp32():
    q = torch.zeros(1, 1, 64, device="cuda")
    kc = torch.zeros(4, 1, 16, 64, device="cuda")
    tab = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    ctx = torch.ones(1, dtype=torch.int32, device="cuda")
    with pytest.raises(_pk().PAError) as e:
        _pk().prefill(q, kc, kc, tab, cu, ctx, 0.1, 1)
    assert e.value.status == -2
    torch.cuda.synchronize()
