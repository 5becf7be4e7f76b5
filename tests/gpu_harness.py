"""Test helpers: run a workload's op script through the library on the GPU and
compare with the oracle.  Test infrastructure only."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
import synth

TOL = 2e-3   # max |gpu - oracle| on attention outputs (fp32 accumulation, one final rounding)

# Bound of the final round-to-nearest-even cast of a value x to the output type:
# half an ulp, at most 2^-8 |x| for bfloat16 (8-bit significand) and 2^-11 |x|
# for float16.  The configs' outputs are averages over hundreds of N(0,1)
# tokens (|out| << 1), where 2e-3 alone holds; tests with a handful of tokens
# give |out| near 1, where the cast by itself can exceed 2e-3 in bfloat16, so
# those tests allow TOL + CAST_REL[dtype] * |oracle|.
CAST_REL = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def to_dev(arr, dtype_name, device="cuda"):
    return synth.to_torch(arr, dtype_name, device)


def bits(t):
    """Raw storage bits of a device/host tensor as a numpy array."""
    import torch
    view = {2: torch.int16, 4: torch.int32}[t.element_size()]
    return t.detach().contiguous().view(view).cpu().numpy()


def oracle_bits(a, dtype_name):
    if dtype_name == "bf16":
        return np.ascontiguousarray(a).view(np.int16)
    if dtype_name == "f16":
        return np.ascontiguousarray(a).view(np.int16)
    return np.ascontiguousarray(a).view(np.int32)


def run_gpu(wl, partition_tokens=0, fill_nan=True, sharing=True, ring=None, mapped=None):
    """Execute wl.ops with PagedKVEngine; returns dict with the engine and the step output.
    mapped: None = the engine's default staging, else force mapped device staging on
    (True; it must be available) or off (False)."""
    import torch
    from paged_kv_cache_write_amd.engine import PagedKVEngine
    tdt = torch_dtype(wl.dtype)
    eng = PagedKVEngine(wl.NB, wl.H, wl.D, wl.bs, tdt, wl.max_blocks_per_seq, wl.S,
                        free_order=wl.free_order, pad_block=wl.poison_block,
                        fill=float("nan") if fill_nan else 0.0,
                        partition_tokens=partition_tokens, ring=ring)
    eng.set_sharing(sharing)
    if mapped is not None:
        eng.set_mapped_staging(mapped)
    out = None
    for op in wl.ops:
        if op[0] == "add":
            _, seq, n = op
            k, v = wl.kv(seq, 0, n)
            eng.add_sequence(seq, to_dev(k, wl.dtype), to_dev(v, wl.dtype))
        elif op[0] == "fork":
            eng.fork(op[1], op[2])
        elif op[0] == "free":
            eng.free(op[1])
        elif op[0] == "select":
            eng.select(op[1], op[2])
        elif op[0] == "host_pool":
            eng.set_host_pool(op[1])
        elif op[0] == "swap_out":
            eng.swap_out(op[1])
        elif op[0] == "swap_in":
            eng.swap_in(op[1])
        elif op[0] == "extend":
            _, seq, n = op
            t = eng.bm.seq_len(seq)
            k, v = wl.kv(seq, t, t + n)
            eng.extend([seq] * n, to_dev(k, wl.dtype), to_dev(v, wl.dtype))
        else:
            seqs = np.array(op[1], dtype=np.int64)
            ks, vs = [], []
            for s in seqs:
                t = eng.bm.seq_len(int(s))
                k, v = wl.kv(int(s), t, t + 1)
                ks.append(k[0])
                vs.append(v[0])
            q = to_dev(wl.q, wl.dtype)
            out = eng.step(seqs, q, to_dev(np.stack(ks), wl.dtype), to_dev(np.stack(vs), wl.dtype),
                           wl.scale)
    torch.cuda.synchronize()
    return dict(engine=eng, out=out)


def compare_outputs(gpu_out, ref, seqs=None, tol=TOL, what="", cast_dtype=None):
    """Element-wise check of GPU out (torch) against the oracle's fp64 out:
    |gpu - ref| <= tol (+ CAST_REL[cast_dtype] * |ref| when cast_dtype is given)."""
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    rows = list(range(ref.shape[0])) if seqs is None else list(seqs)
    g, r = g[rows], ref[rows]
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = tol + (CAST_REL[cast_dtype] * np.abs(r) if cast_dtype else 0.0)
    worst = float(err.max()) if err.size else 0.0
    rel = float((err / np.maximum(np.abs(r), 1e-3)).max()) if err.size else 0.0
    log(f"{what}: max abs err {worst:.3e}, mean {float(err.mean()) if err.size else 0:.3e}, "
        f"max rel {rel:.3e} over {len(rows)} seqs")
    assert np.all(err <= bound), f"{what}: max abs err {worst} over the bound (tol {tol})"
    return worst



def same_storage(gpu_t, ora, dtype, what):
    g = bits(gpu_t)
    o = oracle_bits(ora, dtype)
    assert g.shape == o.shape, what
    eq = g == o
    if not eq.all():
        fl = {"f32": np.float32, "f16": np.float16, "bf16": None}[dtype]
        if fl is None:
            gn = ((g.view(np.uint16) & 0x7F80) == 0x7F80) & ((g.view(np.uint16) & 0x7F) != 0)
            on = ((o.view(np.uint16) & 0x7F80) == 0x7F80) & ((o.view(np.uint16) & 0x7F) != 0)
        else:
            gn, on = np.isnan(g.view(fl)), np.isnan(o.view(fl))
        bad = ~eq & ~(gn & on)
        assert not bad.any(), f"{what}: {int(bad.sum())} storage elements differ"


def check_workload(wl, seqs=None, partition_tokens=0, tol=TOL, compare_pools=True,
                   cast_bound=False, sharing=True, mapped=None):
    """Run wl through the engine and the oracle: step bookkeeping and pools bit-exact,
    outputs within tol.  Returns (gpu dict, oracle dict, max error)."""
    log(f"case {wl.name}: S={wl.S} H={wl.H} D={wl.D} {wl.dtype} bs={wl.bs} NB={wl.NB} "
        f"sum(ctx)={int(wl.ctx.sum())} partition_tokens={partition_tokens} mapped={mapped}")
    g = run_gpu(wl, partition_tokens=partition_tokens, sharing=sharing, mapped=mapped)
    log("  gpu done; running oracle")
    r = oracle.run_workload(wl, decode_seqs=seqs)
    eng = g["engine"]
    last = eng.last_step
    assert np.array_equal(last["ctx"], r["ctx"]), "context lengths"
    assert np.array_equal(last["slots"], r["step_slots"]), "step slot mapping"
    assert np.array_equal(last["cows"].reshape(-1, 2), r["step_cows"]), "step CoW pairs"
    step = np.array([op for op in wl.ops if op[0] == "step"][-1][1], dtype=np.int64)
    tables, _ = eng.bm.block_tables(step, wl.max_blocks_per_seq, wl.poison_block)
    assert np.array_equal(tables, r["tables"]), "block tables"
    assert eng.bm.refcounts() == r["refcounts"].tolist(), "refcounts"
    if compare_pools:
        same_storage(eng.k_cache, r["k_cache"], wl.dtype, "k_cache")
        same_storage(eng.v_cache, r["v_cache"], wl.dtype, "v_cache")
        log("  pools bit-exact")
    err = compare_outputs(g["out"], r["out"], seqs=seqs, tol=tol, what=wl.name,
                          cast_dtype=wl.dtype if cast_bound else None)
    return g, r, err


def contiguous_kv(wl, ctx, layout):
    """The logical K/V of every sequence as drawn, in a contiguous [S, L, H, D] or
    [S, H, L, D] array (rows past a context are NaN)."""
    L = int(max(ctx.max(), 1))
    dt = synth.DTYPES[wl.dtype][0]
    nan = 0x7FC0 if wl.dtype == "bf16" else np.nan
    k = np.full((wl.S, L, wl.H, wl.D), nan, dtype=dt)
    v = k.copy()
    for s in range(wl.S):
        ks, vs = wl.kv(s, 0, int(ctx[s]))
        k[s, :int(ctx[s])] = ks
        v[s, :int(ctx[s])] = vs
    if layout == "SHLD":
        k, v = np.ascontiguousarray(k.transpose(0, 2, 1, 3)), np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    return k, v
