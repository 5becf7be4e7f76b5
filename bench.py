"""Benchmark: one decode engine step of the LLaMA-13B layer at batch 30 on one MI355X.

A step is one pass of the whole hot path for every sequence of the batch:
host slot assignment (C++ block manager), block tables shipped to the GPU,
copy-on-write copies, the slot-mapped cache write of the new tokens' K/V, and
PagedAttention decode (partition kernel + log-sum-exp reduce).  Inputs are
synthetic (seeded N(0,1) values, seeded context lengths and block placement)
and already resident in HBM when timing starts; each step appends one token
per sequence, so contexts grow by one per step.

Prints ONE JSON line.  Extra diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "pa_decode effective KV GB/s and % of MI355X HBM peak; decode seq-steps/s"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(ctx, H, D, elem, bs):
    """Algorithmic bytes of one decode over contexts ``ctx``: K and V of every
    context token (shared blocks counted once per sequence), q, out, the table
    entries read and the context lengths."""
    ctx = np.asarray(ctx, dtype=np.int64)
    S = ctx.size
    kv = int(ctx.sum()) * H * D * 2 * elem
    return kv + 2 * S * H * D * elem + int((-(-ctx // bs)).sum()) * 4 + 4 * S, kv


def unique_kv_bytes(tables, ctx, H, D, elem, bs):
    """K+V bytes of the distinct physical blocks a decode reads: a block that
    several sequences share counts once, with the most tokens any of them uses."""
    used = {}
    for row, c in zip(tables, np.asarray(ctx, dtype=np.int64)):
        nb = -(-int(c) // bs)
        for j in range(nb):
            n = min(bs, int(c) - j * bs)
            b = int(row[j])
            if used.get(b, 0) < n:
                used[b] = n
    return sum(used.values()) * H * D * 2 * elem


def step_bytes(ctx, H, D, elem, bs, ncow):
    """Whole step: decode + cache write (read k, v; write both rows) + slots + CoW copies."""
    S = len(ctx)
    dec, _ = decode_bytes(ctx, H, D, elem, bs)
    return dec + 4 * S * H * D * elem + 8 * S + ncow * 2 * 2 * H * bs * D * elem


def build_state(wl, dtype, partition_tokens=0, extra_blocks=64):
    """Run the workload's cache-building ops (prefill, forks, extends) on the GPU.
    Returns the engine and the step's sequence list (None without a step)."""
    import torch
    from paged_kv_cache_write_amd.engine import PagedKVEngine
    from synth import to_torch as to_dev
    step_seqs = None
    for op in wl.ops:
        if op[0] == "step":
            step_seqs = np.array(op[1], dtype=np.int64)
    n_seqs = len(step_seqs) if step_seqs is not None else int(wl.S)
    # growth blocks for the timed steps go after the workload's pool, so the
    # workload's own placement is unchanged
    NB = wl.NB + n_seqs * extra_blocks
    free_order = np.concatenate([wl.free_order, np.arange(wl.NB, NB, dtype=np.int32)])
    eng = PagedKVEngine(NB, wl.H, wl.D, wl.bs, dtype, wl.max_blocks_per_seq + extra_blocks,
                        n_seqs, free_order=free_order, pad_block=wl.poison_block,
                        fill=0.0, partition_tokens=partition_tokens)
    for op in wl.ops:
        if op[0] == "add":
            k, v = wl.kv(op[1], 0, op[2])
            eng.add_sequence(op[1], to_dev(k, wl.dtype), to_dev(v, wl.dtype))
        elif op[0] == "fork":
            eng.fork(op[1], op[2])
        elif op[0] == "extend":
            t = eng.bm.seq_len(op[1])
            k, v = wl.kv(op[1], t, t + op[2])
            eng.extend([op[1]] * op[2], to_dev(k, wl.dtype), to_dev(v, wl.dtype))
    torch.cuda.synchronize()
    return eng, step_seqs


_ORACLE_STATE = {}


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _oracle_share(seqs):
    """One worker's share of an oracle step: the step's cache write (into the
    worker's own copy of the pools) and the decode of its sequences."""
    import oracle
    st = _ORACLE_STATE
    oracle.oracle_cache_write(st["new_k"], st["new_v"], st["slots"], st["kc"], st["vc"])
    oracle.oracle_decode(st["q"], st["kc"], st["vc"], st["tables"], st["ctx"], st["scale"],
                         st["dtype"], seqs=list(seqs))
    return len(seqs)


def cpu_baseline(wl, max_seconds=20.0, max_workers=16):
    """The oracle (float64 NumPy, as it stands) on one step of the same workload
    on the host's cores: one forked worker process per core of this process's
    affinity set (at most ``max_workers``), one BLAS thread each; every worker
    takes a contiguous slice of the sequences (slices of about equal context
    sums) and makes the step's cache write in its own copy of the pools.  The
    step is repeated for about 10 s of wall clock (half of ``max_seconds`` when
    that is smaller).  Call it before this process touches the GPU: the workers
    are forked from it."""
    import multiprocessing as mp
    import oracle
    r = oracle.run_workload(wl, decode=False)
    ctx = np.asarray(r["ctx"], dtype=np.int64)
    S = ctx.size
    new_k = np.stack([wl.kv(int(s), int(c) - 1, int(c))[0][0] for s, c in enumerate(ctx)])
    new_v = np.stack([wl.kv(int(s), int(c) - 1, int(c))[1][0] for s, c in enumerate(ctx)])
    _ORACLE_STATE.update(new_k=new_k, new_v=new_v, slots=r["step_slots"], kc=r["k_cache"],
                         vc=r["v_cache"], q=wl.q, tables=r["tables"], ctx=ctx, scale=wl.scale,
                         dtype=wl.dtype)
    cores = max(1, min(len(os.sched_getaffinity(0)), max_workers, S))
    cum = np.cumsum(ctx)
    cuts = [0] + [int(np.searchsorted(cum, cum[-1] * k / cores)) + 1 for k in range(1, cores)] + [S]
    cuts = sorted(set(min(max(c, 0), S) for c in cuts))
    shares = [list(range(a, b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    reps, t_total = 0, 0.0
    min_seconds = min(10.0, max_seconds / 2)
    with mp.get_context("fork").Pool(len(shares), initializer=_one_blas_thread) as pool:
        pool.map(_oracle_share, [[0]] * len(shares))    # fork and first touch, untimed
        while reps == 0 or (t_total < min_seconds and reps < 10000 and
                            t_total * (reps + 1) / reps <= max_seconds):
            t0 = time.perf_counter()
            done = sum(pool.map(_oracle_share, shares, chunksize=1))
            t_total += time.perf_counter() - t0
            reps += 1
            assert done == S
    _ORACLE_STATE.clear()
    per = t_total / reps
    b = step_bytes(ctx, wl.H, wl.D, wl.elem_bytes, wl.bs, 0)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(b / per / 1e9, 4), "unit": "GB/s", "cores": len(shares),
            "kind": "oracle",
            "sample": f"one full step of {wl.name} (cache write of {S} tokens + decode of "
                      f"{S} seqs x {wl.H} heads, sum(ctx)={int(ctx.sum())}), {reps} rep(s), "
                      f"{per:.3f} s each, float64 NumPy, {len(shares)} forked worker processes "
                      f"(one BLAS thread each, contiguous slices of the sequences), {model}",
            "seconds_per_step": round(per, 4)}


def load_traffic(kernel_tag):
    """The committed rocprofv3 traffic record of a kernel (HBM read + write bytes
    per launch and that launch's algorithmic bytes), if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.json")
    if not os.path.exists(path):
        return None
    import hashlib
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec.get("sources", []):
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec.get("source_sha256"):
        return None
    return rec


def contiguous_compare(eng, seqs, q, wl, torch, pk, per_call):
    """Paged decode vs the same decode over the same K/V in contiguous layouts,
    [S, L, H, D] (token-major) and [S, H, L, D] (head-major): same contexts,
    same work list, 20 back-to-back calls each.  The contiguous copies are
    gathered from the pool with torch indexing (set-up, outside the timing)."""
    tables, ctx = eng.bm.block_tables(seqs, eng.maxB, wl.poison_block)
    dev = q.device
    S, bs = len(seqs), wl.bs
    nb = int(-(-int(ctx.max()) // bs))
    tab = torch.from_numpy(tables[:, :nb].astype(np.int64)).to(dev)
    L = nb * bs
    code = pk.DTYPE_CODES()[q.dtype]
    # the engine's automatic work list for these contexts, used by both launches
    items, pt2, mx = pk.decode_schedule(ctx, wl.H, wl.D, bs, code, 0)
    ptc = pt2
    di = dic = torch.from_numpy(items).to(dev)
    dt_, dc = torch.from_numpy(tables).to(dev), torch.from_numpy(ctx).to(dev)
    ws = torch.zeros(max(pk.decode_workspace_size(S, wl.H, wl.D, bs, mx, code, pt2),
                         pk.decode_workspace_size(S, wl.H, wl.D, 16, mx, code, ptc), 16),
                     dtype=torch.uint8, device=dev)
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    paged = lambda: pk.decode_scheduled(q, eng.k_cache, eng.v_cache, dt_, dc, wl.scale, mx, di,
                                        pt2, out=o1, workspace=ws)
    paged()
    tp = per_call(paged)
    kv = decode_bytes(ctx, wl.H, wl.D, wl.elem_bytes, bs)[0]
    res = {"partition_tokens": int(ptc), "paged_decode_us": round(tp * 1e6, 2),
           "paged_gbps": round(kv / tp / 1e9, 1),
           "timing": "20 back-to-back calls between one pair of events, each"}
    for layout, perm in (("SLHD", (0, 1, 3, 2, 4)), ("SHLD", (0, 2, 1, 3, 4))):
        def gather(cache):              # [NB, H, bs, D] -> [S, nb, H, bs, D] -> layout
            g = cache[tab].permute(*perm)
            shape = (S, L, wl.H, wl.D) if layout == "SLHD" else (S, wl.H, L, wl.D)
            return g.reshape(shape).contiguous()
        kc, vc = gather(eng.k_cache), gather(eng.v_cache)
        contig = lambda: pk.decode_contiguous(q, kc, vc, dc, wl.scale, mx, layout=layout,
                                              out=o2, workspace=ws, partition_tokens=ptc,
                                              items=dic)
        contig()
        tc = per_call(contig)
        res[layout] = {"decode_us": round(tc * 1e6, 2), "gbps": round(kv / tc / 1e9, 1),
                       "paged_time_over_contiguous": round(tp / tc, 4)}
        del kc, vc
    return res


MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix cores, published


def prefill_measure(torch, pk, per_call, dtype, seqs=8, prompt=1024, H=40, D=128, bs=16):
    """Paged prefill attention of `seqs` whole prompts of `prompt` tokens: causal
    flops 4*D*H per (query, key <= query), 20 back-to-back calls."""
    import synth
    wl, qn, cu_q = synth.make_prefill(901, H, D, dtype, bs, [0] * seqs, [prompt] * seqs)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    eng, _ = build_state(wl, tdt, 0, extra_blocks=1)
    tables, ctx = eng.bm.block_tables(np.arange(seqs), eng.maxB, wl.poison_block)
    from synth import to_torch as to_dev
    q = to_dev(qn, dtype)
    dt_, dc = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    cu = torch.from_numpy(cu_q).cuda()
    out = torch.empty_like(q)
    run = lambda: pk.prefill(q, eng.k_cache, eng.v_cache, dt_, cu, dc, wl.scale, prompt, out=out)
    # warm-up: ~60 calls (~10 ms): the first few dozen calls after an idle
    # spell run up to ~15% slower (the clocks ramp up under the load)
    for _ in range(60):
        run()
    t = per_call(run)
    pairs = seqs * prompt * (prompt + 1) // 2
    flops = 4.0 * D * H * pairs
    return {"workload": f"{seqs} prompts x {prompt} tokens, {H} heads, head_dim {D}, {dtype}, "
                        f"bs {bs}", "us": round(t * 1e6, 2),
            "tflops": round(flops / t / 1e12, 2), "peak_tflops": MFMA_PEAK_TFLOPS,
            "frac": round(flops / t / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "flops_counted": "4*D*H per causal (query, key) pair",
            "timing": "20 back-to-back calls between one pair of events, after 60 untimed calls"}


def pattern_read(eng, seqs, wl, torch, pk, n=20, reps=5):
    """pa_tile_read over the K and V tiles that the last step's decode reads:
    one unit per (work item, head) in the decode's order (group items first,
    through their first member's table), no arithmetic.  ``n`` back-to-back
    launches between one pair of events, median of ``reps``.  Returns
    (GB/s, bytes per launch, units)."""
    tables, ctx = eng.bm.block_tables(seqs, eng.maxB, wl.poison_block)
    code = pk.DTYPE_CODES()[eng.k_cache.dtype]
    sch = pk.decode_schedule_shared(ctx, tables, wl.H, wl.D, wl.bs, code, eng.partition_tokens)
    H, bs = wl.H, wl.bs
    lists = []

    def add(s, t0, ntok):
        blocks = tables[s, t0 // bs:(t0 + ntok - 1) // bs + 1].astype(np.int64)
        for h in range(H):
            lists.append(blocks * H + h)
    for moff, _cnt, _part, t0, ntok in sch["groups"]:
        if ntok > 0:
            add(int(sch["members"][moff][0]), int(t0), int(ntok))
    for s, _part, t0, ntok, _np in sch["items"]:
        if ntok > 0:
            add(int(s), int(t0), int(ntok))
    offsets = np.zeros(len(lists) + 1, np.int32)
    offsets[1:] = np.cumsum([len(x) for x in lists])
    ids = np.concatenate(lists).astype(np.int32)
    dev = eng.k_cache.device
    od, idd = torch.from_numpy(offsets).to(dev), torch.from_numpy(ids).to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    tile = bs * wl.D * eng.k_cache.element_size()
    run = lambda: pk.tile_read(eng.k_cache, eng.v_cache, tile, od, idd, sink)
    run()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            run()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3 / n)
    nbytes = 2 * int(ids.size) * tile
    return nbytes / float(np.median(ts)) / 1e9, nbytes, len(lists)


class FenceFreeEvents:
    """HIP timing events created with hipEventDisableSystemFence: recording one
    does not write back and invalidate the caches (a default event's system-scope
    release does, and the decode after it then starts cold), so the decode is
    timed as it runs in the marker-free loop.  The calls go to the HIP runtime
    torch loaded, found by its path in /proc/self/maps (one runtime per process)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.c = ctypes
        path = next(line.split()[-1] for line in open("/proc/self/maps")
                    if "libamdhip64.so" in line)
        hip = ctypes.CDLL(path)
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip = hip

    def create(self):
        ev = self.c.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.c.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return ev.value

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.c.c_float()
        if self.hip.hipEventElapsedTime(self.c.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def decode_alone(eng, seqs, q, out_step, wl, torch, pk, hev, n):
    """The decode launch of the engine's last step on its own: the same inputs,
    schedule and workspace, launched ``n`` times back to back through
    pa_decode_scheduled_shared between one pair of fence-free events on the
    launch stream.  Events around every launch each cost the launch a few
    microseconds of gap and a partly cold L2, so one pair over the run gives
    the kernel's own duration as it runs inside the marker-free steps.
    Returns (seconds per launch, context lengths, tables, output == the step's)."""
    tables, ctx = eng.bm.block_tables(seqs, eng.maxB, wl.poison_block)
    dev = q.device
    S = len(seqs)
    code = pk.DTYPE_CODES()[q.dtype]
    sch = pk.decode_schedule_shared(ctx, tables, wl.H, wl.D, wl.bs, code, eng.partition_tokens)
    ws_bytes = eng.workspace.numel()
    if sch["workspace_bytes"] > ws_bytes:
        raise RuntimeError("the engine workspace does not cover the decode")
    dev_arr = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if a.size else None
    dt_, dc = dev_arr(tables), dev_arr(ctx)
    di, dg, dm = dev_arr(sch["items"]), dev_arr(sch["groups"]), dev_arr(sch["members"])
    ptr = lambda t: t.data_ptr() if t is not None else None
    o = torch.empty_like(q)
    st = torch.cuda.current_stream(dev).cuda_stream
    fn = pk.lib().pa_decode_scheduled_shared
    argv = (q.data_ptr(), eng.k_cache.data_ptr(), eng.v_cache.data_ptr(), dt_.data_ptr(),
            int(tables.shape[1]), dc.data_ptr(), S, wl.H, wl.D, wl.bs, eng.NB, float(wl.scale),
            int(sch["max_context_len"]), code, o.data_ptr(), eng.workspace.data_ptr(), ws_bytes,
            int(sch["partition_tokens"]), st, ptr(di), int(sch["items"].shape[0]), ptr(dg),
            int(sch["groups"].shape[0]), ptr(dm))

    def launch():
        rc = fn(*argv)
        if rc != 0:
            raise pk.PAError(rc, "pa_decode_scheduled_shared")
    launch()
    torch.cuda.synchronize()
    same = bool(torch.equal(o, out_step))
    a, b = hev.create(), hev.create()
    hev.record(a, st)
    for _ in range(n):
        launch()
    hev.record(b, st)
    torch.cuda.synchronize()
    sec = hev.elapsed_ms(a, b) * 1e-3 / n
    hev.destroy(a)
    hev.destroy(b)
    return sec, ctx, tables, same


def block_manager_stats(eng, seqs, tables, wl):
    """Memory figures of the pool after the timed steps: useful KV fraction
    sum(ctx) / (sum(ceil(ctx/bs)) * bs) (the waste is only each sequence's
    last block), physical blocks in use, and the saving of shared blocks
    1 - distinct / sum(ceil(ctx/bs))."""
    lens = np.array([eng.bm.seq_len(int(x)) for x in seqs], dtype=np.int64)
    nblk = -(-lens // wl.bs)
    ids = np.concatenate([tables[i, :n] for i, n in enumerate(nblk)]) if len(nblk) else []
    distinct = int(np.unique(ids).size)
    logical = int(nblk.sum())
    return {"useful_kv_fraction": round(float(lens.sum()) / max(logical * wl.bs, 1), 4),
            "blocks_in_use": distinct, "pool_blocks": int(eng.NB),
            "logical_blocks": logical,
            "sharing_saving": round(1.0 - distinct / max(logical, 1), 4)}


def per_call_fn(torch):
    def per_call(fn, n=20):
        """Seconds per call of n back-to-back calls between one pair of events
        (markers around every call would cost more than these short kernels)."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / n
    return per_call


def device_per_call_fn(torch, pk, dev, lead_mib=1024, lead_reads=3):
    """Like per_call, for calls shorter than their host issue (a few us of
    binding and launch each): plain streaming reads of a lead buffer are queued
    first, so all n calls are on the stream before the GPU reaches the first
    event and run back to back.  Returns (seconds per call, queued) where
    queued says the lead reads were still running when the last call had been
    issued (else the figure is bounded by the host, as per_call's)."""
    lead = torch.empty(lead_mib << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def per_call(fn, n=20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        for _ in range(lead_reads):
            pk.stream_read(lead, sink)
        a.record()
        for _ in range(n):
            fn()
        queued = not a.query()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / n, queued
    return per_call


def measure_workload(wl, args, torch, pk, hev, steps, warmup, cold_steps, partition_tokens=0):
    """One workload on the GPU: build its pool, ``warmup`` engine steps, loop 1
    (``steps`` marker-free engine steps, wall clock), loop 2 (``steps`` steps with
    the decode's own start/end events), the decode alone (the last step's decode,
    ``steps`` back-to-back launches) and ``cold_steps`` steps after a cache
    flush.  Returns (record, state) where state keeps what the headline's extra
    measurements reuse."""
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.dtype]
    pt_req = partition_tokens or wl.partition_tokens
    grow = warmup + 2 * steps + cold_steps
    eng, seqs = build_state(wl, tdt, pt_req, extra_blocks=-(-grow // wl.bs) + 1)
    from synth import to_torch as to_dev
    S = seqs.size
    q = to_dev(wl.q, wl.dtype)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    k_new = torch.randn(S, wl.H, wl.D, device=dev, generator=gen).to(tdt)
    v_new = torch.randn(S, wl.H, wl.D, device=dev, generator=gen).to(tdt)
    out = torch.empty_like(q)

    for _ in range(warmup):
        eng.step(seqs, q, k_new, v_new, wl.scale, out=out)
    torch.cuda.synchronize()

    # Loop 1, the steps themselves, right after the warmup: nothing but the
    # steps is enqueued (event markers around every decode would add their own
    # gaps to each step).
    ncows, pts, ngroups = 0, set(), set()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        eng.step(seqs, q, k_new, v_new, wl.scale, out=out)
        ncows += eng.last_info.num_cow
        pts.add(eng.last_info.partition_tokens)
        ngroups.add(eng.last_info.num_group_items)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # Loop 2, the decode launch of each step between HIP events recorded by
    # its own dispatch; the same steps, continued.
    evs = [(hev.create(), hev.create()) for _ in range(steps)]
    stream_handle = torch.cuda.current_stream().cuda_stream
    for a, b in evs:                      # first records outside the timed loop
        hev.record(a, stream_handle)
        hev.record(b, stream_handle)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(steps):
        eng.set_decode_events(*evs[i])
        eng.step(seqs, q, k_new, v_new, wl.scale, out=out)
        pts.add(eng.last_info.partition_tokens)
        ngroups.add(eng.last_info.num_group_items)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    eng.set_decode_events(None, None)

    # The decode kernel alone (the roofline figure): the last step's decode,
    # launched back to back between one pair of events, at that step's
    # contexts (the workload's step contexts + warmup + 2 * steps - 1).
    kern_s, ctx_a, tab_a, same_out = decode_alone(eng, seqs, q, out, wl, torch, pk, hev, steps)
    if not same_out:
        eprint(f"warning: {wl.name}: the back-to-back decode output differs from the step's")

    # each step appends one token to every sequence: the contexts of step i of
    # loop 1 are the workload's step contexts + warmup + i, loop 2 continues
    ctxs = [wl.ctx + warmup + i for i in range(steps)]
    ctxs2 = [wl.ctx + warmup + steps + i for i in range(steps)]
    elem = wl.elem_bytes
    total_step_bytes = sum(step_bytes(c, wl.H, wl.D, elem, wl.bs, 0) for c in ctxs) + \
        ncows * 2 * 2 * wl.H * wl.bs * wl.D * elem
    dec_bytes = [decode_bytes(c, wl.H, wl.D, elem, wl.bs)[0] for c in ctxs2]
    # distinct blocks: the steps only append, so step i's tables are a prefix
    # of the final ones
    tables, _ = eng.bm.block_tables(seqs, eng.maxB, wl.poison_block)
    uniq_bytes = [b - decode_bytes(c, wl.H, wl.D, elem, wl.bs)[1] +
                  unique_kv_bytes(tables, c, wl.H, wl.D, elem, wl.bs)
                  for b, c in zip(dec_bytes, ctxs2)]
    bm_stats = block_manager_stats(eng, seqs, tables, wl)
    elapsed = t1 - t0
    step_ms = np.array([hev.elapsed_ms(a, b) for a, b in evs])
    for a, b in evs:
        hev.destroy(a)
        hev.destroy(b)
    step_s = float(step_ms.mean()) / 1e3

    dec_a, kv_a = decode_bytes(ctx_a, wl.H, wl.D, elem, wl.bs)
    uniq_a = dec_a - kv_a + unique_kv_bytes(tab_a, ctx_a, wl.H, wl.D, elem, wl.bs)
    effective = dec_a / kern_s / 1e9
    achieved = uniq_a / kern_s / 1e9
    shared = max(ngroups) > 0
    rec = {
        "workload": wl.name, "placement": wl.placement if hasattr(wl, "placement") else None,
        "seqs": int(S), "heads": wl.H, "head_dim": wl.D, "block_size": wl.bs,
        "storage_dtype": wl.dtype, "num_blocks": wl.NB,
        "partition_tokens": sorted(pts), "decode_group_items": sorted(ngroups),
        "step_us": round(elapsed / steps * 1e6, 2),
        "step_gbps": round(total_step_bytes / elapsed / 1e9, 2),
        "seq_steps_per_s": round(S * steps / elapsed, 1),
        "decode_us": round(kern_s * 1e6, 2),
        "decode_ctx_sum": int(ctx_a.sum()),
        "decode_gbps": round(achieved, 2),
        "decode_frac": round(achieved / HBM_PEAK_GBS, 4),
        "decode_effective_gbps": round(effective, 2),
        "decode_seq_steps_per_s": round(S / kern_s, 1),
        "decode_bytes_counted": "distinct blocks once (shared prefixes once)",
        "decode_algorithmic_bytes": int(uniq_a),
        "decode_output_same_as_step": bool(same_out),
        "decode_us_in_steps": round(step_s * 1e6, 2),
        "decode_us_in_steps_p10_p90": [round(float(np.percentile(step_ms, 10)) * 1e3, 2),
                                       round(float(np.percentile(step_ms, 90)) * 1e3, 2)],
        "decode_in_steps_distinct_gbps": round(float(np.mean(uniq_bytes)) / step_s / 1e9, 2),
        "ms_per_step_with_decode_events": round((t3 - t2) / steps * 1e3, 4),
        "kernel": (("decode_group_kernel + decode_wave_kernel" if wl.dtype == "f32"
                    else "decode_shared_kernel") + " (pa_decode_scheduled_shared)" if shared
                   else "decode_wave_kernel (pa_decode_scheduled)"),
        "block_manager": bm_stats,
    }
    # cold decode: the same steps after a 1 GiB write (the 256 MB MALL and the
    # L2s hold no K/V when the decode starts); decode events only
    if cold_steps > 0:
        # write 1 GiB (the protocol's flush), then read another 1 GiB so the
        # dirty lines are written back before, not during, the timed decode
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        clean = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(cold_steps)]
        for a, b in cev:
            a.record()
            b.record()
        torch.cuda.synchronize()
        for i in range(cold_steps):
            scratch.fill_(i & 0xFF)
            clean.sum()
            eng.set_decode_events(*cev[i])
            eng.step(seqs, q, k_new, v_new, wl.scale, out=out)
        torch.cuda.synchronize()
        eng.set_decode_events(None, None)
        ctables, _ = eng.bm.block_tables(seqs, eng.maxB, wl.poison_block)
        cms = np.array([a.elapsed_time(b) for a, b in cev]) * 1e3
        c0 = warmup + 2 * steps
        cbytes = [decode_bytes(wl.ctx + c0 + i, wl.H, wl.D, elem, wl.bs)[0]
                  for i in range(cold_steps)]
        cuniq = [b - decode_bytes(wl.ctx + c0 + i, wl.H, wl.D, elem, wl.bs)[1] +
                 unique_kv_bytes(ctables, wl.ctx + c0 + i, wl.H, wl.D, elem, wl.bs)
                 for i, b in enumerate(cbytes)]
        med = float(np.median(cms))
        cg = float(np.mean(cuniq)) / (med * 1e-6) / 1e9
        rec["decode_cold"] = {"steps": cold_steps,
                              "flush": "1 GiB written, then 1 GiB of another buffer read, "
                                       "before each step",
                              "decode_us_median": round(med, 2),
                              "decode_us_p10_p90": [round(float(np.percentile(cms, 10)), 2),
                                                    round(float(np.percentile(cms, 90)), 2)],
                              "decode_gbps": round(cg, 2),
                              "decode_frac": round(cg / HBM_PEAK_GBS, 4)}
        del scratch, clean
    else:
        rec["decode_cold"] = None
    state = dict(eng=eng, seqs=seqs, q=q, k_new=k_new, v_new=v_new, tables=tables, S=S,
                 total_step_bytes=total_step_bytes, elapsed=elapsed, ctxs=ctxs,
                 achieved=achieved, uniq_a=uniq_a, kern_s=kern_s, shared=shared)
    return rec, state


# the other workloads of the same JSON line (compact records): (config, block
# size, placement, also time the decode over contiguous copies of the K/V)
OTHER_WORKLOADS = [(1, None, "random", False), (3, None, "random", True),
                   (4, None, "random", False), (2, None, "identity", False)] + \
                  [(5, b, "random", False) for b in (8, 16, 32, 64, 128)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--bs", type=int, default=None, help="block size (config 5)")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--placement", choices=["random", "identity"], default="random",
                    help="block placement: seeded random (the workloads) or in id order")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps, each after writing 1 GiB of scratch (MALL/L2 flushed)")
    ap.add_argument("--read-gib", type=int, default=4,
                    help="GiB for the plain streaming-read reference (0 = skip)")
    ap.add_argument("--contiguous", action="store_true",
                    help="also time the decode over the same K/V gathered into a contiguous "
                         "[S, L, H, D] layout (pa_decode_contiguous) next to the paged decode")
    ap.add_argument("--prefill", action="store_true",
                    help="also time the paged prefill attention (8 prompts of 1024 tokens at "
                         "the 13B-layer shape) against the matrix cores' peak (the default run "
                         "does, unless --headline-only)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run 3 plain elementwise copies (neg) of this many MiB: a "
                         "known-size reference for the HBM traffic counters")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the compact records of the other workloads")
    ap.add_argument("--other-steps", type=int, default=20,
                    help="timed steps (and back-to-back decodes) per other workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              "cross-GPU component to measure", file=sys.stderr)
        sys.exit(2)

    import synth
    t_setup = time.perf_counter()
    wl = synth.make_workload(args.config, bs=args.bs, placement=args.placement)
    eprint(f"setup {time.perf_counter() - t_setup:.1f} s: {wl.name}, S={wl.S}, "
           f"sum(ctx)={int(wl.ctx.sum())}")
    # The oracle's CPU baseline runs first, before this process touches the
    # GPU: its worker processes are forked from this one.
    cpu = None
    if not args.no_cpu_baseline:
        t = time.perf_counter()
        cpu = cpu_baseline(wl, args.cpu_seconds)
        eprint(f"cpu baseline {time.perf_counter() - t:.1f} s on {cpu['cores']} cores")

    import torch
    import paged_kv_cache_write_amd as pk
    pk.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hev = FenceFreeEvents()
    per_call = per_call_fn(torch)

    if args.copy_calibration_mib:
        # a plain elementwise kernel that reads and writes exactly nbytes each
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 2, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        eprint(f"copy calibration: 3 elementwise kernels reading and writing {nbytes} bytes")

    rec, st = measure_workload(wl, args, torch, pk, hev, args.steps, args.warmup,
                               args.cold_steps, args.partition_tokens)
    S, eng, tables = st["S"], st["eng"], st["tables"]
    value = st["total_step_bytes"] / st["elapsed"] / 1e9
    # HBM traffic per launch: the counters' ratio of (read + write) to algorithmic
    # bytes, measured on a launch of the same workload and kernel source (the
    # profile run's contexts are shorter), applied to this launch's bytes
    trec = load_traffic("decode_" + wl.name)
    traffic, traffic_ratio = None, None
    if trec and trec.get("algorithmic_bytes_per_launch"):
        traffic_ratio = trec["traffic_bytes_per_launch"] / trec["algorithmic_bytes_per_launch"]
        traffic = round(traffic_ratio * int(st["uniq_a"]))
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(st["elapsed"] / args.steps * 1e3, 4),
        "ms_per_step_with_decode_events": rec["ms_per_step_with_decode_events"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "placement": args.placement, "seqs": int(S),
                   "heads": wl.H, "head_dim": wl.D,
                   "block_size": wl.bs, "num_blocks": wl.NB,
                   "ctx_sum_first_step": int(st["ctxs"][0].sum()),
                   "ctx_sum_last_step": int(st["ctxs"][-1].sum()),
                   "partition_tokens": rec["partition_tokens"]},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": rec["seq_steps_per_s"],
        "decode_seq_steps_per_s": rec["decode_seq_steps_per_s"],
        "decode_us": rec["decode_us"],
        "decode_timing": f"the last timed step's decode launched {args.steps} times back "
                         "to back between one pair of events on its stream (same inputs, "
                         "schedule and workspace as the step; output identical to the "
                         f"step's: {rec['decode_output_same_as_step']})",
        "decode_ctx_sum": rec["decode_ctx_sum"],
        "decode_us_in_steps": rec["decode_us_in_steps"],
        "decode_us_in_steps_p10_p90": rec["decode_us_in_steps_p10_p90"],
        "decode_in_steps_distinct_gbps": rec["decode_in_steps_distinct_gbps"],
        "decode_gbps": rec["decode_effective_gbps"],
        "decode_pct_hbm_peak": round(100 * rec["decode_effective_gbps"] / HBM_PEAK_GBS, 2),
        "decode_group_items": rec["decode_group_items"],
        "roofline": {"bound": "hbm", "achieved": round(st["achieved"], 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(st["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": rec["kernel"],
                     "algorithmic_bytes_per_launch": int(st["uniq_a"]),
                     "traffic_over_algorithmic": (round(traffic_ratio, 4)
                                                  if traffic_ratio else None),
                     "traffic_source": (f"{trec['summary']}: {trec['traffic_bytes_per_launch']:.0f}"
                                        f" B per launch of {trec['algorithmic_bytes_per_launch']}"
                                        " algorithmic B (FETCH_SIZE and WRITE_SIZE, scaled by a"
                                        " copy kernel of known size)") if trec else None,
                     "bytes_counted": "distinct blocks once (shared prefixes once)"},
        "decode_cold": rec["decode_cold"],
    }

    # achievable read: the library's plain streaming read over a large buffer
    if args.read_gib > 0:
        buf = torch.zeros(args.read_gib << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        pk.stream_read(buf, sink)
        rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(5)]
        for a, b in rev:
            a.record()
            pk.stream_read(buf, sink)
            b.record()
        torch.cuda.synchronize()
        best = min(a.elapsed_time(b) for a, b in rev) * 1e-3
        rgbps = buf.numel() / best / 1e9
        res["achievable_read"] = {"gbps": round(rgbps, 1), "bytes": buf.numel(),
                                  "kernel": "stream_read_kernel (pa_stream_read), best of 5"}
        res["roofline"]["frac_of_achievable_read"] = round(st["achieved"] / rgbps, 4)
        del buf

    # the decode's own access pattern read without arithmetic: the K and V
    # tiles of the last step's work list, gathered through the tables
    pgbps, pbytes, punits = pattern_read(eng, st["seqs"], wl, torch, pk)
    res["pattern_read"] = {"gbps": round(pgbps, 1), "bytes": pbytes, "units": punits,
                           "kernel": "tile_read_kernel (pa_tile_read): the K and V tiles of the "
                                     "last step's decode work list, one wave per (item, head) "
                                     "in the decode's order, no arithmetic; 20 back-to-back "
                                     "launches, median of 5"}
    res["roofline"]["frac_of_pattern_read"] = round(st["achieved"] / pgbps, 4)

    # secondary: the cache write and the copy-on-write copy on their own, both
    # shorter than their host issue: timed queued behind a lead read
    sec = {}
    dev_call = device_per_call_fn(torch, pk, dev)
    elem = wl.elem_bytes
    k_new, v_new = st["k_new"], st["v_new"]
    last = eng.last_step
    slots_d = torch.from_numpy(last["slots"]).to(dev)
    pk.cache_write(k_new, v_new, slots_d, eng.k_cache, eng.v_cache)
    wt, wq = dev_call(lambda: pk.cache_write(k_new, v_new, slots_d, eng.k_cache, eng.v_cache))
    sec["cache_write_us"] = round(wt * 1e6, 2)
    sec["cache_write_queued"] = wq
    sec["cache_write_gbps"] = round(4 * S * wl.H * wl.D * elem / wt / 1e9, 2)
    sec["cache_write_tokens"] = int(S)
    free = eng.bm.free_list()
    npairs = min(56, len(free))
    if npairs:
        # copies into free blocks, from blocks in use (the copy-on-write pattern)
        used = tables[:, 0]
        pairs = np.stack([np.resize(used, npairs), np.array(free[:npairs])], 1).astype(np.int32)
        pd = torch.from_numpy(pairs).to(dev)
        pk.copy_blocks(eng.k_cache, eng.v_cache, pd)
        ct, cq = dev_call(lambda: pk.copy_blocks(eng.k_cache, eng.v_cache, pd))
        sec["copy_blocks_us"] = round(ct * 1e6, 2)
        sec["copy_blocks_queued"] = cq
        sec["copy_blocks_gbps"] = round(npairs * 2 * 2 * wl.H * wl.bs * wl.D * elem / ct / 1e9, 2)
        sec["copy_pairs"] = int(npairs)
    # swapping (preemption): blocks to a pinned host pool and back over the host link
    nswap = 64
    hk = torch.empty((nswap,) + tuple(eng.k_cache.shape[1:]), dtype=eng.k_cache.dtype,
                     pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    used = np.resize(tables[:, 0], nswap).astype(np.int32)
    out_pairs = torch.from_numpy(np.stack([used, np.arange(nswap, dtype=np.int32)], 1)).to(dev)
    back = free[:nswap] if len(free) >= nswap else None
    pk.copy_blocks_between(eng.k_cache, eng.v_cache, hk, hv, out_pairs)
    so = per_call(lambda: pk.copy_blocks_between(eng.k_cache, eng.v_cache, hk, hv, out_pairs), n=5)
    blk = 2 * wl.H * wl.bs * wl.D * elem
    sec["swap_out_us"] = round(so * 1e6, 2)
    sec["swap_out_gbps"] = round(nswap * blk / so / 1e9, 2)
    if back is not None:
        in_pairs = torch.from_numpy(np.stack([np.arange(nswap, dtype=np.int32),
                                              np.array(back, dtype=np.int32)], 1)).to(dev)
        si = per_call(lambda: pk.copy_blocks_between(hk, hv, eng.k_cache, eng.v_cache, in_pairs),
                      n=5)
        sec["swap_in_us"] = round(si * 1e6, 2)
        sec["swap_in_gbps"] = round(nswap * blk / si / 1e9, 2)
    sec["swap_blocks"] = nswap
    res["secondary"] = sec
    del dev_call
    res["block_manager"] = rec["block_manager"]

    if args.contiguous or not args.headline_only:
        res["contiguous"] = contiguous_compare(eng, st["seqs"], st["q"], wl, torch, pk, per_call)
    if args.prefill or not args.headline_only:
        res["prefill"] = prefill_measure(torch, pk, per_call,
                                         "f16" if wl.dtype == "f32" else wl.dtype)
    del st, eng
    torch.cuda.empty_cache()

    if not args.headline_only:
        others = []
        for cfg, bs, placement, contig in OTHER_WORKLOADS:
            t = time.perf_counter()
            owl = synth.make_workload(cfg, bs=bs, placement=placement)
            orec, ost = measure_workload(owl, args, torch, pk, hev, args.other_steps, 5,
                                         5 if cfg != 1 else 0)
            orec["config"] = cfg
            orec["placement"] = placement
            if contig:
                orec["contiguous"] = contiguous_compare(ost["eng"], ost["seqs"], ost["q"], owl,
                                                        torch, pk, per_call)
            del orec["block_manager"]["pool_blocks"]
            others.append(orec)
            del ost
            torch.cuda.empty_cache()
            eprint(f"{owl.name} bs={owl.bs} {placement}: decode {orec['decode_us']} us "
                   f"({orec['decode_frac']:.3f}), step {orec['step_us']} us, "
                   f"{time.perf_counter() - t:.1f} s")
        res["workloads"] = others
    res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
