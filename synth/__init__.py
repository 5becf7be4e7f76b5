"""Seeded synthetic inputs for the paged KV-cache write + PagedAttention decode path.

This module is shared by the oracle side and the HIP side and holds none of the
method's arithmetic: it draws context lengths, block placements (the order of
the free list), and the query / key / value values, and it describes, as a
script of block-manager operations, how each workload's cache is built.  Each
side executes that script with its own block manager, its own cache write and
its own attention.

Randomness: ``numpy.random.default_rng(SeedSequence([cfg, stream, sub]))`` with
one stream per kind of draw (0 context lengths, 1 placement, 2 q, 3 history K,
4 history V, 5 step-token K/V, 6 tails, 7 fork offsets, 8 fork-tree shape) and ``sub`` naming the
sequence (or prompt group, or block size for placements), so that a sequence's
values do not depend on how many other sequences are drawn.  Values are drawn as
float32 N(0, 1) and rounded to the storage type with round-to-nearest-even.

The workloads follow the shapes that the pages use: the LLaMA-13B layer
(40 heads x head_dim 128 = d_model 5120, brentwoodlivery "5.3.18 LLM serving"
worked example; polomodov.tech "vLLM and PagedAttention" slide 5), a batch of 30
requests (slide 17), the 4096-token worked-example length, parallel sampling
with a shared prompt (comfyai.app "6.4 PagedAttention" 6.4.3; slide 13), and
block sizes around the 16-32 sweet spot (slide 19).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # optional: fast IEEE casts on the CPU
    import torch as _torch
except Exception:  # pragma: no cover
    _torch = None

__all__ = [
    "DTYPES", "Workload", "make_workload", "make_custom", "to_storage", "CONFIG_NAMES",
    "SWEEP_BLOCK_SIZES", "cache_draws", "to_torch", "make_fork_tree", "make_beam_search",
    "make_preemption", "make_prefill",
]

# storage dtype name -> (numpy storage dtype, bytes per element)
DTYPES = {"f32": (np.float32, 4), "f16": (np.float16, 2), "bf16": (np.uint16, 2)}

CONFIG_NAMES = {
    1: "tiny-fp32",
    2: "llama13b-layer-batch30",
    3: "long-context-8x4096",
    4: "shared-prefix-8x8",
    5: "high-batch-bs-sweep",
}
SWEEP_BLOCK_SIZES = (8, 16, 32, 64, 128)

_STREAM_CTX, _STREAM_PLACE, _STREAM_Q, _STREAM_K, _STREAM_V = 0, 1, 2, 3, 4
_STREAM_STEP, _STREAM_TAIL, _STREAM_FORK = 5, 6, 7
_STREAM_TREE = 8


def _rng(cfg: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg, stream, sub]))


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage type (round to nearest, ties to even).

    bf16 is returned as its raw uint16 bit pattern.  torch's CPU casts are used
    when available (they are IEEE round-to-nearest-even, like NumPy's, and
    much faster); the NumPy path gives the same bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if _torch is not None and x.size > 4096:
        t = _torch.from_numpy(x)
        if dtype == "f16":
            return t.to(_torch.float16).numpy()
        if dtype == "bf16":
            return t.to(_torch.bfloat16).view(_torch.int16).numpy().view(np.uint16)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        bits = x.view(np.uint32).astype(np.uint64)
        nan = np.isnan(x)
        rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
        rounded[nan] = 0x7FC0
        return rounded
    raise ValueError(dtype)


def to_torch(arr: np.ndarray, dtype: str, device="cuda"):
    """A storage-typed array as a torch tensor on ``device`` (bf16 from its bits)."""
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    if not _VALUES[0]:
        return np.zeros(shape, dtype=DTYPES[dtype][0])
    return to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


_VALUES = [True]


def _draw_many(cfg: int, stream: int, jobs, dtype: str):
    """Draw one array per (sub, shape) job, each from its own seed stream
    (cfg, stream, sub); threads only change the speed, never the values.
    Draws are cached per (cfg, stream, sub, shape, dtype) for the life of the
    process when ``cache_draws(True)`` is on (the block-size sweep reuses one
    set of logical K/V)."""
    if not _VALUES[0]:
        return [None] * len(jobs)

    def one(job):
        sub, shape = job
        return _normal(_rng(cfg, stream, sub), shape, dtype)
    def cached(job):
        key = (cfg, stream, job[0], tuple(job[1]), dtype)
        if _CACHE_ON[0] and key in _CACHE:
            return _CACHE[key]
        arr = one(job)
        if _CACHE_ON[0]:
            _CACHE[key] = arr
        return arr
    with ThreadPoolExecutor(max_workers=8) as ex:
        return list(ex.map(cached, jobs))


_CACHE: dict = {}
_CACHE_ON = [False]


def cache_draws(on: bool):
    """Keep drawn K/V arrays for reuse (on) or drop them (off)."""
    _CACHE_ON[0] = bool(on)
    if not on:
        _CACHE.clear()


@dataclass
class Workload:
    """One seeded workload: shapes, pool, free-list order, values and the op script.

    ``ops`` is executed in order by each side:
      ("add", seq, n)         new sequence whose first n tokens are written (prefill)
      ("fork", parent, child) child shares all of parent's blocks
      ("extend", seq, n)      append n tokens to seq, one at a time
      ("step", [seqs])        append one token to each listed seq, then decode them
      ("free", seq)           release seq's blocks (shared ones stay with their holders)
      ("select", [(parent, child)], [retired])
                              beam selection: each child forks its parent, then the
                              retired sequences are freed
      ("host_pool", n)        a host pool of n blocks for preempted requests
      ("swap_out", [seqs])    preempt a request (its sequences) to the host pool
      ("swap_in", [seqs])     bring it back
    The values of token t of sequence s are ``kv(s, t, t+1)``; the step token of
    each sequence is its last logical token.
    """
    cfg: int
    name: str
    H: int
    D: int
    dtype: str
    bs: int
    NB: int
    scale: float
    free_order: np.ndarray          # int32, the free list (front is popped first)
    poison_block: int               # a block id never handed out; tests fill it with NaN
    ctx: np.ndarray                 # int64 [S] context length after the step (incl. step token)
    q: np.ndarray                   # [S, H, D] storage dtype
    ops: list
    max_blocks_per_seq: int
    partition_tokens: int = 0       # 0 = let the launcher choose
    _segments: dict = field(default_factory=dict, repr=False)
    notes: str = ""

    @property
    def S(self) -> int:
        return int(self.ctx.shape[0])

    @property
    def elem_bytes(self) -> int:
        return DTYPES[self.dtype][1]

    def kv(self, seq: int, t0: int, t1: int):
        """Logical K and V rows [t0, t1) of sequence ``seq``: arrays [t1-t0, H, D]."""
        parts_k, parts_v = [], []
        for (s0, s1, k, v) in self._segments[seq]:
            a, b = max(t0, s0), min(t1, s1)
            if a < b:
                parts_k.append(k[a - s0:b - s0])
                parts_v.append(v[a - s0:b - s0])
        shape = (0, self.H, self.D)
        empty = np.empty(shape, dtype=DTYPES[self.dtype][0])
        k = np.concatenate(parts_k) if parts_k else empty
        v = np.concatenate(parts_v) if parts_v else empty
        assert k.shape[0] == t1 - t0, (seq, t0, t1, k.shape)
        return k, v

    def kv_bytes_effective(self) -> int:
        """K+V bytes a decode over all sequences reads (shared blocks once per sequence)."""
        return int(self.ctx.sum()) * self.H * self.D * 2 * self.elem_bytes


_IDENTITY = [False]


def _placement(cfg: int, NB: int, sub: int = 0):
    """(poison block, free-list order).  Seeded random placement, or with
    ``placement="identity"`` in make_workload the blocks in id order (each
    sequence's blocks contiguous and ascending), the poison block last."""
    if _IDENTITY[0]:
        return NB - 1, np.arange(NB - 1, dtype=np.int32)
    perm = _rng(cfg, _STREAM_PLACE, sub).permutation(NB).astype(np.int32)
    return int(perm[-1]), perm[:-1].copy()


def _simple(cfg, name, H, D, dtype, bs, NB, ctx, scale, part_tokens=0, seed_sub=0):
    """Independent sequences: prefill of ctx-1 tokens then one decode step."""
    ctx = np.asarray(ctx, dtype=np.int64)
    S = ctx.shape[0]
    poison, free_order = _placement(cfg, NB, seed_sub)
    rs = _rng(cfg, _STREAM_STEP)
    step_k = _normal(rs, (S, H, D), dtype)
    step_v = _normal(rs, (S, H, D), dtype)
    jobs = [(s, (int(ctx[s]) - 1, H, D)) for s in range(S)]
    hks = _draw_many(cfg, _STREAM_K, jobs, dtype)
    hvs = _draw_many(cfg, _STREAM_V, jobs, dtype)
    segs = {}
    for s in range(S):
        n = int(ctx[s]) - 1
        segs[s] = [(0, n, hks[s], hvs[s]), (n, n + 1, step_k[s:s + 1], step_v[s:s + 1])]
    q = _normal(_rng(cfg, _STREAM_Q), (S, H, D), dtype)
    ops = [("add", s, int(ctx[s]) - 1) for s in range(S)]
    ops.append(("step", list(range(S))))
    maxb = int(math.ceil(int(ctx.max()) / bs))
    return Workload(cfg=cfg, name=name, H=H, D=D, dtype=dtype, bs=bs, NB=NB,
                    scale=scale, free_order=free_order, poison_block=poison,
                    ctx=ctx, q=q, ops=ops, max_blocks_per_seq=maxb,
                    partition_tokens=part_tokens, _segments=segs)


def _config4(cow: bool, bs: int = 16) -> Workload:
    """8 groups x 8 samples sharing one 1024-token prompt, private tails U[1,256].

    cow=False: the samples fork right after the prompt, which ends on a block
    boundary, so every tail starts in a fresh private block.
    cow=True: each group first generates r_g in [1,15] common tokens, then forks;
    the shared last block is partly filled, so the first divergent append of all
    but the last sample of a group copies it on write."""
    cfg, H, D, dtype, G, per = 4, 40, 128, "bf16", 8, 8
    prompt = 1024
    NB = 4096
    poison, free_order = _placement(cfg, NB)
    rt = _rng(cfg, _STREAM_TAIL)
    tails = rt.integers(1, 257, size=G * per).astype(np.int64)
    r = _rng(cfg, _STREAM_FORK).integers(1, 16, size=G).astype(np.int64)
    rs = _rng(cfg, _STREAM_STEP)
    step_k = _normal(rs, (G * per, H, D), dtype)
    step_v = _normal(rs, (G * per, H, D), dtype)
    segs, ops, ctx = {}, [], np.zeros(G * per, dtype=np.int64)
    shared_len = [prompt + (int(r[g]) if cow else 0) for g in range(G)]
    # T = tokens after the shared part, including the step token
    T = [int(tails[j]) if not cow else
         max(int(tails[j]), int(r[j // per]) + 1) - int(r[j // per]) for j in range(G * per)]
    jobs = [(g, (shared_len[g], H, D)) for g in range(G)] + \
           [(1000 + j, (T[j] - 1, H, D)) for j in range(G * per)]
    ks = _draw_many(cfg, _STREAM_K, jobs, dtype)
    vs = _draw_many(cfg, _STREAM_V, jobs, dtype)
    for g in range(G):
        shared = shared_len[g]
        pk, pv = ks[g], vs[g]
        members = [g * per + i for i in range(per)]
        for j in members:
            hk, hv = ks[G + j], vs[G + j]
            segs[j] = [(0, shared, pk, pv),
                       (shared, shared + T[j] - 1, hk, hv),
                       (shared + T[j] - 1, shared + T[j], step_k[j:j + 1], step_v[j:j + 1])]
            ctx[j] = shared + T[j]
        ops.append(("add", members[0], shared))
        for j in members[1:]:
            ops.append(("fork", members[0], j))
    for j in range(G * per):
        shared = segs[j][0][1]
        n = int(ctx[j]) - shared - 1
        if n > 0:
            ops.append(("extend", j, n))
    ops.append(("step", list(range(G * per))))
    q = _normal(_rng(cfg, _STREAM_Q), (G * per, H, D), dtype)
    maxb = int(math.ceil(int(ctx.max()) / bs))
    name = CONFIG_NAMES[4] + ("-cow" if cow else "")
    return Workload(cfg=4, name=name, H=H, D=D, dtype=dtype, bs=bs, NB=NB,
                    scale=1.0 / math.sqrt(D), free_order=free_order,
                    poison_block=poison, ctx=ctx, q=q, ops=ops,
                    max_blocks_per_seq=maxb, _segments=segs,
                    notes=("fork after prompt+r_g common tokens" if cow else
                           "fork at the prompt's block boundary"))


def config5_ctx() -> np.ndarray:
    z = _rng(5, _STREAM_CTX).standard_normal(256)
    return np.clip(np.round(512.0 * np.exp(0.8 * z)), 1, 4096).astype(np.int64)


def make_workload(cfg: int, bs: int | None = None, cow: bool = False,
                  S: int | None = None, values: bool = True,
                  placement: str = "random") -> Workload:
    """Build workload ``cfg`` (1..5).

    ``bs`` selects the block size of the config-5 sweep; ``cow`` selects the
    copy-on-write variant of config 4; ``S`` (config 5 only) keeps the first S
    sequences, for smaller CPU-side cases; ``values=False`` skips the K/V
    draws (only the shapes and the op script are built); ``placement``
    "identity" hands out blocks in id order (contiguous tables: the
    indirection's cost is measured against it)."""
    if placement not in ("random", "identity"):
        raise ValueError(placement)
    _VALUES[0] = bool(values)
    _IDENTITY[0] = placement == "identity"
    try:
        wl = _make(cfg, bs, cow, S)
        if _IDENTITY[0]:
            wl.name += "-identity"
        return wl
    finally:
        _VALUES[0] = True
        _IDENTITY[0] = False


def make_custom(seed: int, H: int, D: int, dtype: str, bs: int, ctx, NB: int | None = None,
                scale: float | None = None, part_tokens: int = 0) -> Workload:
    """A small independent-sequence workload with the given shapes (kernel-instance
    coverage): prefill of ctx-1 tokens, one step.  ``seed`` >= 100 keeps its
    streams apart from the five named configs."""
    ctx = np.asarray(ctx, dtype=np.int64)
    demand = int(sum(max(1, math.ceil(int(c) / bs)) for c in ctx))
    NB = NB or demand + 8
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    return _simple(seed, f"custom-{dtype}-D{D}-bs{bs}", H, D, dtype, bs, NB, ctx, sc,
                   part_tokens=part_tokens)


def _make(cfg, bs, cow, S):
    if cfg == 1:
        return _simple(1, CONFIG_NAMES[1], 4, 64, "f32", 16, 64, [1, 17, 33, 100],
                       1.0 / 8.0)
    if cfg == 2:
        ctx = _rng(2, _STREAM_CTX).integers(256, 2049, size=30)
        return _simple(2, CONFIG_NAMES[2], 40, 128, "f16", 16, 4096, ctx,
                       1.0 / math.sqrt(128))
    if cfg == 3:
        return _simple(3, CONFIG_NAMES[3], 40, 128, "f16", 16, 4096, [4096] * 8,
                       1.0 / math.sqrt(128), part_tokens=512)
    if cfg == 4:
        return _config4(cow)
    if cfg == 5:
        bs = 16 if bs is None else int(bs)
        ctx = config5_ctx()
        if S is not None:
            ctx = ctx[:S]
        demand = int(sum(math.ceil(int(c) / bs) for c in ctx))
        NB = int(math.ceil(1.1 * demand))
        wl = _simple(5, CONFIG_NAMES[5] + f"-bs{bs}", 40, 128, "f16", bs, NB, ctx,
                     1.0 / math.sqrt(128), seed_sub=bs)
        return wl
    raise ValueError(f"unknown config {cfg}")


def make_fork_tree(seed: int, H: int, D: int, dtype: str, bs: int, roots: int = 2,
                   forks: int = 10, max_prompt: int = 1400, max_extend: int = 300,
                   prompt_lens=None) -> Workload:
    """A random fork tree (parallel sampling and beam-like branching, comfyai.app
    "6.4 PagedAttention" 6.4.2-6.4.3): ``roots`` prompts, then ``forks`` times a
    random existing sequence is forked and the child (and sometimes the parent)
    generates a random number of tokens, so that sequences share prefixes of
    every length, forks of forks included; then one step over every sequence in
    a random order.  ``prompt_lens`` fixes the root prompt lengths.  ``seed`` >=
    100 keeps the streams apart from the five named configs."""
    rt = _rng(seed, _STREAM_TREE)
    lens, segs, ops = {}, {}, []
    sub = [0]

    def new_tokens(seq, n):
        if n <= 0:
            return
        k = _normal(_rng(seed, _STREAM_K, sub[0]), (n, H, D), dtype)
        v = _normal(_rng(seed, _STREAM_V, sub[0]), (n, H, D), dtype)
        sub[0] += 1
        t = lens[seq]
        segs[seq].append((t, t + n, k, v))
        lens[seq] = t + n

    for r in range(roots):
        n = int(prompt_lens[r]) if prompt_lens is not None else int(rt.integers(0, max_prompt + 1))
        lens[r], segs[r] = 0, []
        new_tokens(r, n)
        ops.append(("add", r, n))
    nxt = roots
    for _ in range(forks):
        parent = int(rt.choice(sorted(lens)))
        child = nxt
        nxt += 1
        L = lens[parent]
        segs[child] = [(a, min(b, L), k[:min(b, L) - a], v[:min(b, L) - a])
                       for (a, b, k, v) in segs[parent] if a < L]
        lens[child] = L
        ops.append(("fork", parent, child))
        n = int(rt.integers(0, max_extend + 1))
        new_tokens(child, n)
        if n:
            ops.append(("extend", child, n))
        if rt.random() < 0.3:
            n = int(rt.integers(1, max_extend + 1))
            new_tokens(parent, n)
            ops.append(("extend", parent, n))
    seqs = [int(x) for x in rt.permutation(nxt)]
    # the step appends one token to every sequence, in the listed order; the
    # decode rows follow that order
    rs = _rng(seed, _STREAM_STEP)
    step_k = _normal(rs, (nxt, H, D), dtype)
    step_v = _normal(rs, (nxt, H, D), dtype)
    for i, s in enumerate(seqs):
        t = lens[s]
        segs[s].append((t, t + 1, step_k[i:i + 1], step_v[i:i + 1]))
        lens[s] = t + 1
    ops.append(("step", seqs))
    # decode rows follow the step list
    ctx = np.array([lens[s] for s in seqs], dtype=np.int64)
    demand = sum(-(-lens[s] // bs) + 1 for s in seqs)
    NB = demand + 8
    poison, free_order = _placement(seed, NB)
    q = _normal(_rng(seed, _STREAM_Q), (nxt, H, D), dtype)
    maxb = int(math.ceil(int(ctx.max()) / bs))
    return Workload(cfg=seed, name=f"fork-tree-{seed}-{dtype}-bs{bs}", H=H, D=D, dtype=dtype,
                    bs=bs, NB=NB, scale=1.0 / math.sqrt(D), free_order=free_order,
                    poison_block=poison, ctx=ctx, q=q, ops=ops, max_blocks_per_seq=maxb,
                    _segments=segs, notes="random fork tree")


def make_beam_search(seed: int, H: int, D: int, dtype: str, bs: int, prompt: int = 600,
                     width: int = 4, steps: int = 12) -> Workload:
    """Beam search as a block tree (polomodov.tech "vLLM and PagedAttention" slide
    14: candidates share prefixes like forked processes; comfyai.app 6.4.2).
    A prompt of ``prompt`` tokens is forked into ``width`` beams; each of
    ``steps`` rounds appends one token to every beam, then selects ``width`` new
    beams, each a fork of a seeded random surviving parent (with repetition),
    and retires the old beams.  A final step appends one more token to every
    beam and decodes them.  Children of one parent share its partly filled last
    block, so their next appends copy it on write."""
    rt = _rng(seed, _STREAM_TREE)
    segs, lens, ops = {}, {}, []
    sub = [0]

    def new_tokens(seq, n):
        k = _normal(_rng(seed, _STREAM_K, sub[0]), (n, H, D), dtype)
        v = _normal(_rng(seed, _STREAM_V, sub[0]), (n, H, D), dtype)
        sub[0] += 1
        t = lens[seq]
        segs[seq].append((t, t + n, k, v))
        lens[seq] = t + n

    def fork(parent, child):
        segs[child] = list(segs[parent])
        lens[child] = lens[parent]

    segs[0], lens[0] = [], 0
    new_tokens(0, prompt)
    ops.append(("add", 0, prompt))
    beams = list(range(1, width + 1))
    for b in beams:
        fork(0, b)
    ops.append(("select", [(0, b) for b in beams], [0]))
    nxt = width + 1
    for _ in range(steps):
        for b in beams:
            new_tokens(b, 1)
            ops.append(("extend", b, 1))
        parents = [beams[int(i)] for i in rt.integers(0, width, size=width)]
        children = list(range(nxt, nxt + width))
        nxt += width
        for p, c in zip(parents, children):
            fork(p, c)
        ops.append(("select", list(zip(parents, children)), list(beams)))
        beams = children   # retired beams keep their segments (the script replays them)
    rs = _rng(seed, _STREAM_STEP)
    step_k = _normal(rs, (width, H, D), dtype)
    step_v = _normal(rs, (width, H, D), dtype)
    for i, b in enumerate(beams):
        t = lens[b]
        segs[b].append((t, t + 1, step_k[i:i + 1], step_v[i:i + 1]))
        lens[b] = t + 1
    ops.append(("step", beams))
    ctx = np.array([lens[b] for b in beams], dtype=np.int64)
    NB = (width + 1) * (-(-int(ctx.max()) // bs) + 2) + 8
    poison, free_order = _placement(seed, NB)
    q = _normal(_rng(seed, _STREAM_Q), (width, H, D), dtype)
    return Workload(cfg=seed, name=f"beam-search-{seed}-{dtype}-bs{bs}-w{width}", H=H, D=D,
                    dtype=dtype, bs=bs, NB=NB, scale=1.0 / math.sqrt(D), free_order=free_order,
                    poison_block=poison, ctx=ctx, q=q, ops=ops,
                    max_blocks_per_seq=int(math.ceil(int(ctx.max()) / bs)), _segments=segs,
                    notes="beam search block tree")


def make_preemption(seed: int, H: int, D: int, dtype: str, bs: int, rounds_before: int = 20,
                    rounds_out: int = 40) -> Workload:
    """Preemption by swapping (polomodov.tech "vLLM and PagedAttention" slide 15:
    when the pool runs short the scheduler evicts the newest request as a
    whole; its blocks go to host memory and come back when there is room).
    Four requests in arrival order: a long single sequence (id 0), a group of 3
    parallel samples of one prompt (comfyai.app 6.4.3), a single sequence and,
    newest, a group of 2 samples.  After ``rounds_before`` rounds of one
    appended token per sequence the pool is nearly full (it has the blocks in
    use then plus 2) and the newest group is swapped out; the others run
    ``rounds_out`` more rounds, taking the blocks the group gave back; request
    0 finishes (freed); the group is swapped in, to other physical blocks, and
    a final step decodes the remaining sequences."""
    rp = _rng(seed, _STREAM_TREE)
    prompts = [40 * bs] + [int(x) for x in rp.integers(bs + 1, 12 * bs, size=3)]
    groups = [[0], [1, 2, 3], [4], [5, 6]]
    segs, lens, ops = {}, {}, []
    sub = [0]

    def new_tokens(seq, n):
        k = _normal(_rng(seed, _STREAM_K, sub[0]), (n, H, D), dtype)
        v = _normal(_rng(seed, _STREAM_V, sub[0]), (n, H, D), dtype)
        sub[0] += 1
        t = lens[seq]
        segs[seq].append((t, t + n, k, v))
        lens[seq] = t + n

    def blocks(gs):
        """Blocks in use by groups gs: a group's full prompt blocks once (its
        members copy the partly filled prompt block on their first append)."""
        n = 0
        for g in gs:
            members = groups[g]
            full = prompts[g] // bs if len(members) > 1 else 0
            n += full + sum(-(-(lens[m] - full * bs) // bs) for m in members)
        return n

    for g, members in enumerate(groups):
        lead = members[0]
        segs[lead], lens[lead] = [], 0
        new_tokens(lead, prompts[g])
        ops.append(("add", lead, prompts[g]))
        for m in members[1:]:
            segs[m], lens[m] = list(segs[lead]), lens[lead]
            ops.append(("fork", lead, m))

    def rounds(seqs, n):
        for _ in range(n):
            for s_ in seqs:
                new_tokens(s_, 1)
                ops.append(("extend", s_, 1))

    rounds([m for g in groups for m in g], rounds_before)
    at_swap = blocks(range(4))
    group_blocks = blocks([3])
    newest = groups[-1]
    ops.append(("host_pool", group_blocks + 2))
    ops.append(("swap_out", list(newest)))
    rounds([m for g in groups[:3] for m in g], rounds_out)
    # the pool: nearly full when the group goes out (2 spare blocks), large
    # enough for the others' growth (which then takes the group's blocks)
    NB = max(at_swap + 2, blocks([0, 1, 2])) + 1        # + the poison block
    ops.append(("free", 0))
    assert NB - 1 - blocks([1, 2]) >= group_blocks, "the swap-in must fit"
    ops.append(("swap_in", list(newest)))
    final = [m for g in groups[1:] for m in g]
    rs = _rng(seed, _STREAM_STEP)
    step_k = _normal(rs, (len(final), H, D), dtype)
    step_v = _normal(rs, (len(final), H, D), dtype)
    for i, s_ in enumerate(final):
        t = lens[s_]
        segs[s_].append((t, t + 1, step_k[i:i + 1], step_v[i:i + 1]))
        lens[s_] = t + 1
    ops.append(("step", final))
    ctx = np.array([lens[s_] for s_ in final], dtype=np.int64)
    poison, free_order = _placement(seed, NB)
    q = _normal(_rng(seed, _STREAM_Q), (len(final), H, D), dtype)
    return Workload(cfg=seed, name=f"preemption-{seed}-{dtype}-bs{bs}", H=H, D=D, dtype=dtype,
                    bs=bs, NB=NB, scale=1.0 / math.sqrt(D), free_order=free_order,
                    poison_block=poison, ctx=ctx, q=q, ops=ops,
                    max_blocks_per_seq=int(math.ceil(int(ctx.max()) / bs)), _segments=segs,
                    notes="newest request swapped out and back in")


def make_prefill(seed: int, H: int, D: int, dtype: str, bs: int, prefix_lens, q_lens):
    """Chunked prefill (brentwoodlivery "5.3.18", the prefill/decode cards;
    comfyai.app 6.4.3): sequence s already holds prefix_lens[s] cached tokens
    (written by an "add"), then a chunk of q_lens[s] new tokens is written
    through the slot mapping (an "extend") and attends causally over the whole
    cache.  Returns (workload, q [sum q_lens, H, D], cu_q int32 [S + 1]); the
    workload has no decode step, its ctx is prefix + chunk."""
    prefix_lens = [int(x) for x in prefix_lens]
    q_lens = [int(x) for x in q_lens]
    S = len(q_lens)
    segs, ops = {}, []
    for s_ in range(S):
        n = prefix_lens[s_] + q_lens[s_]
        k = _normal(_rng(seed, _STREAM_K, s_), (n, H, D), dtype)
        v = _normal(_rng(seed, _STREAM_V, s_), (n, H, D), dtype)
        segs[s_] = [(0, n, k, v)]
        ops.append(("add", s_, prefix_lens[s_]))
    for s_ in range(S):
        if q_lens[s_]:
            ops.append(("extend", s_, q_lens[s_]))
    ctx = np.array([p + q for p, q in zip(prefix_lens, q_lens)], dtype=np.int64)
    NB = int(sum(-(-int(c) // bs) for c in ctx)) + 8
    poison, free_order = _placement(seed, NB)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = _normal(_rng(seed, _STREAM_Q), (int(cu_q[-1]), H, D), dtype)
    wl = Workload(cfg=seed, name=f"prefill-{seed}-{dtype}-bs{bs}", H=H, D=D, dtype=dtype, bs=bs,
                  NB=NB, scale=1.0 / math.sqrt(D), free_order=free_order, poison_block=poison,
                  ctx=ctx, q=np.zeros((S, H, D), dtype=DTYPES[dtype][0]), ops=ops,
                  max_blocks_per_seq=max(1, int(math.ceil(int(ctx.max()) / bs))),
                  _segments=segs, notes="chunked prefill: cached prefix + new chunk")
    return wl, q, cu_q
