"""Oracle for the paged KV-cache write and PagedAttention decode (test infrastructure).

This is a plain, slow, CPU reference written from the pages.  It exists only to
check the HIP path: tests, the smoke check and the benchmark's CPU-baseline leg
may call it; the library never does.  It shares no code with the HIP path.

Arithmetic is float64 (NumPy); K/V/q arrive already rounded to their storage
type (float32, float16, or bfloat16 carried as uint16 bits) and are widened
exactly.  Nothing here is blocked, fused, partitioned or computed online.

Sources (pages of the vLLM / PagedAttention material):
  * comfyai.app "6.4 PagedAttention", 6.4.1 Mechanism: K/V split into
    fixed-length blocks, a block table maps logically contiguous blocks to
    non-contiguous physical blocks allocated as tokens are generated.
  * comfyai.app 6.4.2 Inference Workflows / 6.4.3 Usages in Prefilling and
    Decoding: reference counts on physical blocks and copy-on-write; the sample
    that diverges gets the new block, the other keeps the old one whose count
    drops by one.
  * polomodov.tech "vLLM and PagedAttention" slides 9-13: the kernel fetches
    K/V from non-contiguous blocks by address; logical-to-physical table
    example; a new block only when the previous one is full, the new token goes
    to the free slot of the last block; one shared pool; only the last block is
    copied on write.
  * brentwoodlivery "5.3.18 LLM serving / vLLM / quantized inference": the
    query attends over all previous tokens' cached K/V; PagedAttention changes
    only the memory layout, not the attention computation; KV size
    2*B*S*L*d_model*p and the Llama-2-13B worked example.

Parity pins: every function here is pinned by tests/test_oracle.py against
printed numbers, closed forms, invariants and brute force; see that file.
"""
from __future__ import annotations

import math
from collections import deque

import numpy as np

__all__ = [
    "widen", "oracle_cache_write", "oracle_gather", "oracle_decode",
    "oracle_copy_blocks", "BlockPoolModel", "kv_cache_bytes",
    "kv_bytes_per_token", "useful_kv_fraction", "run_workload",
    "attention_brute_force",
    "oracle_decode_contiguous",
    "oracle_prefill",
]


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64.

    bfloat16 is the upper half of a float32, so its bits shifted left by 16
    are that float32 exactly."""
    if dtype == "bf16":
        x = np.asarray(x, dtype=np.uint16)
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype in ("f16", "f32"):
        return np.asarray(x).astype(np.float64)
    raise ValueError(dtype)


def oracle_cache_write(k, v, slot_mapping, k_cache, v_cache):
    """Slot-mapped write of new tokens' K/V into the block pool, in place.

    Token n goes to block slot//bs, offset slot%bs of every head
    (polomodov.tech slide 11: the new token fills the free slot of the last
    block; comfyai.app 6.4.1: blocks of fixed length).  A negative slot means
    "no write" (padding).  Slots must be distinct.  The copy is exact in the
    storage type.  Layout: k, v [N, H, D]; caches [NB, H, bs, D]."""
    slot_mapping = np.asarray(slot_mapping, dtype=np.int64)
    NB, H, bs, D = k_cache.shape
    assert k.shape == (slot_mapping.shape[0], H, D) and v.shape == k.shape
    keep = slot_mapping >= 0
    slots = slot_mapping[keep]
    assert np.unique(slots).size == slots.size, "slots within one write must be distinct"
    blk, off = slots // bs, slots % bs
    assert np.all(blk < NB), "slot beyond the pool"
    k_cache[blk, :, off, :] = k[keep]
    v_cache[blk, :, off, :] = v[keep]


def oracle_copy_blocks(k_cache, v_cache, pairs):
    """Copy whole physical blocks src -> dst (K and V), in the listed order.

    This is the copy of copy-on-write (comfyai.app 6.4.3: a new physical block
    is created for the writer; polomodov.tech slide 13: only the last block is
    copied)."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def oracle_gather(cache, table_row, ctx):
    """Contiguous [ctx, H, D] view of one sequence's tokens, read through its table.

    Logical block j of the sequence lives in physical block table_row[j]
    (polomodov.tech slide 10, comfyai.app 6.4.1); only the first ceil(ctx/bs)
    entries are read, and only the first ctx tokens are kept."""
    NB, H, bs, D = cache.shape
    nblk = -(-int(ctx) // bs)
    if nblk == 0:
        return np.empty((0, H, D), dtype=cache.dtype)
    blocks = [cache[int(table_row[j])] for j in range(nblk)]      # each [H, bs, D]
    tokens = np.concatenate([b.transpose(1, 0, 2) for b in blocks], axis=0)
    return tokens[:ctx]


def attention_one(q, K, V, scale):
    """Textbook softmax attention of one query head over its cached tokens.

    logits_t = scale * <q, K_t>;  w = exp(logits - max) / sum(exp(logits - max));
    out = sum_t w_t V_t.  q [D], K, V [L, D], all float64.  Returns (out, w)."""
    logits = scale * (K @ q)
    w = np.exp(logits - logits.max())
    w = w / w.sum()
    return w @ V, w


def oracle_decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                  seqs=None, return_weights=False):
    """PagedAttention decode: out[s,h,:] = attention of q[s,h] over the sequence's ctx tokens.

    Paging changes where K/V live, not what attention computes
    (brentwoodlivery 5.3.18, the "PagedAttention makes attention faster"
    common-mistake card), so each sequence's K/V are gathered into a contiguous
    array and plain attention is applied per head.  A sequence with ctx = 0
    gives a zero row.  ``seqs`` restricts the computation to some sequences
    (the other rows are NaN).  Returns float64 [S, H, D]."""
    S, H, D = q.shape
    out = np.full((S, H, D), np.nan)
    weights = {}
    qf = widen(q, dtype)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        if L == 0:
            out[s] = 0.0
            continue
        K = widen(oracle_gather(k_cache, block_tables[s], L), dtype)
        V = widen(oracle_gather(v_cache, block_tables[s], L), dtype)
        for h in range(H):
            o, w = attention_one(qf[s, h], K[:, h, :], V[:, h, :], scale)
            out[s, h] = o
            if return_weights:
                weights[(s, h)] = w
    return (out, weights) if return_weights else out


def oracle_decode_contiguous(q, k, v, context_lens, scale, dtype, layout="SLHD"):
    """Decode over non-paged K/V (polomodov.tech "vLLM and PagedAttention"
    slide 19 compares the paged kernel with this; brentwoodlivery "5.3.18", the
    card saying paging leaves the attention arithmetic unchanged): for each
    sequence s and head h, attention of q[s,h] over the first context_lens[s]
    token rows of k[s] / v[s], laid out [S, L, H, D] ("SLHD") or [S, H, L, D]
    ("SHLD").  A zero context gives a zero row.  Returns float64 [S, H, D]."""
    S, H, D = q.shape
    out = np.zeros((S, H, D))
    qf = widen(q, dtype)
    for s in range(S):
        L = int(context_lens[s])
        if L == 0:
            continue
        ks = widen(k[s, :L] if layout == "SLHD" else k[s, :, :L], dtype)
        vs = widen(v[s, :L] if layout == "SLHD" else v[s, :, :L], dtype)
        for h in range(H):
            kh = ks[:, h, :] if layout == "SLHD" else ks[h]
            vh = vs[:, h, :] if layout == "SLHD" else vs[h]
            out[s, h] = attention_one(qf[s, h], kh, vh, scale)[0]
    return out


def oracle_prefill(q, k_cache, v_cache, block_tables, cu_q, context_lens, scale, dtype):
    """Causal prefill attention over the paged cache (brentwoodlivery "5.3.18",
    the prefill/decode cards; comfyai.app 6.4.3: the prompt's K/V are written
    into blocks first): with q_len = cu_q[s+1] - cu_q[s], query row cu_q[s] + i
    sits at position p = context_lens[s] - q_len + i and attends to the
    sequence's tokens 0..p, gathered from its blocks.  Returns float64 [T, H, D]."""
    T, H, D = q.shape
    out = np.zeros((T, H, D))
    qf = widen(q, dtype)
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        q_len = int(cu_q[s + 1]) - int(cu_q[s])
        if q_len == 0:
            continue
        K = widen(oracle_gather(k_cache, block_tables[s], L), dtype)
        V = widen(oracle_gather(v_cache, block_tables[s], L), dtype)
        for i in range(q_len):
            pos = L - q_len + i
            row = int(cu_q[s]) + i
            for h in range(H):
                out[row, h] = attention_one(qf[row, h], K[:pos + 1, h, :], V[:pos + 1, h, :],
                                            scale)[0]
    return out


def attention_brute_force(q, K, V, scale):
    """Scalar pure-Python attention for tiny cases (one head): nested loops,
    math.exp and math.fsum.  q [D], K, V [L][D] as Python floats."""
    L, D = len(K), len(q)
    logits = [scale * math.fsum(q[d] * K[t][d] for d in range(D)) for t in range(L)]
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    z = math.fsum(e)
    return [math.fsum(e[t] / z * V[t][d] for t in range(L)) for d in range(D)]


class BlockPoolModel:
    """Reference block manager: one shared pool, FIFO free list, refcounts, CoW.

    * One pool serves every sequence; a free block goes to whoever needs it
      next (polomodov.tech slide 12).  The free list is a FIFO: pop from the
      front, freed blocks go to the back.
    * add_seq(n): prefill allocates ceil(n/bs) blocks, refcount 1 each.
    * fork(parent, child): the child's table is a copy of the parent's and every
      block's refcount goes up by one (comfyai.app 6.4.3: A1 and A2 share the
      prompt's blocks; slide 14: candidates share prefixes like forked
      processes).
    * append_slot(seq): the new token has position t = len.  If t is a multiple
      of bs the last block is full (or absent) and a new block is taken
      (slide 11).  Otherwise, if the last block is shared (refcount > 1), it is
      copied on write: the writer gets a fresh block (refcount 1) that receives
      a copy, and the old block's refcount drops by one (comfyai.app 6.4.3;
      slide 13).  slot = table[t // bs] * bs + t % bs.
    * free_seq: every block of the sequence loses one reference; blocks that
      reach zero go back to the free list in logical order.
    * Preemption by swapping (slide 15: the newest request is evicted as a
      whole, its blocks go to host memory and come back later): a second,
      host pool with its own FIFO free list.  swap_out(seqs) requires that the
      group holds its blocks alone (each block's refcount equals the group's
      references to it); walking the group's tables in order, each distinct
      block is given the next host block, keeps its refcount there, and goes
      back to the device free list.  swap_in is the same move in the other
      direction.  Both change nothing when the other pool is short of blocks.
    * blocks_needed(seqs): how many device blocks append_slot over seqs would
      take, without taking them.
    """

    class NoBlocks(Exception):
        pass

    def __init__(self, NB, bs, free_order=None):
        self.NB, self.bs = int(NB), int(bs)
        order = range(self.NB) if free_order is None else [int(b) for b in free_order]
        self.free = deque(order)
        self.ref = [0] * self.NB
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.host_free: deque = deque()
        self.host_ref: list[int] = []
        self.swapped: dict[int, list[int]] = {}   # seq -> host block table
        self.swapped_lens: dict[int, int] = {}

    def _pop(self):
        if not self.free:
            raise BlockPoolModel.NoBlocks()
        b = self.free.popleft()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def add_seq(self, seq, n):
        assert seq not in self.tables
        need = -(-int(n) // self.bs)
        if need > len(self.free):
            raise BlockPoolModel.NoBlocks()
        self.tables[seq] = [self._pop() for _ in range(need)]
        self.lens[seq] = int(n)

    def fork(self, parent, child):
        assert child not in self.tables
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append_slot(self, seq):
        """Returns (slot, cow) where cow is None or (src, dst)."""
        t, table, cow = self.lens[seq], self.tables[seq], None
        if t % self.bs == 0:
            table.append(self._pop())
        elif self.ref[table[-1]] > 1:
            src = table[-1]
            dst = self._pop()
            self.ref[src] -= 1
            table[-1] = dst
            cow = (src, dst)
        slot = table[t // self.bs] * self.bs + t % self.bs
        self.lens[seq] = t + 1
        return slot, cow

    def slots(self, seq, t0, t1):
        table = self.tables[seq]
        return [table[t // self.bs] * self.bs + t % self.bs for t in range(t0, t1)]

    def free_seq(self, seq):
        if seq in self.swapped:
            for b in self.swapped.pop(seq):
                self.host_ref[b] -= 1
                if self.host_ref[b] == 0:
                    self.host_free.append(b)
            del self.swapped_lens[seq]
            return
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[seq]

    def set_host_pool(self, n, free_order=None):
        assert not self.swapped
        order = range(int(n)) if free_order is None else [int(b) for b in free_order]
        self.host_free = deque(order)
        self.host_ref = [0] * int(n)

    @staticmethod
    def _move(seqs, tables, lens, ref, free, to_tables, to_lens, to_ref, to_free):
        """Move the group's tables to the other pool; returns [(src, dst)] pairs."""
        assert len(set(seqs)) == len(seqs)
        count = {}
        order = []
        for s in seqs:
            for b in tables[s]:
                if b not in count:
                    count[b] = 0
                    order.append(b)
                count[b] += 1
        if any(count[b] != ref[b] for b in order):
            raise ValueError("the group shares blocks with a sequence outside it")
        if len(order) > len(to_free):
            raise BlockPoolModel.NoBlocks()
        new = {}
        for b in order:
            nb = to_free.popleft()
            to_ref[nb] = ref[b]
            ref[b] = 0
            free.append(b)
            new[b] = nb
        for s in seqs:
            to_tables[s] = [new[b] for b in tables.pop(s)]
            to_lens[s] = lens.pop(s)
        return [(b, new[b]) for b in order]

    def swap_out(self, seqs):
        return self._move(list(seqs), self.tables, self.lens, self.ref, self.free,
                          self.swapped, self.swapped_lens, self.host_ref, self.host_free)

    def swap_in(self, seqs):
        return self._move(list(seqs), self.swapped, self.swapped_lens, self.host_ref,
                          self.host_free, self.tables, self.lens, self.ref, self.free)

    def blocks_needed(self, seqs):
        """Device blocks append_slot over seqs would take: the append rules replayed
        on copies of the lengths and refcounts (None = the last block is private
        after a new block or a copy)."""
        ref, lens = list(self.ref), dict(self.lens)
        last = {s: (t[-1] if t else None) for s, t in self.tables.items()}
        taken = 0
        for s in seqs:
            t = lens[s]
            if t % self.bs == 0:
                taken += 1
                last[s] = None
            elif last[s] is not None and ref[last[s]] > 1:
                taken += 1
                ref[last[s]] -= 1
                last[s] = None
            lens[s] = t + 1
        return taken

    def table_array(self, seqs, width, pad):
        out = np.full((len(seqs), width), pad, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self.tables[s]
            out[i, :len(t)] = t
        return out


def kv_bytes_per_token(layers, heads, head_dim, elem_bytes):
    """Bytes of K and V one token occupies across all layers: 2 * L * H * D * p."""
    return 2 * layers * heads * head_dim * elem_bytes


def kv_cache_bytes(batch, seq_len, layers, d_model, elem_bytes):
    """KV-cache size 2*B*S*L*d_model*p (brentwoodlivery 5.3.18, formula card)."""
    return 2 * batch * seq_len * layers * d_model * elem_bytes


def useful_kv_fraction(ctx, bs):
    """Share of allocated token slots that hold real tokens: sum(ctx)/sum(ceil(ctx/bs)*bs)."""
    ctx = np.asarray(ctx, dtype=np.int64)
    alloc = (-(-ctx // bs)) * bs
    return float(ctx.sum()) / float(alloc.sum())


def run_workload(wl, decode=True, decode_seqs=None, fill=None):
    """Execute a workload's op script on the CPU and return the final state.

    One step (comfyai.app 6.4.3; polomodov.tech slides 11-13 and 16): every
    listed sequence gets a slot (allocating or copying on write), the copies
    are made, the step's K/V are written, then decode attends over the updated
    context lengths.  Extends and adds write their tokens the same way.

    Never-written pool slots hold NaN (so that reading one poisons the
    output), or zero when ``fill`` is given.  Returns a dict with the pools, the final
    tables, the context lengths, the step's slot mapping and CoW pairs, every
    CoW pair in the order made, and (if ``decode``) the fp64 output."""
    shape = (wl.NB, wl.H, wl.bs, wl.D)
    if wl.dtype == "bf16":
        # bfloat16 pools hold raw bits: 0x7FC0 is a quiet NaN
        k_cache = np.full(shape, 0x7FC0 if fill is None else 0, dtype=np.uint16)
    else:
        np_dt = np.float16 if wl.dtype == "f16" else np.float32
        k_cache = np.full(shape, np.nan if fill is None else 0.0, dtype=np_dt)
    v_cache = k_cache.copy()
    bm = BlockPoolModel(wl.NB, wl.bs, wl.free_order)
    all_cows, step_slots, step_cows, step_seqs = [], None, [], None
    for op in wl.ops:
        kind = op[0]
        if kind == "add":
            _, seq, n = op
            bm.add_seq(seq, n)
            k, v = wl.kv(seq, 0, n)
            oracle_cache_write(k, v, bm.slots(seq, 0, n), k_cache, v_cache)
        elif kind == "fork":
            bm.fork(op[1], op[2])
        elif kind == "free":
            bm.free_seq(op[1])
        elif kind == "host_pool":
            bm.set_host_pool(op[1])
            host_shape = (op[1],) + k_cache.shape[1:]
            poison = 0 if fill is not None else (0x7FC0 if wl.dtype == "bf16" else np.nan)
            k_host = np.full(host_shape, poison, dtype=k_cache.dtype)
            v_host = k_host.copy()
        elif kind == "swap_out":
            # preemption: the group's blocks are copied to the host pool, exactly
            for dev_b, host_b in bm.swap_out(op[1]):
                k_host[host_b] = k_cache[dev_b]
                v_host[host_b] = v_cache[dev_b]
        elif kind == "swap_in":
            for host_b, dev_b in bm.swap_in(op[1]):
                k_cache[dev_b] = k_host[host_b]
                v_cache[dev_b] = v_host[host_b]
        elif kind == "select":
            # beam selection: every (parent, child) fork, then the retired frees
            for parent, child in op[1]:
                bm.fork(parent, child)
            for seq in op[2]:
                bm.free_seq(seq)
        elif kind == "extend":
            _, seq, n = op
            for _ in range(n):
                t = bm.lens[seq]
                slot, cow = bm.append_slot(seq)
                if cow is not None:
                    oracle_copy_blocks(k_cache, v_cache, [cow])
                    all_cows.append(cow)
                k, v = wl.kv(seq, t, t + 1)
                oracle_cache_write(k, v, [slot], k_cache, v_cache)
        elif kind == "step":
            step_seqs = list(op[1])
            step_slots, new_k, new_v = [], [], []
            for seq in step_seqs:
                t = bm.lens[seq]
                slot, cow = bm.append_slot(seq)
                if cow is not None:
                    step_cows.append(cow)
                    all_cows.append(cow)
                step_slots.append(slot)
                k, v = wl.kv(seq, t, t + 1)
                new_k.append(k[0])
                new_v.append(v[0])
            oracle_copy_blocks(k_cache, v_cache, step_cows)
            oracle_cache_write(np.stack(new_k), np.stack(new_v), step_slots,
                               k_cache, v_cache)
        else:
            raise ValueError(kind)
    width = wl.max_blocks_per_seq
    if step_seqs is None:   # no decode step: every resident sequence, by id
        step_seqs = sorted(bm.tables)
    tables = bm.table_array(step_seqs, width, wl.poison_block)
    ctx = np.array([bm.lens[s] for s in step_seqs], dtype=np.int64)
    res = dict(k_cache=k_cache, v_cache=v_cache, tables=tables, ctx=ctx,
               step_slots=np.array(step_slots if step_slots is not None else [], dtype=np.int64),
               step_cows=np.array(step_cows, dtype=np.int64).reshape(-1, 2),
               all_cows=np.array(all_cows, dtype=np.int64).reshape(-1, 2),
               refcounts=np.array(bm.ref, dtype=np.int64), model=bm)
    if decode:
        res["out"] = oracle_decode(wl.q, k_cache, v_cache, tables, ctx, wl.scale,
                                   wl.dtype, seqs=decode_seqs)
    return res
