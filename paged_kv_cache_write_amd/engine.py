"""One decode engine step on one GPU: host slot assignment, table shipment,
copy-on-write copies, slot-mapped cache write and PagedAttention decode.

The step follows the pages' serving loop: the scheduler's block manager gives
every running sequence the slot of its new token (a fresh block when the last
one is full, a copy when the last one is shared), the block tables travel to
the GPU every step (polomodov.tech "vLLM and PagedAttention" slides 11-13 and
16), the copies are made, the new K/V are written, then decode attends over
the updated contexts.  All device work is enqueued on one stream, so the copy
precedes the write and the write precedes the read without host waits.

Host work is the C++ block manager (libpa.so); device work is libpa.so's HIP
kernels.  torch provides the device memory, pinned staging and the stream.
"""
from __future__ import annotations

import numpy as np

from . import BlockManager, DTYPE_CODES, cache_write, copy_blocks, decode, decode_partitions, \
    decode_plan, decode_reduce

__all__ = ["PagedKVEngine"]


class PagedKVEngine:
    """Block pool + block manager + per-step staging for a batch of decoding sequences.

    k_cache / v_cache: [num_blocks, num_heads, block_size, head_dim] of ``dtype``.
    ``pad_block`` fills the unused tail of every exported table row (never read).
    ``max_batch`` bounds the sequences of one step.
    """

    RING = 3  # pinned staging buffers in flight

    def __init__(self, num_blocks, num_heads, head_dim, block_size, dtype, max_blocks_per_seq,
                 max_batch, free_order=None, pad_block=0, device="cuda", fill=None):
        import torch
        self.torch = torch
        self.NB, self.H, self.D, self.bs = int(num_blocks), int(num_heads), int(head_dim), \
            int(block_size)
        self.dtype = dtype
        self.dt_code = DTYPE_CODES()[dtype]
        self.maxB, self.max_batch = int(max_blocks_per_seq), int(max_batch)
        self.pad = int(pad_block)
        self.device = torch.device(device)
        shape = (self.NB, self.H, self.bs, self.D)
        if fill is None:
            self.k_cache = torch.empty(shape, dtype=dtype, device=self.device)
            self.v_cache = torch.empty(shape, dtype=dtype, device=self.device)
        else:
            self.k_cache = torch.full(shape, fill, dtype=dtype, device=self.device)
            self.v_cache = torch.full(shape, fill, dtype=dtype, device=self.device)
        self.bm = BlockManager(self.NB, self.bs, free_order)
        # Packed per-step staging: slots int64[B] | ctx int32[B] | cow int32[2B] | tables int32[B*maxB]
        B = self.max_batch
        self._n_i32 = B + 2 * B + B * self.maxB
        nbytes = 8 * B + 4 * self._n_i32
        self._host = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
                      for _ in range(self.RING)]
        self._events = [None] * self.RING
        self._ring = 0
        self._dev = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self._workspace = None
        self.last_step = {}

    # ------------------------------------------------------------- views
    def _views(self, buf, n):
        B = self.max_batch
        raw = buf.numpy() if buf.device.type == "cpu" else None
        if raw is not None:
            slots = raw[:8 * B].view(np.int64)[:n]
            i32 = raw[8 * B:].view(np.int32)
            ctx = i32[:B][:n]
            cows = i32[B:3 * B]
            tables = i32[3 * B:3 * B + B * self.maxB][:n * self.maxB].reshape(n, self.maxB)
            return slots, ctx, cows, tables
        slots = buf[:8 * B].view(self.torch.int64)[:n]
        i32 = buf[8 * B:].view(self.torch.int32)
        ctx = i32[:B][:n]
        cows = i32[B:3 * B]
        tables = i32[3 * B:3 * B + B * self.maxB][:n * self.maxB].view(n, self.maxB)
        return slots, ctx, cows, tables

    # ------------------------------------------------------ cache building
    def add_sequence(self, seq, k=None, v=None, num_tokens=None):
        """Prefill: a new sequence whose first tokens' K/V ([n, H, D] device tensors) are
        written through the slot mapping."""
        n = int(k.shape[0]) if k is not None else int(num_tokens)
        self.bm.add_seq(seq, n)
        if n and k is not None:
            slots = self.torch.from_numpy(self.bm.slots(seq, 0, n)).to(self.device)
            cache_write(k, v, slots, self.k_cache, self.v_cache)

    def fork(self, parent, child):
        self.bm.fork(parent, child)

    def extend(self, seqs, k, v):
        """Append one token per entry of ``seqs`` (in order; repeats allowed) with K/V rows
        k[i], v[i]: copies first, then the writes."""
        slots, cows = self.bm.append_slots(seqs)
        if cows.size:
            copy_blocks(self.k_cache, self.v_cache,
                        self.torch.from_numpy(cows).to(self.device))
        cache_write(k, v, self.torch.from_numpy(slots).to(self.device), self.k_cache,
                    self.v_cache)
        return slots, cows

    # --------------------------------------------------------------- step
    def step(self, seqs, q, k_new, v_new, scale, out=None, partition_tokens=0, timing=None,
             two_launch=False):
        """One decode step for ``seqs`` (int64 array): append a slot to each, ship the
        tables, copy shared last blocks, write k_new/v_new [S, H, D], decode q [S, H, D].

        ``timing`` (optional) = (start_event, end_event) recorded around the
        decode launch.  ``two_launch`` uses pa_decode_partitions + pa_decode_reduce
        instead of the single-launch pa_decode.  Returns out [S, H, D]."""
        torch = self.torch
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        S = seqs.size
        assert S <= self.max_batch
        i = self._ring
        self._ring = (i + 1) % self.RING
        if self._events[i] is not None:
            self._events[i].synchronize()          # staging buffer i is free again
        host = self._host[i]
        h_slots, h_ctx, h_cows, h_tables = self._views(host, S)
        ncow = self.bm.step_into(seqs, h_slots, h_cows, h_tables, self.pad, h_ctx)
        max_ctx = int(h_ctx.max()) if S else 0
        stream = torch.cuda.current_stream(self.device)
        self._dev.copy_(host, non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        self._events[i] = ev
        d_slots, d_ctx, d_cows, d_tables = self._views(self._dev, S)
        if ncow:
            copy_blocks(self.k_cache, self.v_cache, d_cows[:2 * ncow].view(ncow, 2))
        cache_write(k_new, v_new, d_slots, self.k_cache, self.v_cache)
        if out is None:
            out = torch.empty_like(q)
        _, _, ws = decode_plan(S, self.H, self.D, self.bs, max_ctx, self.dt_code,
                               partition_tokens)
        if ws and (self._workspace is None or self._workspace.numel() < ws):
            # zero-filled: pa_decode's per-row counters must start at zero
            self._workspace = torch.zeros(ws, dtype=torch.uint8, device=self.device)
        args = (q, self.k_cache, self.v_cache, d_tables, d_ctx, scale, max_ctx, out,
                self._workspace, partition_tokens)
        if timing is not None:
            timing[0].record(stream)
        if two_launch:
            decode_partitions(*args)
            decode_reduce(*args)
        else:
            decode(*args)
        if timing is not None:
            timing[1].record(stream)
        self.last_step = dict(num_cow=ncow, max_ctx=max_ctx, ctx=h_ctx.copy(),
                              cows=h_cows[:2 * ncow].reshape(-1, 2).copy(),
                              slots=h_slots.copy())
        return out
