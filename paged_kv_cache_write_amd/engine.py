"""One decode engine step on one GPU: host slot assignment, table shipment,
copy-on-write copies, slot-mapped cache write and PagedAttention decode.

The step itself is native (pa_engine_step in libpa.so): the C++ block
manager appends one slot per sequence, the scheduler orders the decode work,
one host-to-device copy ships slots, tables, context lengths, copy pairs and
work items, and the copy, cache-write and decode kernels are enqueued on the
current stream.  This class owns the device memory (torch), the pinned
staging ring and the handles; prefill (add_sequence) and forks are here too.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import (BlockManager, DTYPE_CODES, StepInfo, _check, _ptr, cache_write, copy_blocks,
               lib)

__all__ = ["PagedKVEngine"]


class PagedKVEngine:
    """Block pool + block manager + native step for a batch of decoding sequences.

    k_cache / v_cache: [num_blocks, num_heads, block_size, head_dim] of ``dtype``.
    ``pad_block`` fills the unused tail of every exported table row (never used
    as an address).  ``max_batch`` bounds the sequences of one step and
    ``max_blocks_per_seq`` the table width (so contexts up to that many blocks).
    ``ring`` pinned staging slots let the host run that many steps ahead; with
    an even count one event guards each half of them.  The default is RING
    slots, or RING_LARGE when RING slots would take more than RING_BYTES of
    pinned memory (batches with wide tables).
    """

    # pinned staging slots in flight: two halves, one guard event each (a guard
    # event costs ~4.5 us of idle GPU, so one per 32 steps instead of 8)
    RING = 64
    RING_LARGE = 16
    RING_BYTES = 64 << 20

    def __init__(self, num_blocks, num_heads, head_dim, block_size, dtype, max_blocks_per_seq,
                 max_batch, free_order=None, pad_block=0, device="cuda", fill=None,
                 partition_tokens=0, ring=None):
        import torch
        self.torch = torch
        self.NB, self.H, self.D, self.bs = int(num_blocks), int(num_heads), int(head_dim), \
            int(block_size)
        self.dtype = dtype
        self.dt_code = DTYPE_CODES()[dtype]
        self.maxB, self.max_batch = int(max_blocks_per_seq), int(max_batch)
        self.pad = int(pad_block)
        self.partition_tokens = int(partition_tokens)
        self.device = torch.device(device)
        shape = (self.NB, self.H, self.bs, self.D)
        if fill is None:
            self.k_cache = torch.empty(shape, dtype=dtype, device=self.device)
            self.v_cache = torch.empty(shape, dtype=dtype, device=self.device)
        else:
            self.k_cache = torch.full(shape, fill, dtype=dtype, device=self.device)
            self.v_cache = torch.full(shape, fill, dtype=dtype, device=self.device)
        self.bm = BlockManager(self.NB, self.bs, free_order)
        L = self._lib = lib()  # the library that owns the handle
        slot = int(L.pa_engine_staging_bytes(self.max_batch, self.maxB, self.bs))
        if ring is None:
            ring = self.RING if slot * self.RING <= self.RING_BYTES else self.RING_LARGE
        self.ring = int(ring)
        self._host = torch.empty(slot * self.ring, dtype=torch.uint8, pin_memory=True)
        self._dev = torch.empty(slot, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        rc = L.pa_engine_create(self.bm._h, self.k_cache.data_ptr(), self.v_cache.data_ptr(),
                                self.NB, self.H, self.D, self.bs, self.dt_code, self.max_batch,
                                self.maxB, self.pad, self._host.data_ptr(), self.ring,
                                self._dev.data_ptr(), ctypes.byref(h))
        _check(rc, "pa_engine_create")
        self._e = h
        # kept on the instance: at interpreter exit module globals may be gone
        self._destroy = L.pa_engine_destroy
        ws = int(L.pa_engine_workspace_bytes(self._e, self.partition_tokens))
        # zero-filled once: the decode's per-row counters start at zero and
        # every completed decode leaves them at zero
        self.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=self.device)
        self._info = StepInfo()
        self._seqs_cache = (None, None, None)  # (seqs object, int64 array, its address)
        self._last_n = 0                       # sequences of the last step
        # the current stream's raw handle without a Stream object (~2 us less per step)
        self._raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        self._dev_index = self.device.index if self.device.index is not None \
            else torch.cuda.current_device()
        self.last_info = None

    def __del__(self):
        e = getattr(self, "_e", None)
        destroy = getattr(self, "_destroy", None)
        if e is not None and destroy is not None:
            destroy(e)
            self._e = None

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

    def set_host_pool(self, num_host_blocks, free_order=None):
        """Pinned host pool of num_host_blocks blocks for preempted requests."""
        torch = self.torch
        shape = (int(num_host_blocks), self.H, self.bs, self.D)
        self.k_host = torch.empty(shape, dtype=self.dtype, pin_memory=True)
        self.v_host = torch.empty(shape, dtype=self.dtype, pin_memory=True)
        self.bm.set_host_pool(num_host_blocks, free_order)

    def swap_out(self, seqs):
        """Preempt a request (a group holding its blocks alone): its blocks are copied
        to the host pool on the current stream and the device blocks are freed.
        Returns the (device, host) block pairs."""
        from . import copy_blocks_between
        pairs = self.bm.swap_out(seqs)
        if pairs.size:
            p = self.torch.from_numpy(pairs).to(self.device)
            copy_blocks_between(self.k_cache, self.v_cache, self.k_host, self.v_host, p)
        return pairs

    def swap_in(self, seqs):
        """Bring a preempted request back into (possibly other) device blocks.
        Returns the (host, device) block pairs."""
        from . import copy_blocks_between
        pairs = self.bm.swap_in(seqs)
        if pairs.size:
            p = self.torch.from_numpy(pairs).to(self.device)
            copy_blocks_between(self.k_host, self.v_host, self.k_cache, self.v_cache, p)
        return pairs

    def free(self, seq):
        """Release a finished sequence's blocks (shared ones stay with their holders)."""
        self.bm.free_seq(seq)

    def select(self, pairs, retire):
        """Beam-search selection: fork each (parent, child), then free ``retire``."""
        self.bm.select(pairs, retire)

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
    def step(self, seqs, q, k_new, v_new, scale, out=None, stream=None):
        """One decode step for ``seqs`` (distinct ids): append a slot to each, ship the
        tables, copy shared last blocks, write k_new/v_new [S, H, D], decode q [S, H, D].
        Returns out [S, H, D]."""
        torch = self.torch
        cached, arr, aptr = self._seqs_cache
        if cached is not seqs:
            arr = np.ascontiguousarray(seqs, dtype=np.int64)
            aptr = arr.__array_interface__["data"][0] if arr.size else None
            # An int64 contiguous array is used in place (arr is seqs), so a
            # later change of its contents is seen through the cached address;
            # anything else (a list, another dtype) is converted on every call.
            self._seqs_cache = (seqs, arr, aptr) if arr is seqs else (None, None, None)
        S = arr.size
        shape = (S, self.H, self.D)
        for t in (q, k_new, v_new):
            if t.shape != shape or t.dtype != self.dtype or not t.is_contiguous() or \
                    not t.is_cuda:
                raise ValueError("q, k_new, v_new must be contiguous [S, H, D] device tensors")
        if out is None:
            out = torch.empty_like(q)
        if stream is not None:
            st = stream.cuda_stream
        elif self._raw_stream is not None:
            st = self._raw_stream(self._dev_index)
        else:
            st = torch.cuda.current_stream(self.device).cuda_stream
        rc = self._lib.pa_engine_step(self._e, aptr, S, q.data_ptr(), k_new.data_ptr(),
                                      v_new.data_ptr(), float(scale), out.data_ptr(),
                                      self.workspace.data_ptr(), self.workspace.numel(),
                                      self.partition_tokens, st, ctypes.byref(self._info))
        _check(rc, "pa_engine_step")
        self._last_n = S
        self.last_info = self._info
        return out

    def set_sharing(self, enable: bool):
        """Shared-prefix groups in later steps (on by default)."""
        _check(self._lib.pa_engine_set_sharing(self._e, 1 if enable else 0),
               "pa_engine_set_sharing")

    @property
    def has_mapped_staging(self) -> bool:
        """True when the engine got host-written (mapped) device staging."""
        return bool(self._lib.pa_engine_has_mapped_staging(self._e))

    def set_mapped_staging(self, enable: bool):
        """Mapped device staging in later steps (on by default where available);
        off: the prologue kernel reads the pinned host slot."""
        _check(self._lib.pa_engine_set_mapped_staging(self._e, 1 if enable else 0),
               "pa_engine_set_mapped_staging")

    def set_decode_events(self, start=None, end=None):
        """Record ``start``/``end`` around the decode launch of the following steps
        (None = stop): torch.cuda.Event objects, or raw hipEvent_t handles (int)."""
        if start is None or end is None:
            _check(self._lib.pa_engine_set_decode_events(self._e, None, None), "set events")
            return
        stream = self.torch.cuda.current_stream(self.device)
        handles = []
        for ev in (start, end):
            if isinstance(ev, int):
                handles.append(ev)
                continue
            if ev.cuda_event == 0:     # torch creates the HIP event on first record
                ev.record(stream)
            handles.append(ev.cuda_event)
        _check(self._lib.pa_engine_set_decode_events(self._e, handles[0], handles[1]),
               "pa_engine_set_decode_events")

    @property
    def last_step(self):
        """Host copies of the last step: dict(ctx, slots, cows, num_cow, ...)."""
        info = self.last_info
        S = self._last_n
        slots = np.empty(S, dtype=np.int64)
        ctx = np.empty(S, dtype=np.int32)
        cows = np.empty((max(info.num_cow, 1), 2), dtype=np.int32)
        _check(self._lib.pa_engine_last_step(self._e, S, _ptr(slots), _ptr(ctx), _ptr(cows),
                                         info.num_cow), "pa_engine_last_step")
        return dict(ctx=ctx, slots=slots, cows=cows[:info.num_cow], num_cow=info.num_cow,
                    max_ctx=info.max_context_len, partition_tokens=info.partition_tokens,
                    num_items=info.num_items, num_group_items=info.num_group_items,
                    sum_ctx=info.sum_context_len)
