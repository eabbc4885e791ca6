"""Block-structured KV pools with host offload and prefetch
(include/spa_kvcache.h): device pools cut into blocks, pinned host arenas,
the block manager and a copy stream.

Review of SparseSpec, 核心方法 / "Dynamic KV-Cache manager" and 关键观察,
observation 5.  Attention keeps page size 1: a request's page-table row maps
position j to slot blk[j / block_slots] * block_slots + j % block_slots, so
the row changes when the request comes back into other blocks.  The copies run
on `self.copy` (a default-priority stream, copy engines) and are ordered
against the compute stream with events: an offload waits for the last step
that read its blocks, and a step that reads prefetched blocks waits for the
prefetch.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as bd


class BlockKV:
    def __init__(self, num_qo_heads, num_kv_heads, head_dim, dtype, dev_blocks, host_chunks,
                 block_slots, max_requests, max_len, device="cuda:0"):
        self.dev = torch.device(device)
        self.Hkv, self.d, self.dtype = num_kv_heads, head_dim, dtype
        self.bs = int(block_slots)
        self.slots = int(dev_blocks) * self.bs
        self.max_len = int(max_len)
        self.k_pool = torch.empty((self.slots, num_kv_heads, head_dim), dtype=dtype, device=self.dev)
        self.v_pool = torch.empty_like(self.k_pool)
        self.lay = bd.layout(num_qo_heads, num_kv_heads, head_dim, dtype, self.slots, self.max_len)
        self.block_bytes = bd.kv_block_bytes(self.lay, self.bs)
        n = max(int(host_chunks), 1) * self.block_bytes
        self.k_arena = torch.empty((n,), dtype=torch.uint8, pin_memory=True)
        self.v_arena = torch.empty((n,), dtype=torch.uint8, pin_memory=True)
        self.kvm = bd.KVManager(dev_blocks, host_chunks, block_slots, max_requests,
                                -(-self.max_len // self.bs))
        self.copy = torch.cuda.Stream(self.dev)
        self.last_moves = (np.zeros(0, np.int32), np.zeros(0, np.int32))  # (blocks, chunks)

    def write(self, req, k_rows, v_rows):
        """Admits `req` with the K and V rows of its positions ([L][H_kv][d]
        device tensors) on the current stream; False if the device blocks ran
        out."""
        L = k_rows.shape[0]
        if not self.kvm.reserve(req, L):
            return False
        slots = torch.from_numpy(self.kvm.page_row(req, L).astype(np.int64)).to(self.dev)
        self.k_pool.index_copy_(0, slots, k_rows.to(self.dtype))
        self.v_pool.index_copy_(0, slots, v_rows.to(self.dtype))
        return True

    def page_rows(self, reqs, lens, stride=None) -> torch.Tensor:
        """Device page table [len(reqs)][stride] of resident requests."""
        stride = int(stride or self.max_len)
        pt = np.zeros((len(reqs), stride), np.int32)
        for i, (r, L) in enumerate(zip(reqs, lens)):
            pt[i, :L] = self.kvm.page_row(r, L)
        return torch.from_numpy(pt).to(self.dev)

    def _after(self, wait):
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream(self.dev) if wait is None else wait)
        return ev

    def offload(self, need_free, keep=(), after=None):
        """Plans and enqueues offloads until `need_free` device blocks are free.
        The copies wait for the work queued so far on the current stream (or
        for the event `after`).  Returns (requests, done event, blocks moved);
        the freed blocks must not be written before the done event."""
        blocks, chunks, reqs = self.kvm.plan_offload(need_free, keep)
        self.last_moves = (blocks, chunks)
        done = torch.cuda.Event()
        bd.kv_offload(self.lay, self.bs, blocks, chunks, self.k_pool, self.v_pool, self.k_arena,
                      self.v_arena, stream=self.copy, wait_event=after or self._after(None),
                      done_event=done)
        return reqs, done, len(blocks)

    def prefetch(self, keep_free=0, after=None):
        """Plans and enqueues prefetches (first offloaded first).  Returns
        (requests, done event, blocks moved); steps that read them must wait
        for the done event (torch.cuda.current_stream().wait_event(done))."""
        chunks, blocks, reqs = self.kvm.plan_prefetch(keep_free)
        self.last_moves = (blocks, chunks)
        done = torch.cuda.Event()
        bd.kv_prefetch(self.lay, self.bs, chunks, blocks, self.k_arena, self.v_arena, self.k_pool,
                       self.v_pool, stream=self.copy, wait_event=after or self._after(None),
                       done_event=done)
        return reqs, done, len(blocks)

    def free_blocks(self, lens: dict) -> np.ndarray:
        """Device blocks no resident request holds; lens maps every request
        the manager may hold to its length (host side)."""
        used = np.zeros(self.slots // self.bs, bool)
        for r, L in lens.items():
            if self.kvm.where(r) == 1 and L > 0:
                used[self.kvm.page_row(r, L) // self.bs] = True
        return np.nonzero(~used)[0]
