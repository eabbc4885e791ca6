"""Runs spa_unified_step across decode steps under the scheduler of
include/spa_sched.h: bucket-balanced phases, delayed verification, and list
persistence (a verify writes its request's list segment, the request's next
drafts read it).

Review of SparseSpec, 核心方法 / "Unified batch scheduler + fused attention
kernel" and "Delayed verification"; blog sections 4.2-4.3.  The model is not
run: the accepted-token counts come from the scheduler's seeded acceptance
process, and Q, K and V are synthetic N(0, 1) draws.  Device buffers are
sized once for the scheduler's capacity, except the workspace and the plan
buffers, which grow (after the device drains) when a step needs more.

With ``dependent=True`` the host waits, before it plans a step, for the
earlier step whose verify outcomes that plan needs (a real server reads them
back to run accept/reject): the step just before it, or with delayed
verification the one before that -- so delayed verification lets the host's
planning of step t+1 overlap the GPU's step t.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import binding as bd


class SchedDriver:
    def __init__(self, slots, spec_k, num_qo_heads, num_kv_heads, head_dim, sparsity, prompt,
                 output, delayed=False, accept_prob=bd.ACCEPT_PROB_6_16_OF_8, seed=0,
                 device="cuda:0", dtype=torch.bfloat16, max_len=None, num_cus=0):
        k = int(spec_k)
        max_len = int(max_len or (prompt[1] + output[1] + k + 1))
        self.sched = bd.Scheduler(slots, k, num_qo_heads, num_kv_heads, sparsity, prompt, output,
                                  max_len, delayed=delayed, accept_prob=accept_prob, seed=seed)
        self.dev = torch.device(device)
        self.k, self.Hq, self.Hkv, self.d = k, num_qo_heads, num_kv_heads, head_dim
        self.slots, self.max_len = int(slots), max_len
        self.k_cap = self.sched.idx_elems // (self.slots * num_kv_heads)
        g = torch.Generator(device=self.dev).manual_seed(int(seed) * 1000003 + 7)
        self.gen = g
        # every slot owns a page-table row of max_len distinct pool slots
        self.num_slots = 2 * self.slots * max_len
        perm = torch.randperm(self.num_slots, generator=g, device=self.dev)[:self.slots * max_len]
        self.page_table = perm.to(torch.int32).view(self.slots, max_len).contiguous()
        self.k_pool = torch.randn((self.num_slots, num_kv_heads, head_dim), generator=g,
                                  device=self.dev).to(dtype)
        self.v_pool = torch.randn((self.num_slots, num_kv_heads, head_dim), generator=g,
                                  device=self.dev).to(dtype)
        rows = self.sched.max_rows
        self.q = torch.randn((rows, num_qo_heads, head_dim), generator=g, device=self.dev).to(dtype)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((rows, num_qo_heads), dtype=torch.float32, device=self.dev)
        self.logits = torch.empty((max(self.sched.logits_elems, 1),), dtype=torch.float32,
                                  device=self.dev)
        self.idx = torch.zeros((self.sched.idx_elems,), dtype=torch.int32, device=self.dev)
        self.lay = bd.layout(num_qo_heads, num_kv_heads, head_dim, dtype, self.num_slots, max_len)
        self.ws = bd.workspace(1 << 20, self.dev)
        self.plans = bd.PlanRing(1 << 16)
        # request r of a step reads the page-table row of its slot
        self.opts = bd.Options(num_cus=num_cus or
                               torch.cuda.get_device_properties(self.dev).multi_processor_count)
        self.opts.c.page_table_row_count = self.slots
        self.last = None
        self.delayed = bool(delayed)
        self.done = []  # completion events of the last two steps

    def _init_lists(self, a):
        """Initial lists of new requests (what their prefill would leave):
        K = ceil(s L) positions of [0, L) per KV head, one drawn uniformly in
        each of K equal strata (floor(i L / K) .. floor((i+1) L / K) - 1), so
        they are distinct and ascending."""
        for s, L, K in zip(a["new_slots"].tolist(), a["new_len"].tolist(), a["new_count"].tolist()):
            base = s * self.Hkv * self.k_cap
            i = torch.arange(K + 1, device=self.dev, dtype=torch.int64)
            edge = (i * L) // K
            lo, width = edge[:-1], edge[1:] - edge[:-1]  # width >= 1 since K <= L
            u = torch.rand((self.Hkv, K), generator=self.gen, device=self.dev, dtype=torch.float64)
            pos = lo + torch.minimum((u * width).long(), width - 1)
            self.idx[base:base + self.Hkv * K] = pos.to(torch.int32).reshape(-1)

    def _sizes(self, st, a):
        args = (self.lay, st.B, self.k, a["is_verify"], a["seq_lens"], a["idx_count"], self.opts)
        ws, plan = bd.workspace_bytes(*args), bd.plan_bytes(*args)
        if ws > self.ws.numel() or plan > self.plans.nbytes:
            torch.cuda.synchronize(self.dev)  # the old buffers may still be read
            if ws > self.ws.numel():
                self.ws = bd.workspace(int(ws * 1.25), self.dev)
            if plan > self.plans.nbytes:
                self.plans = bd.PlanRing(int(plan * 1.25))

    def plan(self, fresh_q=False, dependent=False):
        """Plans the next step: the scheduler's step record and its arrays
        (fresh_q: new query rows drawn for it; dependent: first wait for the
        step whose verify outcomes this plan needs)."""
        if dependent:
            lag = 2 if self.delayed else 1
            if len(self.done) >= lag:
                self.done[-lag].synchronize()
        st = self.sched.next()
        a = self.sched.arrays(st)
        if st.n_new:
            self._init_lists(a)
        if fresh_q:
            self.q[:st.rows].normal_(generator=self.gen)
        self._sizes(st, a)
        self.opts.c.page_table_rows = st.slot
        self.last = (st, a)
        return st, a

    def launch(self):
        """Runs the planned step on the current stream."""
        st, a = self.last
        plan = self.plans.next()
        vp = C.c_void_p
        bd._check(bd.load().spa_unified_step(
            C.byref(self.lay), st.B, self.k, vp(st.is_verify), vp(st.seq_lens), vp(st.q_indptr),
            bd._dptr(self.page_table), bd._dptr(self.q), bd._dptr(self.k_pool),
            bd._dptr(self.v_pool), vp(st.idx_count), vp(st.idx_off), bd._dptr(self.idx),
            bd._dptr(self.o), bd._dptr(self.lse), bd._dptr(self.logits), vp(st.logits_off), 1,
            self.k, bd._dptr(self.ws), self.ws.numel(), bd._hptr(plan), bd._nbytes(plan),
            C.byref(self.opts.c), bd._stream(self.q)))
        ev = torch.cuda.Event()
        ev.record()
        self.done = (self.done + [ev])[-2:]

    def commit(self):
        self.sched.commit()

    def step(self, fresh_q=False, dependent=False):
        st, a = self.plan(fresh_q, dependent)
        self.launch()
        self.commit()
        return st
