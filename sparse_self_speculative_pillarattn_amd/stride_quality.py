"""How well a verify's PillarAttn lists serve the k drafts of the following
speculation stride.

Review of SparseSpec, 关键观察 (the critical tokens of one step stay critical
over the next k steps, which is why the pattern can be refreshed once per
stride) and 核心方法 / PillarAttn versus Quest (lists judged by attention
coverage and top-10 recall).  The chain, all through the C ABI:

  1. a verify over context L_r (spa_verify_attn, k+1 rows) and PillarAttn's
     top-K over its k draft rows and GQA group (spa_pillar_topk), K_r =
     ceil(s L_r) positions per KV head;
  2. for each stride position i = 1..k a draft query q_i drifting away from
     the verify's last row (synth.drift_queries) at context L_r + i, scored
     exactly over its whole context (spa_verify_attn with spec_k = 1, the
     query in row 1);
  3. spa_list_quality of the verify's lists against that row (coverage: the
     draft's attention mass on the list; recall@T: the share of its top-T
     positions on the list), and of a fresh list for comparison (PillarAttn's
     top-K of the draft row itself, same K_r: the best a list of that size
     built from this row's own scores does).

The draft reads only its list, so the positions L_r .. L_r + i - 1 written
after the verify count against coverage.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as bd
from . import synth


class StrideRun:
    def __init__(self, b: synth.Batch, verify_lens, sigma: float, seed: int = 0,
                 top_t: int = 10):
        w = b.w
        self.b, self.w = b, w
        self.k, self.Hq, self.Hkv, self.d = w.spec_k, w.num_qo_heads, w.num_kv_heads, w.head_dim
        self.B = b.B
        self.vlens = [int(L) for L in verify_lens]
        assert all(L + self.k <= Lb for L, Lb in zip(self.vlens, b.seq_lens))
        self.K = [synth.topk_count(L, w.sparsity) for L in self.vlens]
        self.top_t = int(top_t)
        dev = b.q.device
        self.dev = dev
        self.lay = bd.layout(self.Hq, self.Hkv, self.d, b.q.dtype, b.num_slots, b.stride)
        k, Hq, Hkv = self.k, self.Hq, self.Hkv
        # verify buffers
        self.vloff = np.concatenate([[0], np.cumsum([(k + 1) * Hq * L for L in self.vlens])[:-1]]
                                    ).astype(np.int64)
        self.vlogits = torch.empty((int(sum((k + 1) * Hq * L for L in self.vlens)),), device=dev)
        self.vlse = torch.empty((self.B * (k + 1), Hq), device=dev)
        self.vo = torch.empty_like(b.q)
        self.ioff = np.concatenate([[0], np.cumsum([Hkv * K for K in self.K])[:-1]]).astype(np.int64)
        self.lists = torch.zeros((int(sum(Hkv * K for K in self.K)) + 1,), dtype=torch.int32,
                                 device=dev)
        self.fresh = torch.zeros_like(self.lists)
        # the verify's last row per request, and the drafts drifting from it
        last = torch.tensor([b.q_indptr[r] + k for r in range(self.B)], device=dev)
        self.q_draft = synth.drift_queries(b.q.index_select(0, last), k, sigma, seed)
        ws_v = bd.workspace_bytes(self.lay, self.B, k, [1] * self.B, self.vlens, self.K)
        dlens = [L + k for L in self.vlens]
        ws_d = bd.workspace_bytes(self.lay, self.B, 1, [1] * self.B, dlens, self.K)
        self.ws = bd.workspace(max(ws_v, ws_d), dev)
        self.qws = bd.workspace(bd.list_quality_workspace_bytes(self.B, Hq, dlens), dev)
        self.dlogits = torch.empty((int(sum(2 * Hq * L for L in dlens)),), device=dev)
        self.dlse = torch.empty((2 * self.B, Hq), device=dev)
        self.top = torch.empty((self.B, Hq, self.top_t), dtype=torch.int32, device=dev)
        self.cov = torch.empty((self.B, Hq), device=dev)
        self.rec = torch.empty((self.B, Hq), device=dev)

    def verify(self):
        """Step 1: the verify and its PillarAttn lists (rows 1..k averaged)."""
        b, k = self.b, self.k
        bd.verify_attn(self.lay, self.B, k, self.vlens, b.page_table, b.q, b.k_pool, b.v_pool,
                       self.vo, self.vlse, self.vlogits, self.vloff, self.ws)
        bd.pillar_topk(self.B, k, self.Hq, self.Hkv, 1, k, self.vlens, self.K, self.vlogits,
                       self.vloff, self.vlse, self.lists, self.ioff, self.ws)

    def draft_lens(self, i: int) -> list:
        return [L + i for L in self.vlens]

    def score_draft(self, i: int):
        """Step 2: exact attention of the stride's i-th draft query (row 1 of a
        2-row spec_k = 1 verify) over its context L_r + i.  Returns the host
        logits offsets."""
        lens = self.draft_lens(i)
        qi = self.q_draft[i - 1]                                  # [B][Hq][d]
        q2 = torch.stack([qi, qi], dim=1).reshape(-1, self.Hq, self.d).contiguous()
        loff = np.concatenate([[0], np.cumsum([2 * self.Hq * L for L in lens])[:-1]]
                              ).astype(np.int64)
        o = torch.empty_like(q2)
        b = self.b
        bd.verify_attn(self.lay, self.B, 1, lens, b.page_table, q2, b.k_pool, b.v_pool, o,
                       self.dlse, self.dlogits, loff, self.ws)
        return loff

    def quality(self, i: int, loff, lists: torch.Tensor):
        """Step 3: coverage and recall@T of `lists` (K_r per KV head at
        self.ioff) against the scored draft row."""
        bd.list_quality(self.B, 1, self.Hq, self.Hkv, 1, self.top_t, self.draft_lens(i),
                        self.dlogits, loff, self.dlse, self.K, self.ioff, lists, self.top,
                        self.cov, self.rec, self.qws)

    def fresh_lists(self, i: int, loff):
        """PillarAttn's top-K_r of the draft row itself (row 1, its GQA group)."""
        bd.pillar_topk(self.B, 1, self.Hq, self.Hkv, 1, 1, self.draft_lens(i), self.K,
                       self.dlogits, loff, self.dlse, self.fresh, self.ioff, self.ws)

    def run(self, positions=None) -> dict:
        """Whole chain; per stride position: coverage and recall arrays [B][Hq]
        of the verify's lists ("pillar") and of the fresh lists ("fresh")."""
        self.verify()
        out = {}
        for i in (positions or range(1, self.k + 1)):
            loff = self.score_draft(i)
            self.quality(i, loff, self.lists)
            pc, pr = self.cov.clone(), self.rec.clone()
            self.fresh_lists(i, loff)
            self.quality(i, loff, self.fresh)
            out[i] = {"pillar": (pc, pr), "fresh": (self.cov.clone(), self.rec.clone())}
        torch.cuda.synchronize(self.dev)
        return out
