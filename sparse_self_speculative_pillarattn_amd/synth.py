"""Seeded synthetic inputs for the unified draft/verify decode-attention step.

This module only draws inputs: batch composition, sequence lengths, a page-size-1
paged KV pool with a shuffled page table, queries, keys and values, planted
"pillar" key columns, and the draft index lists a previous verify would have left
behind.  It holds none of the attention, averaging or top-K arithmetic; both the
HIP path and the oracle consume what it returns.

Workload shapes follow the attention layers of the Qwen3 models and the
reasoning-decode setting of "SparseSpec-MLSys26" (awesome-system-papers review):
Qwen3-1.7B / 8B / 14B, k = 8 (12 for the 14B shape), s = 0.05, batch up to 256,
outputs of 8K tokens and an AIME-like mean of about 13.5K tokens for Qwen3-14B
(section "问题与动机" and "实验与结果").  No benchmark item or model weight is
used: Q, K and V are N(0, 1) draws, with a few key columns pushed towards the
queries so that the attention has the pillar-shaped structure the blog describes
(marsggbo.github.io "SparseSpec", section 2 and 4.1).

All draws go through one ``torch.Generator`` seeded per workload, on the device
the caller names, so a run is reproducible on that device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Optional

import torch


# --------------------------------------------------------------------------- #
# workloads
# --------------------------------------------------------------------------- #
@dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic decode-attention step."""

    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                    # "bf16" or "f32"
    spec_k: int                   # speculation stride k; verify requests own k+1 rows
    sparsity: Fraction            # s, kept rational so that K = ceil(s L) is exact
    lengths: tuple                # ("fixed", L) | ("uniform", lo, hi) | ("lognormal", mean, sigma, lo, hi)
    n_verify: Optional[int] = None    # None: max(1, round(B / (k + 1)))
    pillars: tuple = ("frac", Fraction(1, 20))  # ("count", n) | ("frac", f)
    pillar_drift: float = 0.0     # fraction of pillar positions that a draft list holds stale
    pool_factor: int = 2          # pool slots = pool_factor * sum(L)
    seed: int = 0
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads


TINY = Workload(
    name="tiny-h4kv2-d64-f32-L256", batch=2, num_qo_heads=4, num_kv_heads=2, head_dim=64,
    dtype="f32", spec_k=4, sparsity=Fraction(1, 20), lengths=("fixed", 256), n_verify=1,
    pillars=("count", 8), seed=1)

QWEN3_1_7B = Workload(
    name="qwen3-1.7b-attn-B64-L2K-8K", batch=64, num_qo_heads=16, num_kv_heads=8, head_dim=128,
    dtype="bf16", spec_k=8, sparsity=Fraction(1, 20), lengths=("uniform", 2048, 8192),
    pillars=("frac", Fraction(1, 20)), seed=2)

QWEN3_8B = Workload(
    name="qwen3-8b-attn-B128-L8192", batch=128, num_qo_heads=32, num_kv_heads=8, head_dim=128,
    dtype="bf16", spec_k=8, sparsity=Fraction(1, 20), lengths=("fixed", 8192),
    pillars=("frac", Fraction(1, 20)), seed=3)

QWEN3_14B = Workload(
    name="qwen3-14b-attn-B256-lognormal13.5K", batch=256, num_qo_heads=40, num_kv_heads=8,
    head_dim=128, dtype="bf16", spec_k=12, sparsity=Fraction(1, 20),
    lengths=("lognormal", 13500.0, 0.6, 1024, 32768), pillars=("frac", Fraction(1, 20)),
    pillar_drift=0.3, seed=4)

LONG_CTX = Workload(
    name="long-ctx-B16-L64K-128K", batch=16, num_qo_heads=32, num_kv_heads=8, head_dim=128,
    dtype="bf16", spec_k=8, sparsity=Fraction(1, 50), lengths=("uniform", 65536, 131072),
    pillars=("frac", Fraction(1, 50)), seed=5)

WORKLOADS = {w.name: w for w in (TINY, QWEN3_1_7B, QWEN3_8B, QWEN3_14B, LONG_CTX)}
ORDERED = [TINY, QWEN3_1_7B, QWEN3_8B, QWEN3_14B, LONG_CTX]


def topk_count(length: int, s: Fraction) -> int:
    """K = ceil(s * L) in exact integer arithmetic, clamped to [1, L].

    The review of SparseSpec gives the default sparsity s = 0.05 for PillarAttn's
    top-K ("核心方法", PillarAttn); 256 tokens at s = 0.05 give 13 selected
    tokens.  A float ceil would turn 0.05 * 8200 into 411, hence the fraction.
    """
    s = Fraction(s)
    k = -((-length * s.numerator) // s.denominator)
    return max(1, min(length, k))


# --------------------------------------------------------------------------- #
# batch
# --------------------------------------------------------------------------- #
@dataclass
class Batch:
    """Everything one step consumes, on one device, plus host copies of the metadata."""

    w: Workload
    B: int
    seq_lens: list            # host ints, L_r (includes the k+1 verify tokens)
    is_verify: list           # host bools
    q_indptr: list            # host ints, B+1
    idx_count: list           # host ints: verify -> K_r to produce, draft -> list length
    idx_off: list             # host ints (elements into idx)
    logits_off: list          # host ints (elements into logits); -1 for drafts
    pillar_pos: list          # per request: int64 tensor [H_kv][n_p] (host), planted positions
    q: torch.Tensor           # [rows][H_q][d]
    k_pool: torch.Tensor      # [slots][H_kv][d]
    v_pool: torch.Tensor      # [slots][H_kv][d]
    page_table: torch.Tensor  # int32 [B][stride]
    idx: torch.Tensor         # int32, draft lists filled, verify segments zero
    num_slots: int
    stride: int
    logits_elems: int
    idx_elems: int

    @property
    def rows(self) -> int:
        return self.q_indptr[-1]

    def to(self, device) -> "Batch":
        """A copy whose tensors live on ``device`` (host metadata is shared)."""
        from dataclasses import replace
        return replace(self, q=self.q.to(device), k_pool=self.k_pool.to(device),
                       v_pool=self.v_pool.to(device), page_table=self.page_table.to(device),
                       idx=self.idx.to(device))


def _torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _draw_lengths(w: Workload, g: torch.Generator) -> list:
    kind = w.lengths[0]
    B = w.batch
    if kind == "fixed":
        return [int(w.lengths[1])] * B
    if kind == "uniform":
        lo, hi = int(w.lengths[1]), int(w.lengths[2])
        u = torch.randint(lo, hi + 1, (B,), generator=g, device="cpu")
        return [int(x) for x in u]
    if kind == "lognormal":
        mean, sigma, lo, hi = w.lengths[1:]
        mu = math.log(mean) - sigma * sigma / 2.0
        z = torch.randn((B,), generator=g, dtype=torch.float64, device="cpu")
        vals = torch.exp(mu + sigma * z).round().clamp(lo, hi)
        return [int(x) for x in vals]
    raise ValueError(kind)


def _n_pillars(w: Workload, L: int) -> int:
    kind, v = w.pillars
    if kind == "count":
        return min(int(v), L)
    n = int(Fraction(v) * L + Fraction(1, 2))  # round half up
    return max(1, min(n, L))


@dataclass
class Meta:
    """Host-side batch composition: lengths, phases, row and list offsets."""

    seq_lens: list
    is_verify: list
    q_indptr: list
    idx_count: list
    idx_off: list
    logits_off: list
    num_slots: int
    stride: int
    logits_elems: int
    idx_elems: int


def _draw_meta(w: Workload, hg: torch.Generator, seq_lens=None, is_verify=None,
               num_slots=None) -> Meta:
    B, k, Hq, Hkv = w.batch, w.spec_k, w.num_qo_heads, w.num_kv_heads
    lens = list(seq_lens) if seq_lens is not None else _draw_lengths(w, hg)
    assert len(lens) == B
    if is_verify is None:
        nv = w.n_verify if w.n_verify is not None else max(1, round(B / (k + 1)))
        nv = min(nv, B)
        perm = torch.randperm(B, generator=hg)
        ver = [False] * B
        for i in perm[:nv].tolist():
            ver[i] = True
    else:
        ver = [bool(x) for x in is_verify]
    for r in range(B):
        if ver[r] and lens[r] < k + 1:
            lens[r] = k + 1
    q_indptr = [0]
    for r in range(B):
        q_indptr.append(q_indptr[-1] + (k + 1 if ver[r] else 1))
    idx_count, idx_off, logits_off = [], [], []
    ioff = loff = 0
    for r in range(B):
        kr = topk_count(lens[r], w.sparsity)
        idx_count.append(kr)
        idx_off.append(ioff)
        ioff += Hkv * kr
        if ver[r]:
            logits_off.append(loff)
            loff += (k + 1) * Hq * lens[r]
        else:
            logits_off.append(-1)
    total = sum(lens)
    nslots = num_slots if num_slots is not None else max(1, w.pool_factor * total)
    assert nslots >= total
    return Meta(seq_lens=lens, is_verify=ver, q_indptr=q_indptr, idx_count=idx_count,
                idx_off=idx_off, logits_off=logits_off, num_slots=nslots,
                stride=max(lens) if B else 1, logits_elems=max(loff, 1), idx_elems=max(ioff, 1))


def make_meta(w: Workload, seed: Optional[int] = None, **kw) -> Meta:
    """The batch composition ``make_batch`` would draw, without any tensor."""
    seed = w.seed if seed is None else seed
    return _draw_meta(w, torch.Generator(device="cpu").manual_seed(seed), **kw)


def make_batch(w: Workload, device="cpu", seed: Optional[int] = None,
               seq_lens: Optional[list] = None, is_verify: Optional[list] = None,
               num_slots: Optional[int] = None, chunk_slots: int = 1 << 18) -> Batch:
    """Draw one step's inputs for workload ``w`` on ``device``.

    Recipe (all from one seeded generator):
      * lengths per ``w.lengths``; n_V = max(1, round(B/(k+1))) verify requests at
        seeded positions in the batch, the rest draft;
      * pool of ``pool_factor * sum(L)`` slots, page table = a seeded random
        permutation of the pool cut into consecutive per-request runs;
      * Q, K, V ~ N(0, 1), rounded to the workload dtype;
      * per (request, KV head) n_p pillar positions: their keys become
        z + 3 sqrt(d) u, u the unit mean query direction of that request and group;
      * draft lists: the pillar positions (a ``pillar_drift`` fraction swapped for
        stale random ones) plus seeded random fill up to K_r = ceil(s L), ascending.
    """
    seed = w.seed if seed is None else seed
    dev = torch.device(device)
    hg = torch.Generator(device="cpu").manual_seed(seed)            # metadata draws
    dg = torch.Generator(device=dev).manual_seed(seed * 7919 + 17)   # bulk tensor draws
    B = w.batch
    Hq, Hkv, d = w.num_qo_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    dt = _torch_dtype(w.dtype)
    meta = _draw_meta(w, hg, seq_lens, is_verify, num_slots)
    lens, ver, q_indptr = meta.seq_lens, meta.is_verify, meta.q_indptr
    rows = q_indptr[-1]
    total = sum(lens)
    nslots, stride = meta.num_slots, meta.stride

    # page table: a random permutation of the pool, consecutive runs per request
    perm = torch.randperm(nslots, generator=hg)[:total].to(torch.int32)
    pt = torch.zeros((B, stride), dtype=torch.int32)
    off = 0
    for r in range(B):
        pt[r, :lens[r]] = perm[off:off + lens[r]]
        off += lens[r]

    # Host draws first (pillar positions, then the draft lists), so that the
    # bulk device generation below is the last work of the setup: the GPU is
    # still busy with it when the caller's first steps are queued, instead of
    # idling through the host work (after an idle period the GPU's clocks take
    # about 10 ms of load to settle again).
    pillar_pos = []
    for r in range(B):
        L = lens[r]
        npil = _n_pillars(w, L)
        pos = torch.stack([torch.randperm(L, generator=hg)[:npil] for _ in range(Hkv)])
        pos, _ = pos.sort(dim=1)
        pillar_pos.append(pos)

    # index lists: verify requests will write K_r entries, drafts read theirs
    idx_count, idx_off = meta.idx_count, meta.idx_off
    idx = torch.zeros((meta.idx_elems,), dtype=torch.int32)
    for r in range(B):
        if ver[r]:
            continue
        L, kr = lens[r], idx_count[r]
        for g in range(Hkv):
            pil = pillar_pos[r][g]
            if w.pillar_drift > 0 and len(pil) > 0:
                nstale = int(round(w.pillar_drift * len(pil)))
                keep = torch.randperm(len(pil), generator=hg)[:len(pil) - nstale]
                pil = pil[keep]
            pil = pil[:kr]
            mask = torch.ones(L, dtype=torch.bool)
            mask[pil] = False
            rest = torch.nonzero(mask).flatten()
            fill = rest[torch.randperm(len(rest), generator=hg)[:kr - len(pil)]]
            lst, _ = torch.cat([pil, fill]).sort()
            idx[idx_off[r] + g * kr: idx_off[r] + (g + 1) * kr] = lst.to(torch.int32)

    # every pillar key as (request, KV head, slot): slots are distinct within a
    # request (a permutation) and across requests, so the planting below
    # writes each (slot, head) once
    pil_r, pil_g, pil_s = [], [], []
    for r in range(B):
        pos = pillar_pos[r]
        pil_r.append(torch.full((pos.numel(),), r, dtype=torch.int64))
        pil_g.append(torch.arange(Hkv, dtype=torch.int64).repeat_interleave(pos.shape[1]))
        pil_s.append(pt[r].long()[pos.reshape(-1)])

    # host-to-device copies of what the device work below needs, queued before
    # it (a copy from pageable memory waits for the work queued ahead of it)
    pt_dev, idx_dev = pt.to(dev), idx.to(dev)
    per_row = torch.repeat_interleave(
        torch.arange(B), torch.tensor([q_indptr[r + 1] - q_indptr[r] for r in range(B)],
                                      dtype=torch.int64)).to(dev)
    nrow = torch.tensor([(q_indptr[r + 1] - q_indptr[r]) * G for r in range(B)],
                        dtype=torch.float32).to(dev)
    rr, gg, ss = (torch.cat(t).to(dev) if B else None for t in (pil_r, pil_g, pil_s))

    # Q, K, V
    q = torch.randn((rows, Hq, d), generator=dg, device=dev, dtype=torch.float32).to(dt)
    k_pool = torch.empty((nslots, Hkv, d), device=dev, dtype=dt)
    v_pool = torch.empty((nslots, Hkv, d), device=dev, dtype=dt)
    for s0 in range(0, nslots, chunk_slots):
        s1 = min(nslots, s0 + chunk_slots)
        k_pool[s0:s1] = torch.randn((s1 - s0, Hkv, d), generator=dg, device=dev,
                                    dtype=torch.float32).to(dt)
        v_pool[s0:s1] = torch.randn((s1 - s0, Hkv, d), generator=dg, device=dev,
                                    dtype=torch.float32).to(dt)

    # pillars: each key gets 3 sqrt(d) u added, u the unit mean of the
    # request's query rows over the G heads of the key's KV head
    if B > 0:
        qsum = torch.zeros((B, Hkv, d), device=dev, dtype=torch.float32)
        qsum.index_add_(0, per_row, q.float().reshape(rows, Hkv, G, d).sum(dim=2))
        qbar = qsum / nrow[:, None, None]
        u = qbar / qbar.norm(dim=2, keepdim=True).clamp_min(1e-30)       # [B][Hkv][d]
        z = k_pool[ss, gg].float()
        k_pool[ss, gg] = (z + 3.0 * math.sqrt(d) * u[rr, gg]).to(dt)

    return Batch(w=w, B=B, seq_lens=lens, is_verify=ver, q_indptr=q_indptr,
                 idx_count=idx_count, idx_off=idx_off, logits_off=meta.logits_off,
                 pillar_pos=pillar_pos, q=q, k_pool=k_pool, v_pool=v_pool,
                 page_table=pt_dev, idx=idx_dev, num_slots=nslots, stride=stride,
                 logits_elems=meta.logits_elems, idx_elems=meta.idx_elems)


def uniform_batch(w: Workload, B: int, L: int, verify_mask: list, device="cpu",
                  seed: int = 0) -> Batch:
    """A batch with every length fixed to ``L`` and an explicit verify/draft mask."""
    from dataclasses import replace
    w2 = replace(w, batch=B, lengths=("fixed", L))
    return make_batch(w2, device=device, seed=seed, is_verify=verify_mask)


def stride_batch(w: Workload, device="cpu", seed: Optional[int] = None,
                 n_req: Optional[int] = None) -> tuple:
    """Inputs of one speculation stride: a batch whose requests all verify
    (k+1 rows each) at context L_r, with K/V and page-table entries for L_r + k
    positions, so that the k drafts after the verify (contexts L_r + 1 ..
    L_r + k) read positions the pool holds.  Lengths, pool, Q, K, V and pillar
    planting follow ``make_batch`` (pillars are drawn over [0, L_r + k) and
    point along the verify rows' mean query direction); ``n_req`` takes the
    first n_req requests of the workload's length draw.  Returns (batch over
    L_r + k, [L_r]): the verify runs with the shorter lengths."""
    from dataclasses import replace
    seed = w.seed if seed is None else seed
    lens = make_meta(w, seed).seq_lens
    if n_req is not None:
        lens = lens[:n_req]
    B, k = len(lens), w.spec_k
    lens = [max(L, k + 1) for L in lens]
    w2 = replace(w, batch=B)
    b = make_batch(w2, device=device, seed=seed, seq_lens=[L + k for L in lens],
                   is_verify=[True] * B)
    return b, lens


def drift_queries(q0: torch.Tensor, steps: int, sigma: float, seed: int) -> torch.Tensor:
    """Draft queries that drift away from q0 [B][H_q][d] over ``steps`` decode
    steps: a seeded random walk, q_i = (q0 + sigma * (e_1 + ... + e_i)) /
    sqrt(1 + i sigma^2) with e_j ~ N(0, 1) i.i.d., so q_i keeps q0's per-entry
    variance and cos(q0, q_i) is about 1 / sqrt(1 + i sigma^2).  Returns
    [steps][B][H_q][d] in q0's dtype (computed in fp32)."""
    g = torch.Generator(device=q0.device).manual_seed(int(seed) * 104729 + 3)
    base = q0.float()
    walk = torch.zeros_like(base)
    out = []
    for i in range(1, steps + 1):
        walk += torch.randn(base.shape, generator=g, device=q0.device, dtype=torch.float32)
        out.append(((base + sigma * walk) / math.sqrt(1.0 + i * sigma * sigma)).to(q0.dtype))
    return torch.stack(out)
