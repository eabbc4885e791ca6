"""Comparison helpers: HIP outputs against the oracle, element by element.

Tolerances (floating point):
  O, bf16 outputs   |o - o_ref| <= 2e-2 + 2e-2 |o_ref|
  O, fp32 outputs   |o - o_ref| <= 1e-4 + 1e-4 |o_ref|
  LSE               |x - x_ref| <= 1e-3 |x_ref| + 1e-6 (relative; the 1e-6 is the fp32
                    resolution of a sum near 1, for an LSE near 0)
  logits            |x - x_ref| <= 1e-3 max(1, |x_ref|) (a logit is a scaled dot product
                    whose rounding error scales with |q| |k|, not with the logit)
  both              -inf exactly where the oracle has -inf
Top-K (an index set decided by floating point): with tau the oracle's K-th
largest averaged score, every position scoring above tau (1 + 1e-3) must be
selected and none scoring below tau (1 - 1e-3); the list holds K distinct
in-range positions, ascending.  Positions inside the band may go either way.
"""
from __future__ import annotations

import numpy as np
import torch

from conftest import to_np, widen

O_TOL = {"bf16": (2e-2, 2e-2), "f32": (1e-4, 1e-4)}
LSE_REL = 1e-3
LSE_ABS = 1e-6
TOPK_BAND = 1e-3


def oracle_inputs(b, avg_row_begin=1, avg_row_count=None):
    return dict(k=b.w.spec_k, Hq=b.w.num_qo_heads, Hkv=b.w.num_kv_heads,
                sm_scale=1.0 / np.sqrt(b.w.head_dim), is_verify=b.is_verify,
                seq_lens=b.seq_lens, q_indptr=b.q_indptr, page_table=to_np(b.page_table),
                q=to_np(b.q), k_pool=to_np(b.k_pool), v_pool=to_np(b.v_pool),
                idx_count=b.idx_count, idx_off=b.idx_off, idx=to_np(b.idx),
                logits_off=b.logits_off, logits_elems=b.logits_elems,
                row_begin=avg_row_begin,
                row_count=b.w.spec_k if avg_row_count is None else avg_row_count)


def oracle_inputs_compact(b, avg_row_begin=1, avg_row_count=None):
    """oracle_inputs over host copies of exactly the pool rows the requests
    read, re-laid-out in page-table order (results do not depend on where a
    slot lives), for batches whose pools are too large to copy whole."""
    lens = b.seq_lens
    flat = torch.cat([b.page_table[r, :lens[r]].long() for r in range(b.B)])
    pt = np.zeros((b.B, max(lens)), np.int32)
    off = 0
    for r in range(b.B):
        pt[r, :lens[r]] = np.arange(off, off + lens[r], dtype=np.int32)
        off += lens[r]
    d = oracle_inputs_meta(b, avg_row_begin, avg_row_count)
    d.update(page_table=pt, q=to_np(b.q), k_pool=to_np(b.k_pool.index_select(0, flat)),
             v_pool=to_np(b.v_pool.index_select(0, flat)), idx=to_np(b.idx))
    return d


def oracle_inputs_meta(b, avg_row_begin=1, avg_row_count=None):
    return dict(k=b.w.spec_k, Hq=b.w.num_qo_heads, Hkv=b.w.num_kv_heads,
                sm_scale=1.0 / np.sqrt(b.w.head_dim), is_verify=b.is_verify,
                seq_lens=b.seq_lens, q_indptr=b.q_indptr, idx_count=b.idx_count,
                idx_off=b.idx_off, logits_off=b.logits_off, logits_elems=b.logits_elems,
                row_begin=avg_row_begin,
                row_count=b.w.spec_k if avg_row_count is None else avg_row_count)


def assert_o(got, ref, dtype, what="O"):
    atol, rtol = O_TOL[dtype]
    got = widen(got) if got.dtype == np.uint16 else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)} got {got[tuple(i)]} want {ref[tuple(i)]}; "
                             f"max err {err[~np.isnan(err)].max() if (~np.isnan(err)).any() else 'nan'}")


def assert_lse(got, ref, what="LSE"):
    _assert_close_ninf(got, ref, what, floor=False)


def assert_logits(got, ref, what="logits"):
    _assert_close_ninf(got, ref, what, floor=True)


def _assert_close_ninf(got, ref, what, floor):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    ninf_ref = np.isneginf(ref)
    ninf_got = np.isneginf(got)
    if not np.array_equal(ninf_ref, ninf_got):
        i = np.argwhere(ninf_ref != ninf_got)[0]
        raise AssertionError(f"{what}: -inf pattern differs at {tuple(i)}: got {got[tuple(i)]} "
                             f"want {ref[tuple(i)]}")
    f = ~ninf_ref
    err = np.abs(got[f] - ref[f])
    a = np.abs(ref[f])
    bad = ~(err <= (LSE_REL * np.maximum(1.0, a) if floor else LSE_REL * a + LSE_ABS))
    if bad.any():
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance, max err "
                             f"{np.nanmax(err)}")


def assert_topk(sel, pbar_ref, K, what="top-K"):
    sel = np.asarray(sel)
    L = pbar_ref.shape[0]
    assert sel.shape == (K,), (what, sel.shape, K)
    assert np.all(np.diff(sel) > 0), f"{what}: not strictly ascending"
    assert sel.min() >= 0 and sel.max() < L, f"{what}: out of range"
    tau = np.sort(pbar_ref)[::-1][K - 1]
    must = np.nonzero(pbar_ref > tau * (1 + TOPK_BAND))[0]
    never = set(np.nonzero(pbar_ref < tau * (1 - TOPK_BAND))[0].tolist())
    s = set(sel.tolist())
    missing = [j for j in must if j not in s]
    assert not missing, f"{what}: {len(missing)} clear top-K positions missing, e.g. {missing[:5]}"
    wrong = s & never
    assert not wrong, f"{what}: {len(wrong)} clearly-low positions selected, e.g. {sorted(wrong)[:5]}"


def oracle_pbar(orc, ref_logits, ref_lse, b, r, avg_row_begin=1, avg_row_count=None):
    """Oracle averaged scores [H_kv][L] of verify request r from oracle logits/LSE."""
    w = b.w
    k, Hq, L = w.spec_k, w.num_qo_heads, b.seq_lens[r]
    off = b.logits_off[r]
    lg = ref_logits[off:off + (k + 1) * Hq * L].reshape(k + 1, Hq, L)
    r0 = b.q_indptr[r]
    lse = ref_lse[r0:r0 + k + 1]
    n = k if avg_row_count is None else avg_row_count
    return orc.average(lg, lse, w.num_kv_heads, avg_row_begin, n)


def compare_step(orc, b, gpu, ref, avg_row_begin=1, avg_row_count=None, check_logits=True):
    """gpu: dict of tensors (o, lse, logits, idx) after the unified step; ref: oracle.step()."""
    w = b.w
    o = to_np(gpu["o"])
    assert_o(o, ref["o"], w.dtype)
    assert_lse(to_np(gpu["lse"]), ref["lse"])
    idx = to_np(gpu["idx"])
    logits = to_np(gpu["logits"]) if check_logits else None
    for r in range(b.B):
        if not b.is_verify[r]:
            seg = slice(b.idx_off[r], b.idx_off[r] + w.num_kv_heads * b.idx_count[r])
            assert np.array_equal(idx[seg], to_np(b.idx)[seg]), f"draft list {r} was modified"
            continue
        L, k, Hq = b.seq_lens[r], w.spec_k, w.num_qo_heads
        if check_logits:
            off = b.logits_off[r]
            n = (k + 1) * Hq * L
            assert_logits(logits[off:off + n], ref["logits"][off:off + n], f"logits req {r}")
        pbar = oracle_pbar(orc, ref["logits"], ref["lse"], b, r, avg_row_begin, avg_row_count)
        K = b.idx_count[r]
        for g in range(w.num_kv_heads):
            sel = idx[b.idx_off[r] + g * K: b.idx_off[r] + (g + 1) * K]
            assert_topk(sel, pbar[g], K, f"top-K req {r} head {g}")


def request_inputs(b, r):
    """Host copies of what request r reads: its q rows and the K/V pool rows of
    its L positions, re-laid-out in position order (so its page table becomes
    0..L-1; results do not depend on where a slot lives)."""
    L = b.seq_lens[r]
    slots = b.page_table[r, :L].long()
    kp = to_np(b.k_pool.index_select(0, slots))
    vp = to_np(b.v_pool.index_select(0, slots))
    rows = slice(b.q_indptr[r], b.q_indptr[r + 1])
    return to_np(b.q[rows]), kp, vp, np.arange(L, dtype=np.int32)


def compare_sampled(orc, b, gpu, verify_reqs, draft_reqs):
    """Full-size check of chosen requests against the oracle, one request at a
    time: verify O, LSE, every dumped logit and the per-KV-head top-K; draft O
    and LSE.  gpu: dict of tensors (o, lse, logits, idx) after the step."""
    w = b.w
    k, Hq, Hkv, d = w.spec_k, w.num_qo_heads, w.num_kv_heads, w.head_dim
    sm = 1.0 / np.sqrt(d)
    for r in verify_reqs:
        assert b.is_verify[r]
        L = b.seq_lens[r]
        q, kp, vp, ptr = request_inputs(b, r)
        lg, lse, o = orc.verify_request(q, kp, vp, ptr, L, k, Hq, Hkv, sm)
        rows = slice(b.q_indptr[r], b.q_indptr[r + 1])
        assert_o(to_np(gpu["o"][rows]), o, w.dtype, f"O req {r}")
        assert_lse(to_np(gpu["lse"][rows]), lse, f"LSE req {r}")
        off, n = b.logits_off[r], (k + 1) * Hq * L
        assert_logits(to_np(gpu["logits"][off:off + n]), lg.reshape(-1), f"logits req {r}")
        pbar = orc.average(lg, lse, Hkv, 1, k)
        K = b.idx_count[r]
        idx = to_np(gpu["idx"][b.idx_off[r]:b.idx_off[r] + Hkv * K]).reshape(Hkv, K)
        for g in range(Hkv):
            assert_topk(idx[g], pbar[g], K, f"top-K req {r} head {g}")
    for r in draft_reqs:
        assert not b.is_verify[r]
        L, K = b.seq_lens[r], b.idx_count[r]
        q, kp, vp, ptr = request_inputs(b, r)
        lst = to_np(b.idx[b.idx_off[r]:b.idx_off[r] + Hkv * K]).reshape(Hkv, K)
        o, lse = orc.draft_request(q[0], kp, vp, ptr, L, lst, Hkv, sm)
        row = b.q_indptr[r]
        assert_o(to_np(gpu["o"][row]), o, w.dtype, f"O draft {r}")
        assert_lse(to_np(gpu["lse"][row]), lse, f"LSE draft {r}")


def check_whole_batch_properties(b, gpu):
    """Properties that hold at any size, for every request: finite LSE and O,
    each verify row's causally hidden logits exactly -inf, and every top-K list
    K distinct in-range positions, ascending."""
    w = b.w
    k, Hq, Hkv = w.spec_k, w.num_qo_heads, w.num_kv_heads
    lse = to_np(gpu["lse"])
    assert np.isfinite(lse).all(), "non-finite LSE"
    o = gpu["o"].float()
    assert bool(torch.isfinite(o).all()), "non-finite O"
    idx = to_np(gpu["idx"])
    logits = gpu["logits"]
    for r in range(b.B):
        if not b.is_verify[r]:
            continue
        L, K = b.seq_lens[r], b.idx_count[r]
        lst = idx[b.idx_off[r]:b.idx_off[r] + Hkv * K].reshape(Hkv, K)
        assert (np.diff(lst, axis=1) > 0).all(), f"top-K req {r} not strictly ascending"
        assert lst.min() >= 0 and lst.max() < L, f"top-K req {r} out of range"
        lg = logits[b.logits_off[r]:b.logits_off[r] + (k + 1) * Hq * L].view(k + 1, Hq, L)
        for i in range(k):  # row i hides the last k - i positions
            tail = lg[i, :, L - k + i:]
            assert bool(torch.isneginf(tail).all()), f"req {r} row {i}: hidden logits not -inf"
            assert bool(torch.isfinite(lg[i, :, :L - k + i]).all()), f"req {r} row {i}: non-finite logits"
