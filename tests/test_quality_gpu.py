"""List quality (attention coverage and recall of the exact top-T) on the HIP
path against the oracle -- needs an MI355X.

A draft query is scored over its whole context by spa_verify_attn with spec_k
= 1 (the query in row 1, which sits at the last position), then
spa_list_quality measures index lists against that row.  The oracle runs its
own chain from the same seeded inputs: fp64 verify attention, then its list
quality.  Coverage is compared within a tolerance; the GPU's top-T must pass
the same band rule as PillarAttn's top-K, and its recall must equal the
overlap of that top-T with the list exactly."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import to_np
import parity
from sparse_self_speculative_pillarattn_amd import binding as bd
from sparse_self_speculative_pillarattn_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def score_drafts(b, reqs):
    """Row-1 logits and LSE of the draft queries of ``reqs`` (spec_k = 1): the
    tensors and host offsets spa_list_quality reads."""
    w = b.w
    Hq, Hkv, d = w.num_qo_heads, w.num_kv_heads, w.head_dim
    q2 = torch.stack([torch.stack([b.q[b.q_indptr[r]], b.q[b.q_indptr[r]]]) for r in reqs])
    q2 = q2.reshape(-1, Hq, d).contiguous()
    pt = torch.stack([b.page_table[r] for r in reqs]).contiguous()
    lens = [b.seq_lens[r] for r in reqs]
    loff = np.concatenate([[0], np.cumsum([2 * Hq * L for L in lens])[:-1]]).astype(np.int64)
    logits = torch.empty((int(sum(2 * Hq * L for L in lens)),), device=q2.device)
    lse = torch.empty((2 * len(reqs), Hq), device=q2.device)
    o = torch.empty_like(q2)
    lay = bd.layout(Hq, Hkv, d, b.q.dtype, b.num_slots, b.stride)
    ws = bd.workspace(bd.workspace_bytes(lay, len(reqs), 1, [1] * len(reqs), lens, [1] * len(reqs)),
                      q2.device)
    bd.verify_attn(lay, len(reqs), 1, lens, pt, q2, b.k_pool, b.v_pool, o, lse, logits, loff, ws)
    return lens, logits, loff, lse


def run_quality(b, reqs, lists, T):
    """lists: per request an int32 array [Hkv][n]; returns host top, coverage,
    recall and the scoring tensors."""
    w = b.w
    Hq, Hkv = w.num_qo_heads, w.num_kv_heads
    lens, logits, loff, lse = score_drafts(b, reqs)
    cnt = [a.shape[1] for a in lists]
    coff = np.concatenate([[0], np.cumsum([Hkv * c for c in cnt])[:-1]]).astype(np.int64)
    flat = np.concatenate([a.reshape(-1) for a in lists] + [np.zeros(1, np.int32)])
    dl = torch.from_numpy(flat.astype(np.int32)).to(logits.device)
    nb = len(reqs)
    top = torch.full((nb, Hq, T), -7, dtype=torch.int32, device=logits.device)
    cov = torch.full((nb, Hq), float("nan"), device=logits.device)
    rec = torch.full((nb, Hq), float("nan"), device=logits.device)
    ws = bd.workspace(bd.list_quality_workspace_bytes(nb, Hq, lens), logits.device)
    print(f"[quality] {w.name} T={T} lens={lens} lists={cnt}", flush=True)
    bd.list_quality(nb, 1, Hq, Hkv, 1, T, lens, logits, loff, lse, cnt, coff, dl, top, cov, rec, ws)
    torch.cuda.synchronize()
    return to_np(top), to_np(cov), to_np(rec)


def check_request(oracle, b, r, lst, T, top, cov, rec):
    """One request against the oracle's own chain."""
    w = b.w
    Hq, Hkv = w.num_qo_heads, w.num_kv_heads
    G = Hq // Hkv
    L = b.seq_lens[r]
    qh, kp, vp, ptr = parity.request_inputs(b, r)
    q2 = np.stack([qh[0], qh[0]])
    lg, lse, _ = oracle.verify_request(q2, kp, vp, ptr, L, 1, Hq, Hkv, 1.0 / np.sqrt(w.head_dim))
    _, ocov, _ = oracle.list_quality(lg[1], lse[1], lst, T)
    p = np.exp(np.where(np.isinf(lg[1]), -np.inf, lg[1] - lse[1][:, None]))
    for h in range(Hq):
        g = h // G
        assert abs(cov[h] - ocov[h]) <= 2e-3 + 2e-3 * abs(ocov[h]), (r, h, cov[h], ocov[h])
        parity.assert_topk(top[h], p[h], T, f"top-{T} req {r} head {h}")
        members = {int(x) for x in lst[g] if 0 <= x < L}
        hits = sum(1 for x in top[h] if int(x) in members)
        assert rec[h] == pytest.approx(hits / T, abs=1e-7), (r, h, rec[h], hits)


def _lists(rng, L, Hkv, kind):
    if kind == "random":   # repeats and entries outside [0, L)
        a = rng.integers(-3, L + 4, size=(Hkv, max(4, L // 10))).astype(np.int32)
        a[:, 1] = a[:, 0]
        return a
    if kind == "all":
        return np.tile(np.arange(L, dtype=np.int32), (Hkv, 1))
    if kind == "none":
        return np.full((Hkv, 3), -1, np.int32)
    if kind == "empty":
        return np.zeros((Hkv, 0), np.int32)
    raise ValueError(kind)


@pytest.mark.parametrize("T,dtype", [(1, "bf16"), (10, "bf16"), (64, "bf16"), (10, "f32")])
def test_list_quality_matches_oracle(oracle, T, dtype):
    w = synth.Workload(name=f"quality-{T}-{dtype}", batch=6, num_qo_heads=16, num_kv_heads=4,
                       head_dim=128, dtype=dtype, spec_k=8, sparsity=Fraction(1, 20),
                       lengths=("uniform", 70, 2500), n_verify=0, seed=40 + T)
    b = synth.make_batch(w, is_verify=[False] * 6)
    bd_ = b.to(DEV)
    rng = np.random.default_rng(T)
    kinds = ["stored", "random", "all", "none", "empty", "stored"]
    lists = []
    for r, kind in enumerate(kinds):
        if kind == "stored":   # the seeded draft list (pillars plus fill)
            K = b.idx_count[r]
            lists.append(to_np(b.idx[b.idx_off[r]:b.idx_off[r] + w.num_kv_heads * K]).reshape(-1, K))
        else:
            lists.append(_lists(rng, b.seq_lens[r], w.num_kv_heads, kind))
    reqs = list(range(b.B))
    top, cov, rec = run_quality(bd_, reqs, lists, T)
    for r in reqs:
        check_request(oracle, b, r, lists[r], T, top[r], cov[r], rec[r])


def test_list_quality_edge_lengths(oracle):
    """The shortest context the scoring allows (L = 2), T = L, and a context
    longer than one selection pass holds in registers (L > 8192)."""
    w = synth.Workload(name="quality-edge", batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=64,
                       dtype="bf16", spec_k=8, sparsity=Fraction(1, 20), lengths=("fixed", 2),
                       n_verify=0, seed=77)
    for L, T in ((2, 2), (2, 1), (9000, 10)):
        b = synth.make_batch(w, is_verify=[False] * 3, seq_lens=[L] * 3)
        bd_ = b.to(DEV)
        rng = np.random.default_rng(L)
        lists = [_lists(rng, L, 2, "random"), _lists(rng, L, 2, "all"),
                 np.stack([np.sort(rng.choice(L, min(L, 5), replace=False))] * 2).astype(np.int32)]
        top, cov, rec = run_quality(bd_, [0, 1, 2], lists, T)
        for r in range(3):
            check_request(oracle, b, r, lists[r], T, top[r], cov[r], rec[r])


def test_list_quality_full_size_sampled(oracle):
    """All 114 drafts of the Qwen3-8B-shaped batch (L = 8192) scored against
    their stored lists: three drafts against the oracle, and every request's
    coverage in [0, 1], recall in [0, 1], top-10 ascending and in range."""
    w = synth.QWEN3_8B
    print(f"[full-size quality] {w.name}", flush=True)
    b = synth.make_batch(w, device=DEV)
    dra = [r for r in range(b.B) if not b.is_verify[r]]
    Hkv = w.num_kv_heads
    lists = [to_np(b.idx[b.idx_off[r]:b.idx_off[r] + Hkv * b.idx_count[r]]).reshape(Hkv, -1)
             for r in dra]
    top, cov, rec = run_quality(b, dra, lists, 10)
    assert np.isfinite(cov).all() and (cov >= 0).all() and (cov <= 1 + 1e-4).all()
    assert ((rec >= 0) & (rec <= 1)).all()
    assert (np.diff(top, axis=2) > 0).all() and top.min() >= 0 and top.max() < 8192
    for i in sorted({0, len(dra) // 2, len(dra) - 1}):
        check_request(oracle, b, dra[i], lists[i], 10, top[i], cov[i], rec[i])
    del b
    torch.cuda.empty_cache()
