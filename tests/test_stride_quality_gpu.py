"""One speculation stride chained on the HIP path against the oracle -- needs
an MI355X.

The chain (stride_quality.StrideRun): a verify over context L_r and its
PillarAttn lists; then, for every stride position i = 1..k, a draft query
drifting from the verify's last row, scored exactly over context L_r + i,
and the quality (coverage, recall@T) of the verify's lists and of a fresh
top-K of the draft row.  Every link is checked against the oracle on the
same inputs: the verify's lists and the fresh lists by the top-K band rule
on the oracle's averaged scores, each draft row's top-T by the same rule,
coverage within a tolerance, and recall as the exact overlap of the GPU's
top-T with the list."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import to_np
import parity
from sparse_self_speculative_pillarattn_amd import synth
from sparse_self_speculative_pillarattn_amd.stride_quality import StrideRun

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # H_q, H_kv, d, k, dtype, lengths, sigma
    (8, 2, 128, 4, "bf16", ("uniform", 60, 900), 0.3),
    (16, 4, 128, 8, "bf16", ("uniform", 300, 2500), 1.0),
    (4, 1, 64, 3, "f32", ("uniform", 20, 400), 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"h{c[0]}kv{c[1]}d{c[2]}k{c[3]}{c[4]}-s{c[6]}")
def test_stride_chain_matches_oracle(oracle, case):
    Hq, Hkv, d, k, dtype, lengths, sigma = case
    w = synth.Workload(name="stride", batch=3, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                       dtype=dtype, spec_k=k, sparsity=Fraction(1, 10), lengths=lengths, seed=91)
    b, vlens = synth.stride_batch(w, device=DEV)
    print(f"[stride] {case} verify lens={vlens}", flush=True)
    T = 10
    sr = StrideRun(b, vlens, sigma, seed=5, top_t=T)
    sr.verify()
    torch.cuda.synchronize()
    lists = to_np(sr.lists)
    scale = 1.0 / np.sqrt(d)
    G = Hq // Hkv
    inputs = [parity.request_inputs(b, r) for r in range(b.B)]
    # link 1: the verify's lists
    for r in range(b.B):
        qv, kp, vp, ptr = inputs[r]
        L, K = vlens[r], sr.K[r]
        lg, lse, _ = oracle.verify_request(qv, kp, vp, ptr, L, k, Hq, Hkv, scale)
        pbar = oracle.average(lg, lse, Hkv, 1, k)
        for g in range(Hkv):
            parity.assert_topk(lists[sr.ioff[r] + g * K: sr.ioff[r] + (g + 1) * K], pbar[g], K,
                               f"verify list req {r} head {g}")
    qd = to_np(sr.q_draft)
    for i in range(1, k + 1):
        loff = sr.score_draft(i)
        sr.quality(i, loff, sr.lists)
        torch.cuda.synchronize()
        got = {"pillar": (lists, to_np(sr.top), to_np(sr.cov), to_np(sr.rec))}
        sr.fresh_lists(i, loff)
        sr.quality(i, loff, sr.fresh)
        torch.cuda.synchronize()
        got["fresh"] = (to_np(sr.fresh), to_np(sr.top), to_np(sr.cov), to_np(sr.rec))
        for r in range(b.B):
            _, kp, vp, ptr = inputs[r]
            Ld, K = vlens[r] + i, sr.K[r]
            q2 = np.stack([qd[i - 1, r], qd[i - 1, r]])
            lg, lse, _ = oracle.verify_request(q2, kp, vp, ptr, Ld, 1, Hq, Hkv, scale)
            p = np.exp(np.where(np.isinf(lg[1]), -np.inf, lg[1] - lse[1][:, None]))
            for kind, (lst_all, top, cov, rec) in got.items():
                lst = lst_all[sr.ioff[r]: sr.ioff[r] + Hkv * K].reshape(Hkv, K)
                if kind == "fresh":
                    pbar = oracle.average(lg, lse, Hkv, 1, 1)
                    for g in range(Hkv):
                        parity.assert_topk(lst[g], pbar[g], K, f"fresh list i={i} req {r} head {g}")
                _, ocov, _ = oracle.list_quality(lg[1], lse[1], lst, T)
                for h in range(Hq):
                    what = f"{kind} i={i} req {r} head {h}"
                    assert abs(cov[r, h] - ocov[h]) <= 2e-3 + 2e-3 * abs(ocov[h]), \
                        (what, cov[r, h], ocov[h])
                    parity.assert_topk(top[r, h], p[h], T, f"top-{T} {what}")
                    members = {int(x) for x in lst[h // G]}
                    hits = sum(1 for x in top[r, h] if int(x) in members)
                    assert rec[r, h] == pytest.approx(hits / T, abs=1e-7), (what, rec[r, h], hits)


def test_stride_run_full_chain_shapes():
    """run() returns every stride position's pillar and fresh arrays, finite
    and in [0, 1]; a fresh list never covers less than the verify's list by
    more than rounding, on average over heads (it is the row's own top-K of
    the GQA-averaged scores)."""
    w = synth.Workload(name="stride-run", batch=4, num_qo_heads=16, num_kv_heads=8, head_dim=128,
                       dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                       lengths=("uniform", 1000, 3000), seed=92)
    b, vlens = synth.stride_batch(w, device=DEV)
    out = StrideRun(b, vlens, 0.5, seed=1).run()
    assert sorted(out) == list(range(1, 9))
    for i, res in out.items():
        for kind in ("pillar", "fresh"):
            cov, rec = (to_np(x) for x in res[kind])
            assert cov.shape == (4, 16) and np.isfinite(cov).all()
            assert (cov >= 0).all() and (cov <= 1 + 1e-4).all() and (rec >= 0).all() and (rec <= 1).all()
        assert to_np(res["fresh"][0]).mean() >= to_np(res["pillar"][0]).mean() - 1e-3
