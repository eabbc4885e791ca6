"""The scheduler of include/spa_sched.h on the CPU: the invariants that the
review of SparseSpec (核心方法 / "Unified batch scheduler", "Delayed
verification") and the acceptance process fix, over hundreds of steps.

- Buckets: every new request joins the emptiest one, so bucket sizes stay
  within one of each other, and each step's verify count is floor or ceil of
  slots / C (C = k+1, or k+2 with delayed verification).
- Rows: a step's query rows are drafts + (k+1) verifies; without delay their
  mean is the page's (2k+1)/(k+1) slots.
- Phases: a request drafts k times (contexts c+1 .. c+k), then (delayed)
  sits out one step, then verifies with context c+k+1; the verify commits
  a+1 tokens, 0 <= a <= k.
- Acceptance: a is the leading run of independent draws accepted with
  probability p, whose mean is p (1 - p^k) / (1 - p) (6.16 of 8 at the
  default p).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from sparse_self_speculative_pillarattn_amd import binding as bd


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(bd.LIB_PATH):
        from sparse_self_speculative_pillarattn_amd import build
        build.build()
    return bd.load()


def sched(slots=128, k=8, delayed=False, prompt=(2000, 8000), output=(200, 2000), p=None,
          seed=3, s=Fraction(1, 20), Hq=32, Hkv=8):
    return bd.Scheduler(slots, k, Hq, Hkv, s, prompt, output, prompt[1] + output[1] + k + 1,
                        delayed=delayed, accept_prob=bd.ACCEPT_PROB_6_16_OF_8 if p is None else p,
                        seed=seed)


@pytest.mark.parametrize("delayed", [False, True])
@pytest.mark.parametrize("slots,k", [(128, 8), (256, 12), (16, 3), (7, 1)])
def test_verify_count_and_rows_per_step(slots, k, delayed):
    sc = sched(slots, k, delayed, output=(20, 200))
    C = k + 1 + int(delayed)
    lo, hi = slots // C, -(-slots // C)
    rows = []
    for _ in range(400):
        st = sc.next()
        assert lo <= st.n_verify <= hi, (st.step, st.n_verify)
        assert st.n_waiting == 0 if not delayed else lo <= st.n_waiting <= hi
        assert st.B == st.n_verify + st.n_draft
        assert st.B + st.n_waiting == slots
        assert st.rows == st.n_draft + (k + 1) * st.n_verify
        a = sc.arrays(st)
        assert int(a["is_verify"].sum()) == st.n_verify
        assert np.array_equal(np.diff(a["q_indptr"]), np.where(a["is_verify"] == 1, k + 1, 1))
        b = sc.buckets()
        assert b.max() - b.min() <= 1 and b.sum() == slots
        rows.append(st.rows)
        sc.commit()
    if not delayed:
        assert abs(np.mean(rows) - (2 * k + 1) / (k + 1) * slots) <= k
    assert sc.stats()["retired"] > 0  # requests came and went


def _trace(sc, n_steps, slots):
    """Per slot, per step: ("D"|"V"|"W", context or None)."""
    roles = {s: [] for s in range(slots)}
    for _ in range(n_steps):
        st = sc.next()
        a = sc.arrays(st)
        present = dict(zip(a["slot"].tolist(), zip(a["is_verify"].tolist(), a["seq_lens"].tolist())))
        for s in range(slots):
            v = present.get(s)
            roles[s].append(("W", None) if v is None else ("V" if v[0] else "D", v[1]))
        sc.commit()
    return roles


@pytest.mark.parametrize("delayed", [False, True])
def test_phases_and_context_lengths(delayed):
    """Long outputs (no request retires in the window): each slot's roles repeat
    with the cycle D..D V (W), drafts extend the context one position at a
    time, the verify's context is the last draft's + 1, and the next draft
    after a verify starts 1..k+1 positions further (a + 1 committed)."""
    k, S = 4, 12
    sc = sched(S, k, delayed, output=(5000, 5000))
    C = k + 1 + int(delayed)
    cycle = "D" * k + "V" + ("W" if delayed else "")
    tr = _trace(sc, 6 * C, S)
    for s in range(S):
        seq = "".join(r for r, _ in tr[s])
        L = [x for _, x in tr[s]]
        assert all(seq[t] == seq[t - C] for t in range(C, len(seq)))
        assert seq[:C] in [cycle[i:] + cycle[:i] for i in range(C)]
        for t in range(1, len(seq)):
            if seq[t] == "D" and seq[t - 1] == "D":
                assert L[t] == L[t - 1] + 1
            if seq[t] == "V" and seq[t - 1] == "D":
                assert L[t] == L[t - 1] + 1
            tv = t - 1 - int(delayed)
            if seq[t] == "D" and tv >= 0 and seq[tv] == "V":
                grown = L[t] - 1 - (L[tv] - k - 1)  # new committed length - old
                assert 1 <= grown <= k + 1


@pytest.mark.parametrize("delayed", [False, True])
def test_new_request_joins_its_bucket_mid_cycle(delayed):
    """A request admitted into a bucket at any phase is first issued with
    context P + 1 (P its prompt) and first verifies k+1 rows ending at most k
    drafts past P."""
    k, S = 5, 20
    sc = sched(S, k, delayed, output=(3, 9), prompt=(50, 90))
    pending, first_seen = {}, 0
    verified = 0
    for _ in range(300):
        st = sc.next()
        a = sc.arrays(st)
        for s, P in zip(a["new_slots"].tolist(), a["new_len"].tolist()):
            pending[s] = [P, False]
        present = dict(zip(a["slot"].tolist(), zip(a["is_verify"].tolist(), a["seq_lens"].tolist())))
        for s, rec in list(pending.items()):
            if s not in present:
                continue
            v, L = present[s]
            if not rec[1]:
                assert L == rec[0] + 1, (s, L, rec[0])
                rec[1] = True
                first_seen += 1
            if v:
                assert rec[0] + 1 <= L <= rec[0] + k + 1
                verified += 1
                del pending[s]
        sc.commit()
    assert first_seen > 50 and verified > 50


def test_verify_lists_hold_ceil_s_l():
    sc = sched(64, 8, False, s=Fraction(1, 20))
    for _ in range(50):
        st = sc.next()
        a = sc.arrays(st)
        for v, L, K in zip(a["is_verify"], a["seq_lens"], a["idx_count"]):
            if v:
                assert K == -((-int(L)) // 20)
        sc.commit()


@pytest.mark.parametrize("p,k", [(bd.ACCEPT_PROB_6_16_OF_8, 8), (0.7, 5), (0.0, 8), (1.0, 8)])
def test_mean_accepted_follows_the_leading_run_law(p, k):
    """After every slot's first (possibly shortened) cycle, each verify checks
    k drafts and accepts their leading run of Bernoulli(p) draws."""
    sc = sched(256, k, False, output=(10**6, 10**6), prompt=(100, 100), p=p)
    for _ in range(k + 1):
        sc.next()
        sc.commit()
    s0 = sc.stats()
    while sc.stats()["verifies"] - s0["verifies"] < 20000:
        sc.next()
        sc.commit()
    s1 = sc.stats()
    n = s1["verifies"] - s0["verifies"]
    assert s1["drafted"] - s0["drafted"] == k * n
    assert s1["committed"] - s0["committed"] == s1["accepted"] - s0["accepted"] + n
    mean = (s1["accepted"] - s0["accepted"]) / n
    want = k if p == 1.0 else p * (1 - p ** k) / (1 - p)
    if p in (0.0, 1.0):
        assert mean == want
        return
    # a leading run of at most k has standard deviation below k / 2
    assert abs(mean - want) <= 4 * (k / 2) / math.sqrt(n), (mean, want)
    if k == 8 and p == bd.ACCEPT_PROB_6_16_OF_8:
        assert abs(want - 6.16) < 1e-6


def test_seeded_and_deterministic():
    def run(seed):
        sc = sched(32, 4, True, output=(10, 50), seed=seed)
        out = []
        for _ in range(60):
            st = sc.next()
            a = sc.arrays(st)
            out.append((a["slot"].tolist(), a["seq_lens"].tolist(), a["is_verify"].tolist()))
            sc.commit()
        return out
    assert run(5) == run(5)
    assert run(5) != run(6)


def test_capacity_bounds_every_step():
    sc = sched(64, 8, False, output=(10, 400))
    for _ in range(300):
        st = sc.next()
        a = sc.arrays(st)
        assert st.rows <= sc.max_rows
        assert st.logits_elems <= sc.logits_elems
        ends = a["idx_off"] + 8 * a["idx_count"].astype(np.int64)
        assert ends.max() <= sc.idx_elems
        # a slot's list segment is its own
        assert len(set(a["slot"].tolist())) == st.B
        sc.commit()


def test_new_requests_are_reported_once():
    sc = sched(16, 3, False, output=(2, 6))
    st = sc.next()
    assert st.n_new == 16  # every slot starts with a new request
    sc.commit()
    seen = 0
    for _ in range(100):
        st = sc.next()
        a = sc.arrays(st)
        seen += st.n_new
        assert np.all(a["new_count"] == -((-a["new_len"]) // 20))
        assert len(set(a["new_slots"].tolist())) == st.n_new
        sc.commit()
    seen += sc.next().n_new
    # each retirement brings one new request, reported at the following step
    assert seen == sc.stats()["retired"] > 0


@pytest.mark.parametrize("kw", [dict(slots=0), dict(k=0), dict(prompt=(8, 10)),
                                dict(output=(5, 4)), dict(p=1.5), dict(s=Fraction(3, 2))])
def test_invalid_configs_are_rejected(kw):
    with pytest.raises(bd.SpaError):
        sched(**kw)
