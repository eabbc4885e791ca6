"""Pins of the C oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:
  * an independent library routine on a special case (PyTorch CPU
    scaled_dot_product_attention / softmax / logsumexp / topk in float64);
  * a closed form (uniform keys, one key, two keys, duplicate entries);
  * an invariant of the definitions (softmax rows sum to one, averaged
    scores sum to one, masked logits are exactly -inf, permutation and
    masking invariance of the draft list);
  * brute-force enumeration on tiny inputs (top-K with ties).

test_oracle_pins.py runs them on the real oracle; test_oracle_mutants.py runs
them on builds with one planted mistake each and requires that some pin fails.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch
import torch.nn.functional as F

TOL = 1e-10


def _case(seed, Hq=4, Hkv=2, d=16, L=23, k=4, nslots=64, dtype=np.float32):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((k + 1, Hq, d)).astype(np.float32)
    kp = rng.standard_normal((nslots, Hkv, d)).astype(np.float32)
    vp = rng.standard_normal((nslots, Hkv, d)).astype(np.float32)
    pt = rng.permutation(nslots)[:L].astype(np.int32)
    return q, kp, vp, pt


def _gather(pool, pt, upto, g):
    """K or V rows of KV head g for positions [0, upto) as float64 torch."""
    return torch.from_numpy(pool[pt[:upto], g].astype(np.float64))


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
        bad = ~(err <= tol * (1.0 + np.abs(np.where(both_inf, 0.0, b))))  # NaN counts as bad
    assert not bad.any(), f"{what}: max err {err.max():.3e}"


# --------------------------------------------------------------------------- #
# full attention of the verify rows
# --------------------------------------------------------------------------- #
def pin_verify_vs_sdpa(orc):
    """Row i of a verify request equals single-query attention over the first
    L-(k+1)+i+1 positions (PyTorch SDPA, float64, GQA by explicit head map)."""
    Hq, Hkv, d, L, k = 4, 2, 16, 23, 4
    G = Hq // Hkv
    q, kp, vp, pt = _case(1, Hq, Hkv, d, L, k)
    scale = 1.0 / math.sqrt(d)
    logits, lse, o = orc.verify_request(q, kp, vp, pt, L, k, Hq, Hkv, scale)
    for i in range(k + 1):
        n = L - (k + 1) + i + 1
        for h in range(Hq):
            g = h // G
            Kt = _gather(kp, pt, n, g)
            Vt = _gather(vp, pt, n, g)
            qt = torch.from_numpy(q[i, h].astype(np.float64))
            ref_o = F.scaled_dot_product_attention(qt[None, None, None], Kt[None, None],
                                                   Vt[None, None], scale=scale)[0, 0, 0]
            s = torch.matmul(Kt, qt) * scale
            ref_lse = torch.logsumexp(s, 0)
            _close(o[i, h], ref_o.numpy(), 1e-12, f"O row {i} head {h}")
            _close(lse[i, h], ref_lse.item(), 1e-12, f"LSE row {i} head {h}")
            _close(logits[i, h, :n], s.numpy(), 1e-12, f"logits row {i} head {h}")


def pin_uniform_keys(orc):
    """All keys equal -> uniform weights: O = mean of visible V rows,
    LSE = l0 + ln(#visible)."""
    Hq, Hkv, d, L, k = 4, 2, 8, 17, 3
    G = Hq // Hkv
    q, kp, vp, pt = _case(2, Hq, Hkv, d, L, k)
    kp[:] = kp[0:1]          # every slot holds the same key per head
    scale = 0.37
    logits, lse, o = orc.verify_request(q, kp, vp, pt, L, k, Hq, Hkv, scale)
    for i in range(k + 1):
        n = L - (k + 1) + i + 1
        for h in range(Hq):
            g = h // G
            l0 = scale * float(np.dot(q[i, h].astype(np.float64), kp[0, g].astype(np.float64)))
            _close(lse[i, h], l0 + math.log(n), 1e-12, "uniform LSE")
            _close(o[i, h], vp[pt[:n], g].astype(np.float64).mean(0), 1e-12, "uniform O")


def pin_one_and_two_keys(orc):
    """L = k+1: row 0 sees one key (O = V_0, LSE = l_0); row 1 sees two
    (weights sigma(l_0 - l_1), sigma(l_1 - l_0))."""
    Hq, Hkv, d, k = 2, 1, 8, 3
    L = k + 1
    q, kp, vp, pt = _case(3, Hq, Hkv, d, L, k)
    scale = 0.5
    logits, lse, o = orc.verify_request(q, kp, vp, pt, L, k, Hq, Hkv, scale)
    for h in range(Hq):
        l0 = scale * float(np.dot(q[0, h].astype(np.float64), kp[pt[0], 0].astype(np.float64)))
        _close(lse[0, h], l0, 1e-12, "one key LSE")
        _close(o[0, h], vp[pt[0], 0], 1e-12, "one key O")
        a0 = scale * float(np.dot(q[1, h].astype(np.float64), kp[pt[0], 0].astype(np.float64)))
        a1 = scale * float(np.dot(q[1, h].astype(np.float64), kp[pt[1], 0].astype(np.float64)))
        w0 = 1.0 / (1.0 + math.exp(a1 - a0))
        v0 = vp[pt[0], 0].astype(np.float64)
        v1 = vp[pt[1], 0].astype(np.float64)
        _close(o[1, h], w0 * v0 + (1 - w0) * v1, 1e-12, "two keys O")
        _close(lse[1, h], max(a0, a1) + math.log1p(math.exp(-abs(a0 - a1))), 1e-12,
               "two keys LSE")


def pin_dump_consistency(orc):
    """exp(logit - LSE) over visible positions sums to one for every row; the
    positions after row i's own are exactly -inf (k - i of them)."""
    Hq, Hkv, d, L, k = 6, 3, 16, 40, 6
    q, kp, vp, pt = _case(4, Hq, Hkv, d, L, k)
    logits, lse, o = orc.verify_request(q, kp, vp, pt, L, k, Hq, Hkv, 0.25)
    for i in range(k + 1):
        last = L - (k + 1) + i
        assert np.all(np.isneginf(logits[i, :, last + 1:])), "hidden logits must be -inf"
        assert np.all(np.isfinite(logits[i, :, :last + 1])), "visible logits must be finite"
        s = np.exp(logits[i] - lse[i][:, None]).sum(axis=1)
        _close(s, np.ones(Hq), 1e-12, "softmax sum")


# --------------------------------------------------------------------------- #
# averaging
# --------------------------------------------------------------------------- #
def pin_average(orc):
    """Averaged scores: rows sum to one per KV head; with one row they equal
    PyTorch's softmax of that row averaged over the group's heads; the k-row
    average is the mean of the single-row averages."""
    Hq, Hkv, d, L, k = 6, 2, 16, 30, 4
    G = Hq // Hkv
    q, kp, vp, pt = _case(5, Hq, Hkv, d, L, k)
    scale = 1.0 / math.sqrt(d)
    logits, lse, o = orc.verify_request(q, kp, vp, pt, L, k, Hq, Hkv, scale)
    pbar = orc.average(logits, lse, Hkv, 1, k)
    _close(pbar.sum(axis=1), np.ones(Hkv), 1e-12, "pbar sum")
    singles = []
    for i in range(1, k + 1):
        p1 = orc.average(logits, lse, Hkv, i, 1)
        n = L - (k + 1) + i + 1
        for g in range(Hkv):
            ref = np.zeros(L)
            Kt = _gather(kp, pt, n, g)
            for hh in range(G):
                h = g * G + hh
                qt = torch.from_numpy(q[i, h].astype(np.float64))
                ref[:n] += torch.softmax(torch.matmul(Kt, qt) * scale, 0).numpy()
            _close(p1[g], ref / G, 1e-12, f"single-row average row {i}")
        singles.append(p1)
    _close(pbar, np.mean(singles, axis=0), 1e-12, "average linearity")


# --------------------------------------------------------------------------- #
# top-K
# --------------------------------------------------------------------------- #
def _brute_topk(scores, K):
    best = None
    for comb in itertools.combinations(range(len(scores)), K):
        tot = sum(scores[j] for j in comb)
        key = (-tot, comb)           # integer scores: exact sums
        if best is None or key < best:
            best = key
    return list(best[1])


def pin_topk_bruteforce(orc):
    """Tiny integer score vectors with ties: the chosen set is the max-sum
    K-subset, ties going to lower positions; output ascending."""
    rng = np.random.default_rng(6)
    for L in range(1, 10):
        for K in range(1, L + 1):
            for _ in range(3):
                s = rng.integers(0, 4, size=L).astype(np.float64)
                got = orc.topk(s, K).tolist()
                assert got == _brute_topk(s.tolist(), K), (L, K, s, got)


def pin_topk_vs_torch(orc):
    """Distinct scores: same set as torch.topk, returned ascending."""
    rng = np.random.default_rng(7)
    for L, K in [(1000, 50), (257, 13), (64, 64), (5, 1)]:
        s = rng.permutation(L).astype(np.float64) / L + rng.random(L) * 1e-6
        ref = torch.topk(torch.from_numpy(s), K).indices.sort().values.numpy()
        got = orc.topk(s, K)
        assert np.array_equal(got, ref), (L, K)


def pin_topk_special(orc):
    """K = L returns every position; equal scores return the first K."""
    for L in (1, 7, 100):
        assert orc.topk(np.random.default_rng(L).random(L), L).tolist() == list(range(L))
    assert orc.topk(np.full(50, 0.02), 13).tolist() == list(range(13))


# --------------------------------------------------------------------------- #
# sparse draft attention
# --------------------------------------------------------------------------- #
def pin_draft_full_list(orc):
    """A list holding every position equals dense single-query attention
    (SDPA float64) and logsumexp over all L keys."""
    Hq, Hkv, d, L = 4, 2, 16, 29
    G = Hq // Hkv
    q, kp, vp, pt = _case(8, Hq, Hkv, d, L, 0)
    qd = q[0]
    idx = np.tile(np.arange(L, dtype=np.int32), (Hkv, 1))
    scale = 1.0 / math.sqrt(d)
    o, lse = orc.draft_request(qd, kp, vp, pt, L, idx, Hkv, scale)
    for h in range(Hq):
        g = h // G
        Kt, Vt = _gather(kp, pt, L, g), _gather(vp, pt, L, g)
        qt = torch.from_numpy(qd[h].astype(np.float64))
        ref = F.scaled_dot_product_attention(qt[None, None, None], Kt[None, None], Vt[None, None],
                                             scale=scale)[0, 0, 0]
        _close(o[h], ref.numpy(), 1e-12, "draft full-list O")
        _close(lse[h], torch.logsumexp(torch.matmul(Kt, qt) * scale, 0).item(), 1e-12,
               "draft full-list LSE")


def pin_draft_invariances(orc):
    """Permuting the list changes nothing; entries outside [0, L) are ignored;
    a doubled entry adds ln 2 to the LSE; an all-invalid list gives O = 0,
    LSE = -inf."""
    Hq, Hkv, d, L = 4, 2, 16, 50
    q, kp, vp, pt = _case(9, Hq, Hkv, d, L, 0)
    qd = q[0]
    rng = np.random.default_rng(9)
    base = np.stack([np.sort(rng.choice(L, 12, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    o0, l0 = orc.draft_request(qd, kp, vp, pt, L, base, Hkv, 0.3)
    perm = np.stack([rng.permutation(row) for row in base]).astype(np.int32)
    o1, l1 = orc.draft_request(qd, kp, vp, pt, L, perm, Hkv, 0.3)
    _close(o1, o0, 1e-12, "permuted list O")
    _close(l1, l0, 1e-12, "permuted list LSE")
    junk = np.concatenate([base, np.full((Hkv, 3), L, np.int32), np.full((Hkv, 2), -5, np.int32),
                           np.full((Hkv, 1), L + 7, np.int32)], axis=1)
    o2, l2 = orc.draft_request(qd, kp, vp, pt, L, junk, Hkv, 0.3)
    _close(o2, o0, 1e-12, "masked entries O")
    _close(l2, l0, 1e-12, "masked entries LSE")
    one = np.full((Hkv, 1), 7, np.int32)
    two = np.full((Hkv, 2), 7, np.int32)
    o3, l3 = orc.draft_request(qd, kp, vp, pt, L, one, Hkv, 0.3)
    o4, l4 = orc.draft_request(qd, kp, vp, pt, L, two, Hkv, 0.3)
    _close(o4, o3, 1e-12, "duplicate O")
    _close(l4, l3 + math.log(2.0), 1e-12, "duplicate LSE")
    G = Hq // Hkv
    for h in range(Hq):
        _close(o3[h], vp[pt[7], h // G], 1e-12, "single entry O = V")
    bad = np.array([[L, -1], [L + 1, -2]], np.int32)
    o5, l5 = orc.draft_request(qd, kp, vp, pt, L, bad, Hkv, 0.3)
    assert np.all(o5 == 0.0) and np.all(np.isneginf(l5)), "all-masked list"


def pin_draft_matches_last_verify_row(orc):
    """The last verify row sees every position, so a draft with that query and
    the full list reproduces its O and LSE."""
    Hq, Hkv, d, L, k = 4, 2, 16, 31, 5
    q, kp, vp, pt = _case(10, Hq, Hkv, d, L, k)
    scale = 0.2
    logits, lse, o = orc.verify_request(q, kp, vp, pt, L, k, Hq, Hkv, scale)
    idx = np.tile(np.arange(L, dtype=np.int32), (Hkv, 1))
    od, ld = orc.draft_request(np.ascontiguousarray(q[k]), kp, vp, pt, L, idx, Hkv, scale)
    _close(od, o[k], 1e-12, "draft vs verify row k O")
    _close(ld, lse[k], 1e-12, "draft vs verify row k LSE")


def pin_bf16_widening(orc):
    """bf16 inputs are the high halves of binary32: a bf16 run equals the fp32
    run on the same (exactly representable) values."""
    Hq, Hkv, d, L, k = 2, 1, 8, 12, 2
    q, kp, vp, pt = _case(11, Hq, Hkv, d, L, k)
    to_bits = lambda a: (torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy()
                         .view(np.uint16))
    qb, kb, vb = to_bits(q), to_bits(kp), to_bits(vp)
    back = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    r1 = orc.verify_request(qb, kb, vb, pt, L, k, Hq, Hkv, 0.3)
    r2 = orc.verify_request(back(qb), back(kb), back(vb), pt, L, k, Hq, Hkv, 0.3)
    for a, b in zip(r1, r2):
        _close(a, b, 0.0, "bf16 widening")


# --------------------------------------------------------------------------- #
# recallable index (sinks + stored important positions + recent tokens)
# --------------------------------------------------------------------------- #
def pin_recall_special_cases(orc):
    """No sinks and no window return the stored list itself; sinks or a window
    covering the whole context return every position; padding is -1."""
    got, u = orc.recall_index(40, 0, 0, [2, 5, 17, 39], 6)
    assert u == 4 and list(got) == [2, 5, 17, 39, -1, -1], (u, got)
    for S, W in ((40, 0), (0, 40), (25, 15), (100, 3)):
        got, u = orc.recall_index(40, S, W, [7, 7, 60, -3], 40)
        assert u == 40 and list(got) == list(range(40)), (S, W, u)
    got, u = orc.recall_index(1, 0, 0, [], 1)
    assert u == 0 and list(got) == [-1]
    # stored entries past the context or negative name no position
    got, u = orc.recall_index(30, 2, 0, [5, 30, 33, -1, 5], 8)
    assert u == 3 and list(got) == [0, 1, 5, -1, -1, -1, -1, -1], (u, got)


def pin_recall_newest_tokens(orc):
    """A window of w keeps exactly the last w positions, so the newest token a
    draft appended (position L-1) is always recalled when w >= 1."""
    for L in (1, 2, 9, 33):
        for w in (1, 3, 8):
            got, u = orc.recall_index(L, 0, w, [], L)
            assert list(got[:u]) == list(range(max(0, L - w), L)), (L, w, got)


def pin_recall_set_properties(orc):
    """Random stored lists (with duplicates and out-of-range entries): the
    output is strictly ascending, holds every sink, every recent position and
    every valid stored entry, nothing else, and its size matches the count of
    the union worked out from interval lengths."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        L = int(rng.integers(1, 300))
        S = int(rng.integers(0, 12))
        W = int(rng.integers(0, 20))
        n = int(rng.integers(0, 40))
        stored = rng.integers(-4, L + 6, size=n).astype(np.int32)
        cap = L + 2
        got, u = orc.recall_index(L, S, W, stored, cap)
        body = np.asarray(got[:u], np.int64)
        assert np.all(got[u:] == -1), "padding"
        assert np.all(np.diff(body) > 0), "not strictly ascending"
        assert body.size == 0 or (body[0] >= 0 and body[-1] < L), "out of range"
        s_end = min(S, L)
        r_begin = max(s_end, L - W)
        valid = {int(p) for p in stored if 0 <= p < L}
        want_count = s_end + (L - r_begin) + sum(1 for p in valid if s_end <= p < r_begin)
        assert u == want_count, (trial, u, want_count)
        members = set(body.tolist())
        assert set(range(s_end)) <= members and set(range(r_begin, L)) <= members
        assert valid <= members
        for p in members:
            assert p < S or p >= L - W or p in valid, (trial, p)


# --------------------------------------------------------------------------- #
# quality of an index list (attention coverage, recall of the exact top-T)
# --------------------------------------------------------------------------- #
def _row(seed, Hq=4, L=60, hide=0):
    rng = np.random.default_rng(seed)
    lg = torch.from_numpy(rng.standard_normal((Hq, L)) * 2.0)
    if hide:
        lg[:, L - hide:] = -math.inf
    return lg, torch.logsumexp(lg, dim=1)


def pin_quality_full_and_empty_lists(orc):
    """Every position covers the whole softmax mass and recalls everything;
    a list of positions outside the context covers nothing."""
    lg, lse = _row(1, hide=5)
    full = np.stack([np.arange(60), np.arange(60)]).astype(np.int32)
    _, cov, rec = orc.list_quality(lg.numpy(), lse.numpy(), full, 7)
    _close(cov, np.ones(4), 1e-12, "coverage of every position")
    _close(rec, np.ones(4), 0, "recall of every position")
    bad = np.array([[-1, 60, 99], [60, -5, 1 << 30]], np.int32)
    _, cov, rec = orc.list_quality(lg.numpy(), lse.numpy(), bad, 7)
    _close(cov, np.zeros(4), 0, "coverage of no position")
    _close(rec, np.zeros(4), 0, "recall of no position")


def pin_quality_vs_torch(orc):
    """Coverage equals the softmax mass PyTorch assigns to the list's positions,
    the top-T equals torch.topk (no ties here), and recall is the overlap."""
    Hq, Hkv, L, T = 6, 2, 80, 10
    lg, lse = _row(2, Hq=Hq, L=L)
    rng = np.random.default_rng(3)
    lists = np.stack([np.sort(rng.choice(L, 20, replace=False)) for _ in range(Hkv)]).astype(np.int32)
    top, cov, rec = orc.list_quality(lg.numpy(), lse.numpy(), lists, T)
    prob = torch.softmax(lg, dim=1)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        _close(cov[h], float(prob[h, torch.from_numpy(lists[g]).long()].sum()), 1e-12, f"coverage h{h}")
        want = np.sort(torch.topk(prob[h], T).indices.numpy())
        assert np.array_equal(top[h], want), (h, top[h], want)
        _close(rec[h], len(set(want.tolist()) & set(lists[g].tolist())) / T, 0, f"recall h{h}")


def pin_quality_ties_bruteforce(orc):
    """Equal scores go to the lower position: brute force over all T-subsets
    of a tiny row with many ties."""
    L, T = 9, 4
    lg = torch.tensor([[0.5, 1.0, 1.0, 0.2, 1.0, 0.5, -math.inf, 1.0, 0.2]], dtype=torch.float64)
    lse = torch.logsumexp(lg, dim=1)
    top, _, _ = orc.list_quality(lg.numpy(), lse.numpy(), np.array([[1]], np.int32), T)
    assert np.array_equal(top[0], _brute_topk(lg[0].numpy(), T)), top


def pin_quality_repeats_count_once(orc):
    """Repeated list entries add their position's mass once."""
    lg, lse = _row(4, Hq=2, L=30)
    once = np.array([[3, 7, 11]], np.int32)
    many = np.array([[3, 3, 7, 11, 11, 11]], np.int32)
    _, c1, r1 = orc.list_quality(lg.numpy(), lse.numpy(), once, 3)
    _, c2, r2 = orc.list_quality(lg.numpy(), lse.numpy(), many, 3)
    _close(c1, c2, 1e-14, "coverage with repeats")
    _close(r1, r2, 0, "recall with repeats")


ALL_PINS = [pin_verify_vs_sdpa, pin_uniform_keys, pin_one_and_two_keys, pin_dump_consistency,
            pin_average, pin_topk_bruteforce, pin_topk_vs_torch, pin_topk_special,
            pin_draft_full_list, pin_draft_invariances, pin_draft_matches_last_verify_row,
            pin_bf16_widening, pin_recall_special_cases, pin_recall_newest_tokens,
            pin_recall_set_properties, pin_quality_full_and_empty_lists, pin_quality_vs_torch,
            pin_quality_ties_bruteforce, pin_quality_repeats_count_once]
