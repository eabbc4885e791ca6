"""HIP path against the oracle on seeded inputs -- needs an MI355X.

Every case runs through the C ABI (binding -> libspa.so) and compares O, LSE,
logits and the selected lists with the oracle element by element (tolerances in
parity.py)."""
from dataclasses import replace
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import to_np, widen
import parity
from sparse_self_speculative_pillarattn_amd import binding as bd
from sparse_self_speculative_pillarattn_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_unified(b, avg_row_begin=1, avg_row_count=None, opts=None):
    bufs = bd.StepBuffers(b, avg_row_begin, avg_row_count, opts=opts)
    bufs.logits.fill_(float("nan"))
    bufs.o.fill_(float("nan"))
    bufs.lse.fill_(float("nan"))
    bufs.step()
    torch.cuda.synchronize()
    return {"o": bufs.o, "lse": bufs.lse, "logits": bufs.logits, "idx": bufs.idx}


def check(oracle, w, seed=0, avg_row_begin=1, avg_row_count=None, opts=None, **kw):
    b = synth.make_batch(w, seed=seed, **kw)
    print(f"[case] {w.name} seed={seed} lens={b.seq_lens} verify={b.is_verify}", flush=True)
    ref = oracle.step(**parity.oracle_inputs(b, avg_row_begin, avg_row_count))
    gpu = run_unified(b.to(DEV), avg_row_begin, avg_row_count, opts)
    parity.compare_step(oracle, b, gpu, ref, avg_row_begin, avg_row_count)
    return b, gpu, ref


def test_tiny_fp32_workload(oracle):
    check(oracle, synth.TINY)


MIXED = [
    # (H_q, H_kv, d, k, lengths)
    (4, 2, 64, 4, ("uniform", 20, 300)),
    (8, 8, 128, 1, ("uniform", 2, 200)),
    (16, 8, 128, 8, ("uniform", 60, 700)),
    (32, 8, 128, 8, ("uniform", 500, 1500)),
    (40, 8, 128, 12, ("uniform", 13, 1200)),
    (16, 2, 128, 4, ("uniform", 100, 2100)),
    (8, 1, 64, 8, ("uniform", 9, 400)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", MIXED, ids=lambda s: f"h{s[0]}kv{s[1]}d{s[2]}k{s[3]}")
def test_mixed_batch(oracle, shape, dtype):
    Hq, Hkv, d, k, lengths = shape
    w = synth.Workload(name=f"mix-{Hq}-{Hkv}-{d}-{k}-{dtype}", batch=7, num_qo_heads=Hq,
                       num_kv_heads=Hkv, head_dim=d, dtype=dtype, spec_k=k,
                       sparsity=Fraction(1, 20), lengths=lengths, n_verify=3, seed=21)
    check(oracle, w)


@pytest.mark.parametrize("shape", [(32, 2, 128, 6, ("uniform", 7, 900)),
                                   (64, 4, 128, 3, ("uniform", 40, 1300)),
                                   (16, 1, 64, 2, ("uniform", 3, 500))],
                         ids=lambda s: f"h{s[0]}kv{s[1]}d{s[2]}k{s[3]}")
def test_large_group_bf16(oracle, shape):
    """GQA groups above 8 (bf16 only): draft rows of G = 16 heads, and the
    largest verify row count, (k+1) G = 112, i.e. seven MFMA row tiles."""
    Hq, Hkv, d, k, lengths = shape
    w = synth.Workload(name=f"bigg-{Hq}-{Hkv}-{d}-{k}", batch=6, num_qo_heads=Hq,
                       num_kv_heads=Hkv, head_dim=d, dtype="bf16", spec_k=k,
                       sparsity=Fraction(1, 10), lengths=lengths, n_verify=2, seed=31)
    check(oracle, w)


@pytest.mark.parametrize("L", [9, 63, 64, 65, 127, 129, 1000, 2049])
def test_ragged_lengths(oracle, L):
    w = synth.Workload(name=f"ragged-{L}", batch=3, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                       lengths=("fixed", L), n_verify=1, seed=L)
    check(oracle, w)


@pytest.mark.parametrize("overlap", [True, False])
def test_overlap_switch(oracle, overlap):
    """The unified step with the draft attention on the side stream and in one
    launch with the verify attention: same results."""
    w = synth.Workload(name=f"ovl{int(overlap)}", batch=9, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, dtype="bf16", spec_k=8, sparsity=Fraction(1, 4),
                       lengths=("uniform", 300, 5000), n_verify=3, seed=41)
    check(oracle, w, opts=bd.Options(overlap=overlap))


@pytest.mark.parametrize("split", [(64, 16), (2048, 2048), (320, 100), (40, 7)])
def test_split_invariance(oracle, split):
    w = synth.Workload(name="split", batch=6, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                       dtype="bf16", spec_k=8, sparsity=Fraction(1, 5),
                       lengths=("uniform", 900, 2600), n_verify=2, seed=5)
    check(oracle, w, opts=bd.Options(verify_chunk=split[0], draft_chunk=split[1]))


@pytest.mark.parametrize("L,s", [(8192, Fraction(1, 20)), (8193, Fraction(1, 20)),
                                 (12289, Fraction(1, 20)), (20001, Fraction(1, 50)),
                                 (40000, Fraction(1, 20)), (30001, Fraction(1, 2)),
                                 (270001, Fraction(1, 50))])
def test_long_rows(oracle, L, s):
    """Rows longer than one selection workgroup's registers (8192 scores),
    which the selection re-reads chunk by chunk after its histogram-seeded
    start.  Lengths around the boundary, odd lengths (rows not 16-byte
    aligned), a large K (half the row), and a row longer than the selection's
    LDS position bitmap (262,144 positions), which is compacted by a second
    pass over the row instead."""
    w = synth.Workload(name=f"long-{L}", batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                       dtype="bf16", spec_k=2, sparsity=s, lengths=("fixed", L), n_verify=2,
                       seed=L)
    check(oracle, w)


def test_long_row_all_scores_tied(oracle):
    """Every position of a 10,000-token verify request reads the same K/V
    slot, so all but the causally hidden tail tie: the selection, seeded by a
    histogram whose one bin holds them all, must keep the lowest positions."""
    L = 10000
    w = synth.Workload(name="long-tied", batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                       dtype="bf16", spec_k=2, sparsity=Fraction(1, 20), lengths=("fixed", L),
                       n_verify=1, seed=77)
    b = synth.make_batch(w)
    r = int(np.nonzero(b.is_verify)[0][0])
    b.page_table[r, :L] = b.page_table[r, 0]
    ref = oracle.step(**parity.oracle_inputs(b))
    gpu = run_unified(b.to(DEV))
    parity.compare_step(oracle, b, gpu, ref)
    K = b.idx_count[r]
    seg = to_np(gpu["idx"])[b.idx_off[r]:b.idx_off[r] + w.num_kv_heads * K].reshape(w.num_kv_heads, K)
    assert np.array_equal(seg, np.tile(np.arange(K), (w.num_kv_heads, 1)))


@pytest.mark.parametrize("K", [5, 15])
def test_long_row_tie_across_the_kth_score(oracle, K):
    """A 20,001-token verify request whose 12 highest scores tie: 12 spread
    positions read one K/V slot whose keys point along the request's mean query
    of each group.  Long rows are written from a bitmap of the selected
    positions; with K = 5 the five lowest tied positions must be taken, with
    K = 15 all twelve and the three next-highest."""
    L = 20001
    w = synth.Workload(name=f"long-tie-{K}", batch=2, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, dtype="bf16", spec_k=2, sparsity=Fraction(1, 20),
                       lengths=("fixed", L), n_verify=1, seed=91)
    b = synth.make_batch(w)
    r = int(np.nonzero(b.is_verify)[0][0])
    tied = [100, 1700, 3000, 9000, 9001, 12000, 15000, 16000, 17000, 18000, 19000, 19500]
    slot = int(b.page_table[r, tied[0]])
    b.page_table[r, torch.tensor(tied)] = slot
    G, d = w.num_qo_heads // w.num_kv_heads, w.head_dim
    qr = b.q[b.q_indptr[r]:b.q_indptr[r + 1]].float()
    for g in range(w.num_kv_heads):
        u = qr[:, g * G:(g + 1) * G].reshape(-1, d).mean(dim=0)
        b.k_pool[slot, g] = (8.0 * d ** 0.5 * u / u.norm()).to(b.k_pool.dtype)
    b.idx_count[r] = K
    print(f"[case] tie K={K} r={r} slot={slot}", flush=True)
    ref = oracle.step(**parity.oracle_inputs(b))
    gpu = run_unified(b.to(DEV))
    parity.compare_step(oracle, b, gpu, ref)
    seg = to_np(gpu["idx"])[b.idx_off[r]:b.idx_off[r] + w.num_kv_heads * K].reshape(w.num_kv_heads, K)
    for g in range(w.num_kv_heads):
        if K < len(tied):
            assert seg[g].tolist() == tied[:K], (g, seg[g])
        else:
            assert set(tied) <= set(seg[g].tolist()), (g, seg[g])


# chunk edges of a 40,000-score row (position 39,999 is visible to the last
# averaged row only, so its score would not tie)
CHUNK_EDGES = [8191, 8192, 16383, 16384, 24575, 24576, 32767, 32768, 39998]


@pytest.mark.parametrize("n_tied,K", [(12, 5), (12, 15), (300, 150), (300, 305)])
def test_chunked_long_row_ties(oracle, n_tied, K):
    """A 40,000-token verify request, longer than 32,768 scores, is selected
    by one workgroup per 8192-score chunk.  Its n_tied highest scores tie, at
    positions spread over every chunk and on the chunks' edges, so each chunk
    must know how many tied positions the earlier chunks took.  With K below
    n_tied the lowest K tied positions are taken; above it, all of them and the
    next highest.  Twelve tied keys are ranked by one wave; three hundred are
    more than a wave ranks directly and are walked digit by digit in LDS."""
    L = 40000
    w = synth.Workload(name=f"chunk-tie-{n_tied}-{K}", batch=2, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, dtype="bf16", spec_k=2, sparsity=Fraction(1, 20),
                       lengths=("fixed", L), n_verify=1, seed=93)
    b = synth.make_batch(w)
    r = int(np.nonzero(b.is_verify)[0][0])
    rng = np.random.default_rng(n_tied)
    rest = rng.choice(np.setdiff1d(np.arange(L - 2), CHUNK_EDGES), n_tied - len(CHUNK_EDGES),
                      replace=False)
    tied = sorted(CHUNK_EDGES + [int(x) for x in rest])
    slot = int(b.page_table[r, tied[0]])
    b.page_table[r, torch.tensor(tied)] = slot
    G, d = w.num_qo_heads // w.num_kv_heads, w.head_dim
    qr = b.q[b.q_indptr[r]:b.q_indptr[r + 1]].float()
    for g in range(w.num_kv_heads):
        u = qr[:, g * G:(g + 1) * G].reshape(-1, d).mean(dim=0)
        b.k_pool[slot, g] = (8.0 * d ** 0.5 * u / u.norm()).to(b.k_pool.dtype)
    b.idx_count[r] = K
    print(f"[case] chunked tie n={n_tied} K={K} r={r} slot={slot}", flush=True)
    ref = oracle.step(**parity.oracle_inputs(b))
    gpu = run_unified(b.to(DEV))
    parity.compare_step(oracle, b, gpu, ref)
    seg = to_np(gpu["idx"])[b.idx_off[r]:b.idx_off[r] + w.num_kv_heads * K].reshape(w.num_kv_heads, K)
    for g in range(w.num_kv_heads):
        if K < len(tied):
            assert seg[g].tolist() == tied[:K], (g, seg[g][:20])
        else:
            assert set(tied) <= set(seg[g].tolist()), g


def test_chunked_long_row_all_scores_tied(oracle):
    """Every position of a 40,000-token verify request reads one K/V slot:
    the boundary bin holds more keys than a chunked row keeps as candidates,
    so the row's first chunk workgroup selects it alone; the lowest positions
    are kept."""
    L = 40000
    w = synth.Workload(name="chunk-tied", batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                       dtype="bf16", spec_k=2, sparsity=Fraction(1, 20), lengths=("fixed", L),
                       n_verify=1, seed=78)
    b = synth.make_batch(w)
    r = int(np.nonzero(b.is_verify)[0][0])
    b.page_table[r, :L] = b.page_table[r, 0]
    ref = oracle.step(**parity.oracle_inputs(b))
    gpu = run_unified(b.to(DEV))
    parity.compare_step(oracle, b, gpu, ref)
    K = b.idx_count[r]
    seg = to_np(gpu["idx"])[b.idx_off[r]:b.idx_off[r] + w.num_kv_heads * K].reshape(w.num_kv_heads, K)
    assert np.array_equal(seg, np.tile(np.arange(K), (w.num_kv_heads, 1)))


def test_chunked_row_of_the_longest_verify(oracle):
    """The longest verify row the split-K merge takes (256 chunks of 2048
    positions, 524,288 scores) is 64 selection chunks, one per lane of the
    wave that scans the chunks' counts.  One KV head of 64 dimensions keeps
    the oracle's work small."""
    L = 524288
    w = synth.Workload(name=f"chunks-{L}", batch=2, num_qo_heads=2, num_kv_heads=1, head_dim=64,
                       dtype="bf16", spec_k=2, sparsity=Fraction(1, 50), lengths=("fixed", L),
                       n_verify=1, seed=288)
    check(oracle, w)


def test_chunked_long_rows_fp32(oracle):
    """Rows selected in chunks on the fp32 path: two verify requests of
    47,661 and 38,684 scores (six and five chunks, the last ones partial),
    from the VALU attention tile's logits."""
    w = synth.Workload(name="chunk-f32", batch=4, num_qo_heads=4, num_kv_heads=2, head_dim=64,
                       dtype="f32", spec_k=2, sparsity=Fraction(1, 20),
                       lengths=("uniform", 36001, 49153), n_verify=2, seed=97)
    check(oracle, w)


def test_chunked_long_rows_with_overlap(oracle):
    """Rows selected in chunks while the drafts run as a second attention
    launch on a side stream (the overlap option): the count and chunk launches
    follow the post-pass on the caller's stream."""
    w = synth.Workload(name="chunk-overlap", batch=5, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                       dtype="bf16", spec_k=2, sparsity=Fraction(1, 20), lengths=("fixed", 36001),
                       n_verify=2, seed=95)
    check(oracle, w, opts=bd.Options(overlap=True))


def test_topk_count_extremes(oracle):
    """K = 1 and K = L per verify request."""
    w = synth.Workload(name="kext", batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                       dtype="bf16", spec_k=4, sparsity=Fraction(1, 1), lengths=("fixed", 300),
                       n_verify=2, seed=3)
    b = synth.make_batch(w)
    b.idx_count[1] = 1
    b.idx_off[1] = b.idx_off[0] + w.num_kv_heads * b.idx_count[0]
    ref = oracle.step(**parity.oracle_inputs(b))
    gpu = run_unified(b.to(DEV))
    parity.compare_step(oracle, b, gpu, ref)
    seg = to_np(gpu["idx"])[:w.num_kv_heads * 300].reshape(w.num_kv_heads, 300)
    assert np.array_equal(seg, np.tile(np.arange(300), (w.num_kv_heads, 1)))


def test_averaged_rows_parameter(oracle):
    """The averaged rows are a parameter: all k+1 rows, and rows 0..k-1."""
    w = synth.Workload(name="avg", batch=4, num_qo_heads=16, num_kv_heads=4, head_dim=128,
                       dtype="bf16", spec_k=6, sparsity=Fraction(1, 10),
                       lengths=("uniform", 200, 900), n_verify=2, seed=8)
    check(oracle, w, avg_row_begin=0, avg_row_count=7)
    check(oracle, w, avg_row_begin=0, avg_row_count=6)


def _draft_only(oracle, b, lists, counts, opts=None):
    """Run spa_draft_attn on B draft rows with explicit lists; compare with the oracle."""
    w = b.w
    Hkv = w.num_kv_heads
    offs = np.concatenate([[0], np.cumsum([Hkv * c for c in counts])[:-1]]).astype(np.int64)
    flat = np.concatenate([np.asarray(l, np.int32).ravel() for l in lists])
    dq = b.q[:len(counts)].contiguous()
    lay = bd.layout(w.num_qo_heads, Hkv, w.head_dim, b.q.dtype, b.num_slots, b.stride)
    o = torch.full_like(dq, float("nan"), device=DEV)
    lse = torch.full((len(counts), w.num_qo_heads), float("nan"), device=DEV)
    nbytes = bd.workspace_bytes(lay, len(counts), 1, None, b.seq_lens[:len(counts)], counts, opts)
    ws = bd.workspace(nbytes, DEV)
    bd.draft_attn(lay, len(counts), b.seq_lens[:len(counts)], b.page_table.to(DEV), counts, offs,
                  torch.from_numpy(flat).to(DEV), dq.to(DEV), b.k_pool.to(DEV), b.v_pool.to(DEV),
                  o, lse, ws, opts=opts)
    torch.cuda.synchronize()
    qn, kn, vn, ptn = to_np(dq), to_np(b.k_pool), to_np(b.v_pool), to_np(b.page_table)
    for r, (lst, c) in enumerate(zip(lists, counts)):
        L = b.seq_lens[r]
        ro, rl = oracle.draft_request(np.ascontiguousarray(qn[r]), kn, vn, ptn[r, :L], L,
                                      np.asarray(lst, np.int32).reshape(Hkv, c), Hkv,
                                      1.0 / np.sqrt(w.head_dim))
        parity.assert_o(to_np(o[r]), ro, w.dtype, f"draft {r} O")
        parity.assert_lse(to_np(lse[r]), rl, f"draft {r} LSE")
    return o, lse


def test_draft_list_edge_cases(oracle):
    """Invalid entries are ignored, duplicates count twice, an all-invalid list
    gives O = 0 and LSE = -inf, and the full list equals dense attention."""
    w = synth.Workload(name="edge", batch=5, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                       dtype="bf16", spec_k=4, sparsity=Fraction(1, 20),
                       lengths=("fixed", 400), n_verify=0, seed=4)
    b = synth.make_batch(w, is_verify=[False] * 5)
    rng = np.random.default_rng(0)
    lists, counts = [], []
    base = np.sort(rng.choice(400, 30, replace=False))
    lists.append(np.stack([np.concatenate([base, [400, -1, 1 << 30, -7]])] * 2)); counts.append(34)
    lists.append(np.stack([np.array([5, 5, 9, 9, 9])] * 2)); counts.append(5)
    lists.append(np.stack([np.array([400, -1, 4000])] * 2)); counts.append(3)
    lists.append(np.stack([np.arange(400)] * 2)); counts.append(400)
    lists.append(np.stack([rng.permutation(400)[:50], rng.permutation(400)[:50]])); counts.append(50)
    _draft_only(oracle, b, lists, counts)


def _poison_slot0(b):
    """Moves every token stored in pool slot 0 to an unused slot, then fills
    slot 0's K and V rows with NaN, +Inf and -Inf: no request references it, so
    no output may depend on it."""
    used = set()
    for r in range(b.B):
        used.update(b.page_table[r, :b.seq_lens[r]].tolist())
    free = next(x for x in range(1, b.num_slots) if x not in used)
    for r in range(b.B):
        row = b.page_table[r, :b.seq_lens[r]]
        hit = (row == 0).nonzero().flatten()
        if len(hit):
            row[hit] = free
            b.k_pool[free] = b.k_pool[0]
            b.v_pool[free] = b.v_pool[0]
    bad = torch.tensor([float("nan"), float("inf"), float("-inf"), float("nan")])
    for pool in (b.k_pool, b.v_pool):
        pool[0] = bad.repeat(pool.shape[-1] // 4).to(pool.dtype)


@pytest.mark.parametrize("dtype,packed", [("bf16", False), ("f32", False), ("bf16", True)])
def test_masked_entries_ignore_nonfinite_pool_row(oracle, dtype, packed):
    """Masked list entries (out of range, negative, and the padding of chunks
    that are not a whole number of 32-entry tiles) read pool row 0 on the MFMA
    path; with NaN and Inf there, every draft still matches the oracle, and a
    list with no valid entry gives O = 0 and LSE = -inf exactly."""
    w = synth.Workload(name=f"nanrow-{dtype}", batch=6, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, dtype=dtype, spec_k=4, sparsity=Fraction(1, 20),
                       lengths=("fixed", 400), n_verify=0, seed=44)
    b = synth.make_batch(w, is_verify=[False] * 6)
    _poison_slot0(b)
    rng = np.random.default_rng(3)
    lists, counts = [], []
    base = np.sort(rng.choice(400, 30, replace=False))
    lists.append(np.stack([np.concatenate([base, [400, -1, 1 << 30, -7]])] * 2)); counts.append(34)
    lists.append(np.stack([np.array([400, -1, 4000])] * 2)); counts.append(3)
    lists.append(np.stack([np.array([-1] * 40 + [7])] * 2)); counts.append(41)
    lists.append(np.stack([np.concatenate([rng.choice(400, 33), [-1] * 12])] * 2)); counts.append(45)
    lists.append(np.stack([np.array([123])] * 2)); counts.append(1)
    lists.append(np.stack([np.arange(400)] * 2)); counts.append(400)
    # packed: planned for one CU, so every draft item holds both KV heads
    o, lse = _draft_only(oracle, b, lists, counts, bd.Options(num_cus=1) if packed else None)
    assert bool((o[1].float() == 0).all()), "all-invalid list: O is not 0"
    assert bool(torch.isneginf(lse[1]).all()), "all-invalid list: LSE is not -inf"
    assert bool(torch.isfinite(o.float()).all()), "non-finite O"


def test_masked_entries_nonfinite_pool_row_unified(oracle):
    """The same poisoned pool row under a mixed unified step whose drafts read
    lists padded with -1 (the recallable index's padding)."""
    w = synth.Workload(name="nanrow-unified", batch=7, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                       lengths=("uniform", 300, 1500), n_verify=2, seed=45)
    b = synth.make_batch(w)
    _poison_slot0(b)
    for r in range(b.B):
        if not b.is_verify[r]:
            K = b.idx_count[r]
            seg = b.idx[b.idx_off[r]:b.idx_off[r] + w.num_kv_heads * K].view(w.num_kv_heads, K)
            seg[:, -(K // 3):] = -1
    print(f"[case] {w.name} lens={b.seq_lens}", flush=True)
    ref = oracle.step(**parity.oracle_inputs(b))
    gpu = run_unified(b.to(DEV))
    parity.compare_step(oracle, b, gpu, ref)


PACKED = [
    # (H_q, H_kv, d, lengths, s): the plan for one CU packs up to 4 KV heads
    # of a draft request into one item (2 for H_kv = 2, 8 for G = 2, none for G = 16)
    (32, 8, 128, ("uniform", 50, 3000), Fraction(1, 20)),
    (16, 8, 128, ("uniform", 20, 900), Fraction(1, 10)),
    (8, 2, 64, ("uniform", 40, 2000), Fraction(1, 50)),
    (64, 4, 128, ("uniform", 100, 800), Fraction(1, 20)),
]


@pytest.mark.parametrize("shape", PACKED, ids=lambda s: f"h{s[0]}kv{s[1]}d{s[2]}")
def test_packed_draft_items(oracle, shape):
    """Draft items holding the lists of several KV heads (planned for one CU,
    so that even a small batch packs): every output matches the oracle, and
    the same bits as the unpacked plan."""
    Hq, Hkv, d, lengths, s = shape
    w = synth.Workload(name=f"pack-{Hq}-{Hkv}-{d}", batch=9, num_qo_heads=Hq, num_kv_heads=Hkv,
                       head_dim=d, dtype="bf16", spec_k=4, sparsity=s, lengths=lengths,
                       n_verify=2, seed=Hq + d)
    b, packed, ref = check(oracle, w, opts=bd.Options(num_cus=1, verify_chunk=512))
    # the same verify chunks, drafts unpacked
    plain = run_unified(b.to(DEV), opts=bd.Options(verify_chunk=512))
    for name in ("o", "lse", "logits", "idx"):
        assert np.array_equal(to_np(packed[name]).view(np.uint8), to_np(plain[name]).view(np.uint8)), name


def test_sequential_entry_points_match_unified(oracle):
    """spa_verify_attn + spa_pillar_topk + spa_draft_attn on the same batch give
    what spa_unified_step gives."""
    w = synth.Workload(name="seq", batch=6, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                       dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                       lengths=("uniform", 300, 1800), n_verify=2, seed=9)
    b = synth.make_batch(w)
    bd_ = b.to(DEV)
    uni = run_unified(bd_)
    ver = [r for r in range(b.B) if b.is_verify[r]]
    dra = [r for r in range(b.B) if not b.is_verify[r]]
    k, Hq, Hkv, d = w.spec_k, w.num_qo_heads, w.num_kv_heads, w.head_dim
    lay = bd.layout(Hq, Hkv, d, b.q.dtype, b.num_slots, b.stride)
    # verify-only batch
    qv = torch.cat([bd_.q[b.q_indptr[r]:b.q_indptr[r + 1]] for r in ver]).contiguous()
    ptv = torch.stack([bd_.page_table[r] for r in ver]).contiguous()
    lv = [b.seq_lens[r] for r in ver]
    loff = np.concatenate([[0], np.cumsum([(k + 1) * Hq * L for L in lv])[:-1]]).astype(np.int64)
    ov = torch.empty_like(qv)
    lsev = torch.empty((qv.shape[0], Hq), device=DEV)
    lgv = torch.empty((int(sum((k + 1) * Hq * L for L in lv)),), device=DEV)
    nb = bd.workspace_bytes(lay, len(ver), k, [1] * len(ver), lv, [b.idx_count[r] for r in ver])
    ws = bd.workspace(nb, DEV)
    bd.verify_attn(lay, len(ver), k, lv, ptv, qv, bd_.k_pool, bd_.v_pool, ov, lsev, lgv, loff, ws)
    Kv = [b.idx_count[r] for r in ver]
    ioff = np.concatenate([[0], np.cumsum([Hkv * K for K in Kv])[:-1]]).astype(np.int64)
    idxv = torch.zeros((int(sum(Hkv * K for K in Kv)),), dtype=torch.int32, device=DEV)
    bd.pillar_topk(len(ver), k, Hq, Hkv, 1, k, lv, Kv, lgv, loff, lsev, idxv, ioff, ws)
    # draft-only batch
    qd = torch.stack([bd_.q[b.q_indptr[r]] for r in dra]).contiguous()
    ptd = torch.stack([bd_.page_table[r] for r in dra]).contiguous()
    ld = [b.seq_lens[r] for r in dra]
    Kd = [b.idx_count[r] for r in dra]
    doff = np.concatenate([[0], np.cumsum([Hkv * K for K in Kd])[:-1]]).astype(np.int64)
    idxd = torch.cat([bd_.idx[b.idx_off[r]:b.idx_off[r] + Hkv * b.idx_count[r]] for r in dra])
    od = torch.empty_like(qd)
    lsed = torch.empty((len(dra), Hq), device=DEV)
    bd.draft_attn(lay, len(dra), ld, ptd, Kd, doff, idxd.contiguous(), qd, bd_.k_pool,
                  bd_.v_pool, od, lsed, ws)
    torch.cuda.synchronize()
    uo, ul, ui = to_np(uni["o"]), to_np(uni["lse"]), to_np(uni["idx"])
    row = 0
    for j, r in enumerate(ver):
        a, z = b.q_indptr[r], b.q_indptr[r + 1]
        assert np.array_equal(to_np(ov[row:row + k + 1]), uo[a:z])
        assert np.array_equal(to_np(lsev[row:row + k + 1]), ul[a:z])
        row += k + 1
        assert np.array_equal(to_np(idxv)[ioff[j]:ioff[j] + Hkv * Kv[j]],
                              ui[b.idx_off[r]:b.idx_off[r] + Hkv * Kv[j]])
    for j, r in enumerate(dra):
        assert np.array_equal(to_np(od[j]), uo[b.q_indptr[r]])
        assert np.array_equal(to_np(lsed[j]), ul[b.q_indptr[r]])


@pytest.mark.parametrize("lens", [(20001, 40000), (8193, 9000)])
def test_pillar_topk_alone_long_rows(oracle, lens):
    """spa_pillar_topk on its own starts the selection without a score
    histogram (it has no attention launch to count one); on rows longer than
    the selection's registers it must still pick what the unified step picks
    from the same logits and LSE, and what the oracle's scores allow."""
    w = synth.Workload(name="topk-long", batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=128,
                       dtype="bf16", spec_k=3, sparsity=Fraction(1, 20), lengths=("fixed", 64),
                       n_verify=2, seed=lens[0])
    b = synth.make_batch(w, seq_lens=[lens[0], lens[1], 5000], is_verify=[1, 1, 0])
    print(f"[case] topk alone lens={b.seq_lens}", flush=True)
    ref = oracle.step(**parity.oracle_inputs(b))
    uni = run_unified(b.to(DEV))
    parity.compare_step(oracle, b, uni, ref)
    k, Hq, Hkv = w.spec_k, w.num_qo_heads, w.num_kv_heads
    ver = [r for r in range(b.B) if b.is_verify[r]]
    lv = [b.seq_lens[r] for r in ver]
    Kv = [b.idx_count[r] for r in ver]
    loff = np.array([b.logits_off[r] for r in ver], dtype=np.int64)
    lsev = torch.cat([uni["lse"][b.q_indptr[r]:b.q_indptr[r + 1]] for r in ver]).contiguous()
    ioff = np.concatenate([[0], np.cumsum([Hkv * K for K in Kv])[:-1]]).astype(np.int64)
    idxv = torch.full((int(sum(Hkv * K for K in Kv)),), -7, dtype=torch.int32, device=DEV)
    lay = bd.layout(Hq, Hkv, w.head_dim, b.q.dtype, b.num_slots, b.stride)
    nb = bd.workspace_bytes(lay, len(ver), k, [1] * len(ver), lv, Kv)
    ws = bd.workspace(nb, DEV)
    bd.pillar_topk(len(ver), k, Hq, Hkv, 1, k, lv, Kv, uni["logits"], loff, lsev, idxv, ioff, ws)
    torch.cuda.synchronize()
    got, want = to_np(idxv), to_np(uni["idx"])
    for j, r in enumerate(ver):
        assert np.array_equal(got[ioff[j]:ioff[j] + Hkv * Kv[j]],
                              want[b.idx_off[r]:b.idx_off[r] + Hkv * Kv[j]]), f"request {r}"


def test_chained_verify_then_draft(oracle):
    """A verify step's selected lists feed the next step, where the same
    requests draft over them."""
    w = synth.Workload(name="chain", batch=3, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                       dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                       lengths=("uniform", 1000, 3000), n_verify=3, seed=12)
    b, gpu, ref = check(oracle, w)
    # next step: every request drafts with the list its verify just produced
    b2 = synth.make_batch(replace(w, n_verify=0, seed=13), is_verify=[False] * 3,
                          seq_lens=b.seq_lens)
    b2 = replace(b2, k_pool=b.k_pool, v_pool=b.v_pool, page_table=b.page_table,
                 idx=gpu["idx"].cpu(), idx_count=b.idx_count, idx_off=b.idx_off,
                 num_slots=b.num_slots)
    ref2 = oracle.step(**parity.oracle_inputs(b2))
    gpu2 = run_unified(b2.to(DEV))
    parity.compare_step(oracle, b2, gpu2, ref2)


def test_workspace_reuse_across_batches(oracle):
    """One workspace serves differently shaped batches back to back; all of it
    but the work counters is poisoned with NaN bytes before each call, so a
    read of anything a call did not write itself shows up in the outputs, and
    every call leaves the counters at zero."""
    shapes = [(5, ("uniform", 600, 2500), 2, 3), (3, ("uniform", 100, 1300), 1, 4),
              (6, ("uniform", 1500, 3000), 3, 5)]
    batches = []
    for B, lengths, nv, seed in shapes:
        w = synth.Workload(name=f"reuse{seed}", batch=B, num_qo_heads=32, num_kv_heads=8,
                           head_dim=128, dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                           lengths=lengths, n_verify=nv, seed=seed)
        batches.append(synth.make_batch(w))
    need = 0
    for b in batches:
        lay = bd.layout(32, 8, 128, b.q.dtype, b.num_slots, b.stride)
        need = max(need, bd.workspace_bytes(lay, b.B, 8, b.is_verify, b.seq_lens, b.idx_count))
    ws = bd.workspace(need, DEV)
    for b in batches:
        ws[256:].fill_(0xFF)  # all but the work counters, which calls leave at zero
        bufs = bd.StepBuffers(b.to(DEV))
        bufs.ws = ws
        bufs.step()
        torch.cuda.synchronize()
        assert not bool(ws[:256].any()), "the work counters were not left at zero"
        ref = oracle.step(**parity.oracle_inputs(b))
        parity.compare_step(oracle, b, {"o": bufs.o, "lse": bufs.lse, "logits": bufs.logits,
                                        "idx": bufs.idx}, ref)


@pytest.mark.parametrize("B", [63, 64, 65, 127, 128, 129])
def test_item_counts_around_the_grid(oracle, B):
    """Draft-only batches whose attention item counts sit around the launch's
    workgroup count: workgroup b starts on item b and only later items come
    from the counter, so fewer, as many and a few more items than workgroups
    all occur.  With 256-thread workgroups, two per CU on 256 CUs, B = 63, 64
    and 65 give 504, 512 and 520 items (one KV head's list each), and B = 127,
    128 and 129 give 1016, 512 and 516 (from 128 drafts on, two lists per
    item).  Every output matches the oracle, and the work counters are back
    at zero after the call."""
    w = synth.Workload(name=f"grid{B}", batch=B, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                       dtype="bf16", spec_k=8, sparsity=Fraction(1, 20), lengths=("fixed", 1024),
                       seed=B)
    b = synth.uniform_batch(w, B, 1024, [0] * B, seed=B)
    print(f"[case] grid B={B}", flush=True)
    ref = oracle.step(**parity.oracle_inputs(b))
    bufs = bd.StepBuffers(b.to(DEV))
    bufs.o.fill_(float("nan"))
    bufs.lse.fill_(float("nan"))
    bufs.step()
    torch.cuda.synchronize()
    assert not bool(bufs.ws[:256].any()), "the work counters were not left at zero"
    parity.compare_step(oracle, b, {"o": bufs.o, "lse": bufs.lse, "logits": bufs.logits,
                                    "idx": bufs.idx}, ref)


FULL = [synth.QWEN3_1_7B.name, synth.QWEN3_8B.name, synth.QWEN3_14B.name, synth.LONG_CTX.name]


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_request(oracle, name):
    """Each workload at its full size, in the configuration the benchmark times
    (one unified step, default work split), against the oracle's whole step
    on the same inputs: every request's O and LSE, every verify request's
    dumped logits and per-KV-head top-K; plus size-independent properties over
    the whole batch."""
    w = synth.WORKLOADS[name]
    print(f"[full-size] {name}", flush=True)
    b = synth.make_batch(w, device=DEV)
    bufs = bd.StepBuffers(b)
    bufs.step()
    torch.cuda.synchronize()
    gpu = {"o": bufs.o, "lse": bufs.lse, "logits": bufs.logits, "idx": bufs.idx}
    parity.check_whole_batch_properties(b, gpu)
    ref = oracle.step(**parity.oracle_inputs_compact(b))
    print(f"[full-size] {name}: oracle done ({ref['nthreads']} threads)", flush=True)
    parity.compare_step(oracle, b, gpu, ref)
    del bufs, gpu, b, ref
    torch.cuda.empty_cache()


def test_concurrent_streams_match_sequential():
    """Two batches stepped concurrently on two streams (default priority), many
    times back to back, give bit for bit what each gives alone: every call owns
    its plan slot and item counters, and an item's result does not depend on
    which workgroup draws it."""
    shapes = [(6, ("uniform", 400, 3000), 2, 31), (9, ("uniform", 100, 2000), 3, 32)]
    batches = []
    for B, lengths, nv, seed in shapes:
        w = synth.Workload(name=f"streams{seed}", batch=B, num_qo_heads=32, num_kv_heads=8,
                           head_dim=128, dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                           lengths=lengths, n_verify=nv, seed=seed)
        batches.append(synth.make_batch(w, device=DEV))
    alone = []
    for b in batches:
        bufs = bd.StepBuffers(b)
        bufs.step()
        torch.cuda.synchronize()
        alone.append([to_np(t).copy() for t in (bufs.o, bufs.lse, bufs.logits, bufs.idx)])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [bd.StepBuffers(b) for b in batches]
    torch.cuda.synchronize()
    for _ in range(20):
        for s, bu in zip(streams, bufs):
            with torch.cuda.stream(s):
                bu.step()
    torch.cuda.synchronize()
    for want, bu in zip(alone, bufs):
        got = [to_np(t) for t in (bu.o, bu.lse, bu.logits, bu.idx)]
        for name, a, g in zip(("O", "LSE", "logits", "idx"), want, got):
            assert np.array_equal(a.view(np.uint8), g.view(np.uint8)), f"{name} differs"


def test_stepbuffers_rebinds_replaced_buffers():
    """Replacing the workspace and an output after a step rebinds them: the
    next step writes the new buffers and gives the same bits."""
    w = synth.Workload(name="rebind", batch=5, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                       dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                       lengths=("uniform", 500, 2500), n_verify=2, seed=61)
    b = synth.make_batch(w, device=DEV)
    bufs = bd.StepBuffers(b)
    bufs.step()
    torch.cuda.synchronize()
    first = [to_np(t).copy() for t in (bufs.o, bufs.lse, bufs.logits, bufs.idx)]
    old_ws, old_o = bufs.ws, bufs.o
    bufs.ws = torch.full((old_ws.numel() + 4096,), 0xFF, dtype=torch.uint8, device=DEV)
    bufs.ws[:256] = 0  # a new workspace's work counters start at zero
    bufs.o = torch.full_like(old_o, float("nan"))
    old_o.fill_(0.0)
    bufs.step()
    torch.cuda.synchronize()
    assert bool((old_o == 0).all()), "the replaced output was written"
    second = [to_np(t) for t in (bufs.o, bufs.lse, bufs.logits, bufs.idx)]
    for name, a, g in zip(("O", "LSE", "logits", "idx"), first, second):
        assert np.array_equal(a.view(np.uint8), g.view(np.uint8)), f"{name} differs"


def test_plan_buffers_released_every_way(oracle):
    """Eighty calls on one stream without a synchronisation share two plan
    buffers, so every call waits for a buffer the GPU may still be reading,
    while mixing the four ways a buffer is released: a mixed batch (the
    post-pass reports it), a draft-only batch (the attention launch's last work
    draw), spa_pillar_topk alone (the selection launch) and spa_recall_index
    (a one-thread release launch).  Every output ends bit for bit equal to the
    same call made alone, so no buffer was rewritten while a launch still read
    it."""
    def wl(name, B, nv, seed):
        return synth.Workload(name=name, batch=B, num_qo_heads=16, num_kv_heads=8, head_dim=128,
                              dtype="bf16", spec_k=4, sparsity=Fraction(1, 10),
                              lengths=("uniform", 300, 2500), n_verify=nv, seed=seed)
    mixed = synth.make_batch(wl("rel-mixed", 7, 2, 91), device=DEV)
    drafts = synth.make_batch(wl("rel-draft", 6, 0, 92), device=DEV, is_verify=[False] * 6)
    verify = synth.make_batch(wl("rel-verify", 3, 3, 93), device=DEV, is_verify=[True] * 3)
    bm, bdr, bv = bd.StepBuffers(mixed), bd.StepBuffers(drafts), bd.StepBuffers(verify)
    k, Hq, Hkv = 4, 16, 8
    topk_idx = torch.full_like(bv.idx, -5)
    rec_cnt = [bd.recall_length(L, K, 4, 16) for L, K in zip(drafts.seq_lens, drafts.idx_count)]
    rec_off = np.concatenate([[0], np.cumsum([Hkv * c for c in rec_cnt])[:-1]]).astype(np.int64)
    rec_out = torch.full((int(sum(Hkv * c for c in rec_cnt)),), -9, dtype=torch.int32, device=DEV)
    need = max(bm.plans.nbytes, bdr.plans.nbytes, bv.plans.nbytes,
               bd.recall_plan_bytes(drafts.B))
    shared = bd.PlanRing(need, n=2)
    for sb in (bm, bdr, bv):
        sb.plans = shared

    def topk_call():
        bd.pillar_topk(verify.B, k, Hq, Hkv, 1, k, verify.seq_lens, verify.idx_count, bv.logits,
                       bv.h_logits_off, bv.lse, topk_idx, verify.idx_off, bv.ws,
                       plan=shared.next())

    def recall_call():
        bd.recall_index(drafts.B, Hkv, drafts.seq_lens, 4, 16, drafts.idx_count, drafts.idx_off,
                        bdr.idx, rec_cnt, rec_off, rec_out, plan=shared.next())

    def outputs():
        return [to_np(t).copy() for t in (bm.o, bm.lse, bm.logits, bm.idx, bdr.o, bdr.lse,
                                          bv.o, bv.lse, bv.logits, bv.idx, topk_idx, rec_out)]

    for f in (bm.step, bdr.step, bv.step, topk_call, recall_call):
        f()
        torch.cuda.synchronize()
    alone = outputs()
    for _ in range(16):
        bm.step()
        bdr.step()
        bv.step()
        topk_call()
        recall_call()
    torch.cuda.synchronize()
    for i, (a, g) in enumerate(zip(alone, outputs())):
        assert np.array_equal(a.view(np.uint8), g.view(np.uint8)), f"output {i} differs"


def test_one_plan_buffer_across_two_streams():
    """A single plan buffer used by calls alternating between two streams: each
    call waits until the GPU has finished reading the previous call's plan, so
    the results match each batch stepped alone."""
    shapes = [(6, ("uniform", 400, 3000), 2, 51), (5, ("uniform", 100, 2000), 0, 52)]
    batches = []
    for B, lengths, nv, seed in shapes:
        w = synth.Workload(name=f"oneplan{seed}", batch=B, num_qo_heads=32, num_kv_heads=8,
                           head_dim=128, dtype="bf16", spec_k=8, sparsity=Fraction(1, 20),
                           lengths=lengths, n_verify=nv, seed=seed)
        ver = [False] * B if nv == 0 else None
        batches.append(synth.make_batch(w, device=DEV, is_verify=ver))
    alone = []
    for b in batches:
        bufs = bd.StepBuffers(b)
        bufs.step()
        torch.cuda.synchronize()
        alone.append([to_np(t).copy() for t in (bufs.o, bufs.lse, bufs.idx)])
    bufs = [bd.StepBuffers(b, n_plans=1) for b in batches]
    one = bd.PlanRing(max(bu.plans.nbytes for bu in bufs), n=1)
    for bu in bufs:
        bu.plans = one
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(15):
        for s, bu in zip(streams, bufs):
            with torch.cuda.stream(s):
                bu.step()
    torch.cuda.synchronize()
    for want, bu in zip(alone, bufs):
        got = [to_np(t) for t in (bu.o, bu.lse, bu.idx)]
        for name, a, g in zip(("O", "LSE", "idx"), want, got):
            assert np.array_equal(a.view(np.uint8), g.view(np.uint8)), f"{name} differs"


def test_host_threads_step_concurrently():
    """Three host threads, each stepping its own batch on its own stream 25
    times without synchronising (ctypes releases the interpreter lock during
    the call, so the calls interleave inside the library), end bit for bit
    equal to each batch stepped alone: calls share no state in the library."""
    import threading
    shapes = [(5, 2, 71), (7, 0, 72), (4, 4, 73)]
    batches = []
    for B, nv, seed in shapes:
        w = synth.Workload(name=f"threads{seed}", batch=B, num_qo_heads=16, num_kv_heads=8,
                           head_dim=128, dtype="bf16", spec_k=4, sparsity=Fraction(1, 10),
                           lengths=("uniform", 200, 2200), n_verify=nv, seed=seed)
        ver = [False] * B if nv == 0 else ([True] * B if nv == B else None)
        batches.append(synth.make_batch(w, device=DEV, is_verify=ver))
    alone = []
    for b in batches:
        bufs = bd.StepBuffers(b)
        bufs.step()
        torch.cuda.synchronize()
        alone.append([to_np(t).copy() for t in (bufs.o, bufs.lse, bufs.logits, bufs.idx)])
    bufs = [bd.StepBuffers(b) for b in batches]
    streams = [torch.cuda.Stream() for _ in batches]
    torch.cuda.synchronize()
    errors = []

    def run(bu, st):
        try:
            torch.cuda.set_device(DEV)
            with torch.cuda.stream(st):
                for _ in range(25):
                    bu.step()
        except Exception as e:  # reported below, on the test's thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(bu, st)) for bu, st in zip(bufs, streams)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a stepping thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for want, bu, b in zip(alone, bufs, batches):
        got = [to_np(t) for t in (bu.o, bu.lse, bu.logits, bu.idx)]
        for name, a, g in zip(("O", "LSE", "logits", "idx"), want, got):
            if name == "logits" and not any(b.is_verify):
                continue  # a draft-only batch writes no logits (its buffer is a placeholder)
            assert np.array_equal(a.view(np.uint8), g.view(np.uint8)), f"{name} differs"
