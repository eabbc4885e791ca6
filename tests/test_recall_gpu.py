"""Recallable index (sinks + stored important positions + recent tokens) on the
HIP path against the oracle -- needs an MI355X.

The builder's output is integer work, so it must match the oracle bit for bit,
padding included; memory around the output segments must stay untouched.  The
lists it builds then drive draft attention (alone and inside the unified step)
and are checked against the oracle's own chain: oracle index -> oracle draft
attention, from the same seeded stored lists."""
from dataclasses import replace
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
SENTINEL = 0x5A5A5A5A


def _segments(counts, Hkv, gap):
    off, cur = [], gap
    for c in counts:
        off.append(cur)
        cur += Hkv * c + gap
    return np.asarray(off, np.int64), cur


def run_recall(Hkv, lens, S, W, stored, extra):
    """stored: per request an int32 array [Hkv][n_r]; extra: padding entries
    added to the smallest accepted output length.  Returns (out buffer on the
    host, out offsets, out counts)."""
    in_count = [a.shape[1] for a in stored]
    in_off, in_elems = _segments(in_count, Hkv, 7)
    idx_in = np.full((in_elems,), SENTINEL, np.int32)
    for a, o in zip(stored, in_off):
        idx_in[o:o + a.size] = a.reshape(-1)
    out_count = [bd.recall_length(L, n, S, W) + e for L, n, e in zip(lens, in_count, extra)]
    out_off, out_elems = _segments(out_count, Hkv, 5)
    d_in = torch.from_numpy(idx_in).to(DEV)
    d_out = torch.full((out_elems,), SENTINEL, dtype=torch.int32, device=DEV)
    print(f"[recall] Hkv={Hkv} S={S} W={W} lens={list(lens)} stored={in_count}", flush=True)
    bd.recall_index(len(lens), Hkv, lens, S, W, in_count, in_off, d_in, out_count, out_off,
                    d_out)
    torch.cuda.synchronize()
    return to_np(d_out), out_off, out_count


def check_against_oracle(oracle, Hkv, lens, S, W, stored, out, out_off, out_count):
    covered = np.zeros(out.shape, bool)
    for r, L in enumerate(lens):
        for g in range(Hkv):
            want, _ = oracle.recall_index(L, S, W, stored[r][g], out_count[r])
            a = out_off[r] + g * out_count[r]
            got = out[a:a + out_count[r]]
            assert np.array_equal(got, want), f"request {r} head {g} (L={L})"
            covered[a:a + out_count[r]] = True
    assert (out[~covered] == SENTINEL).all(), "memory outside the output lists was written"


def _stored_lists(rng, Hkv, lens):
    """Unsorted stored lists with duplicates and entries outside [0, L)."""
    out = []
    for r, L in enumerate(lens):
        n = [0, 1, 7, max(1, L // 20), L + 3][r % 5]
        a = rng.integers(-3, L + 5, size=(Hkv, n)).astype(np.int32)
        if n > 4:
            a[:, 1] = a[:, 0]  # a duplicate in every head
        out.append(a)
    return out


LENS = [1, 2, 31, 32, 33, 64, 100, 1000, 8192, 70000, 131072]


@pytest.mark.parametrize("S,W", [(0, 0), (4, 64), (4, 0), (0, 64), (16, 8), (1 << 20, 0),
                                 (0, 1 << 20), (3, 1), (40, 40)])
def test_recall_matches_oracle(oracle, S, W):
    rng = np.random.default_rng(S * 131 + W)
    Hkv = 3
    stored = _stored_lists(rng, Hkv, LENS)
    extra = [int(x) for x in rng.integers(0, 4, size=len(LENS))]
    out, off, cnt = run_recall(Hkv, LENS, S, W, stored, extra)
    check_against_oracle(oracle, Hkv, LENS, S, W, stored, out, off, cnt)


def test_recall_sorted_top_k_lists(oracle):
    """Stored lists shaped like the selection's output (distinct, ascending,
    K = ceil(L/20)), which is what a draft step receives."""
    rng = np.random.default_rng(5)
    Hkv = 8
    lens = [int(x) for x in rng.integers(100, 20000, size=9)]
    stored = [np.sort(np.stack([rng.choice(L, -(-L // 20), replace=False) for _ in range(Hkv)]),
                      axis=1).astype(np.int32) for L in lens]
    out, off, cnt = run_recall(Hkv, lens, 4, 64, stored, [0] * len(lens))
    check_against_oracle(oracle, Hkv, lens, 4, 64, stored, out, off, cnt)


def test_recall_same_buffer_disjoint_segments(oracle):
    """Stored and output lists may share one buffer when they do not overlap."""
    Hkv, L, S, W = 2, 500, 4, 32
    rng = np.random.default_rng(8)
    stored = np.sort(rng.choice(L, (Hkv, 25)), axis=1).astype(np.int32)
    n_out = bd.recall_length(L, 25, S, W)
    buf = torch.full((Hkv * 25 + Hkv * n_out,), SENTINEL, dtype=torch.int32, device=DEV)
    buf[:Hkv * 25] = torch.from_numpy(stored.reshape(-1)).to(DEV)
    bd.recall_index(1, Hkv, [L], S, W, [25], [0], buf, [n_out], [Hkv * 25], buf)
    torch.cuda.synchronize()
    got = to_np(buf)
    assert np.array_equal(got[:Hkv * 25], stored.reshape(-1)), "stored list changed"
    for g in range(Hkv):
        want, _ = oracle.recall_index(L, S, W, stored[g], n_out)
        assert np.array_equal(got[Hkv * 25 + g * n_out:Hkv * 25 + (g + 1) * n_out], want)


def _oracle_recalled(oracle, b, r, S, W, cap):
    """The oracle's recallable index of draft r from its seeded stored list."""
    Hkv, K = b.w.num_kv_heads, b.idx_count[r]
    stored = to_np(b.idx[b.idx_off[r]:b.idx_off[r] + Hkv * K]).reshape(Hkv, K)
    return np.stack([oracle.recall_index(b.seq_lens[r], S, W, stored[g], cap)[0]
                     for g in range(Hkv)])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_recalled_lists_drive_draft_attention(oracle, dtype):
    """Draft attention over recalled lists (with -1 padding) against the
    oracle's index followed by the oracle's draft attention."""
    w = synth.Workload(name=f"recall-draft-{dtype}", batch=6, num_qo_heads=32, num_kv_heads=8,
                       head_dim=128, dtype=dtype, spec_k=8, sparsity=Fraction(1, 20),
                       lengths=("uniform", 200, 3000), n_verify=0, seed=31)
    b = synth.make_batch(w, is_verify=[False] * 6)
    bd_ = b.to(DEV)
    Hq, Hkv, d = w.num_qo_heads, w.num_kv_heads, w.head_dim
    S, W = 4, 16
    cnt = [bd.recall_length(L, K, S, W) for L, K in zip(b.seq_lens, b.idx_count)]
    off = np.concatenate([[0], np.cumsum([Hkv * c for c in cnt])[:-1]]).astype(np.int64)
    rec = torch.full((int(sum(Hkv * c for c in cnt)),), SENTINEL, dtype=torch.int32, device=DEV)
    bd.recall_index(b.B, Hkv, b.seq_lens, S, W, b.idx_count, b.idx_off, bd_.idx, cnt, off, rec)
    lay = bd.layout(Hq, Hkv, d, b.q.dtype, b.num_slots, b.stride)
    q = bd_.q.contiguous()
    o = torch.empty_like(q)
    lse = torch.empty((b.B, Hq), device=DEV)
    ws = bd.workspace(bd.workspace_bytes(lay, b.B, 8, None, b.seq_lens, cnt), DEV)
    bd.draft_attn(lay, b.B, b.seq_lens, bd_.page_table, cnt, off, rec, q, bd_.k_pool,
                  bd_.v_pool, o, lse, ws)
    torch.cuda.synchronize()
    got_lists = to_np(rec)
    sm = 1.0 / np.sqrt(d)
    for r in range(b.B):
        lst = _oracle_recalled(oracle, b, r, S, W, cnt[r])
        assert np.array_equal(got_lists[off[r]:off[r] + Hkv * cnt[r]].reshape(Hkv, cnt[r]), lst)
        qh, kp, vp, ptr = parity.request_inputs(b, r)
        ro, rl = oracle.draft_request(qh[0], kp, vp, ptr, b.seq_lens[r], lst, Hkv, sm)
        parity.assert_o(to_np(o[r]), ro, dtype, f"draft {r} O")
        parity.assert_lse(to_np(lse[r]), rl, f"draft {r} LSE")


def test_recall_in_unified_step_full_size(oracle):
    """The Qwen3-8B-shaped batch (B = 128, L = 8192) with every draft reading a
    recalled list (4 sinks, 64 recent tokens): every recalled list against the
    oracle, then the unified step's sampled verify and draft outputs."""
    w = synth.QWEN3_8B
    S, W = 4, 64
    print(f"[full-size recall] {w.name} S={S} W={W}", flush=True)
    b = synth.make_batch(w, device=DEV)
    Hkv = w.num_kv_heads
    dra = [r for r in range(b.B) if not b.is_verify[r]]
    ver = [r for r in range(b.B) if b.is_verify[r]]
    cnt = {r: bd.recall_length(b.seq_lens[r], b.idx_count[r], S, W) for r in dra}
    new_off, new_cnt = list(b.idx_off), list(b.idx_count)
    cur = b.idx_elems
    for r in dra:
        new_off[r], new_cnt[r] = cur, cnt[r]
        cur += Hkv * cnt[r]
    idx = torch.cat([b.idx, torch.full((cur - b.idx_elems,), SENTINEL, dtype=torch.int32,
                                       device=DEV)])
    bd.recall_index(len(dra), Hkv, [b.seq_lens[r] for r in dra], S, W,
                    [b.idx_count[r] for r in dra], [b.idx_off[r] for r in dra], idx,
                    [cnt[r] for r in dra], [new_off[r] for r in dra], idx)
    b2 = replace(b, idx=idx, idx_off=new_off, idx_count=new_cnt, idx_elems=cur)
    bufs = bd.StepBuffers(b2)
    bufs.step()
    torch.cuda.synchronize()
    host_idx = to_np(idx)
    for r in dra:
        lst = _oracle_recalled(oracle, b, r, S, W, cnt[r])
        got = host_idx[new_off[r]:new_off[r] + Hkv * cnt[r]].reshape(Hkv, cnt[r])
        assert np.array_equal(got, lst), f"recalled list of draft {r}"
    gpu = {"o": bufs.o, "lse": bufs.lse, "logits": bufs.logits, "idx": bufs.idx}
    parity.check_whole_batch_properties(b2, gpu)
    parity.compare_sampled(oracle, b2, gpu, [ver[0]], [])
    sm = 1.0 / np.sqrt(w.head_dim)
    for r in sorted({dra[0], dra[len(dra) // 2], dra[-1]}):
        lst = _oracle_recalled(oracle, b, r, S, W, cnt[r])
        qh, kp, vp, ptr = parity.request_inputs(b, r)
        ro, rl = oracle.draft_request(qh[0], kp, vp, ptr, b.seq_lens[r], lst, Hkv, sm)
        row = b.q_indptr[r]
        parity.assert_o(to_np(bufs.o[row]), ro, w.dtype, f"O draft {r}")
        parity.assert_lse(to_np(bufs.lse[row]), rl, f"LSE draft {r}")
    del bufs, gpu, b, b2, idx
    torch.cuda.empty_cache()
