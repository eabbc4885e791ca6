"""Throughput of the unified draft/verify decode-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--workload qwen3-8b-attn-B128-L8192]

One step = one spa_unified_step call over the whole synthetic batch: verify
attention with the logits/LSE dump, draft attention over the stored index
lists, the split-K merge, score averaging and per-KV-head top-K.  Inputs are
generated on the GPU and stay resident in HBM; the timed region covers
exactly --steps steps between two device synchronisations.

Prints one JSON line with steps/s (value), attended KV tokens/s, algorithmic
HBM GB/s against the 8 TB/s peak, the dominant kernel's roofline and the
oracle's time on this machine's host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_self_speculative_pillarattn_amd import binding as bd  # noqa: E402
from sparse_self_speculative_pillarattn_amd import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak of MI355X
METRIC = "mixed draft/verify attn steps/s; attended KV tok/s; HBM GB/s vs 8 TB/s peak"
CSRC = os.path.join(ROOT, "sparse_self_speculative_pillarattn_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# --------------------------------------------------------------------------- #
# algorithmic bytes
# --------------------------------------------------------------------------- #
def algorithmic_bytes(b) -> dict:
    """Bytes the method must move per step (each byte once), by kernel.

    verify request r (L tokens, k+1 rows):  K+V rows of every position
        L*H_kv*d*2e, page-table entries L*4, Q and O (k+1)*H_q*d*e each,
        LSE (k+1)*H_q*4, logits written (k+1)*H_q*L*4; top-K then reads the k
        averaged rows' logits k*H_q*L*4 and writes H_kv*K*4.
    draft request r (K list entries per KV head): K*H_kv*(2*d*e + 4 + 4) for the
        gathered K+V rows, list entries and page-table entries, plus Q, O, LSE.
    """
    w = b.w
    e = 2 if w.dtype == "bf16" else 4
    Hq, Hkv, d, k = w.num_qo_heads, w.num_kv_heads, w.head_dim, w.spec_k
    out = dict(kv_verify=0, kv_draft=0, index=0, qo=0, logits_write=0, logits_read=0, topk_out=0,
               index_verify=0, qo_verify=0)
    tokens = 0
    for r in range(b.B):
        if b.is_verify[r]:
            L = b.seq_lens[r]
            out["kv_verify"] += L * Hkv * d * 2 * e
            out["index"] += L * 4
            out["index_verify"] += L * 4
            out["qo"] += (k + 1) * Hq * (2 * d * e + 4)
            out["qo_verify"] += (k + 1) * Hq * (2 * d * e + 4)
            out["logits_write"] += (k + 1) * Hq * L * 4
            out["logits_read"] += k * Hq * L * 4
            out["topk_out"] += Hkv * b.idx_count[r] * 4
            tokens += L
        else:
            K = b.idx_count[r]
            out["kv_draft"] += K * Hkv * d * 2 * e
            out["index"] += K * Hkv * 8
            out["qo"] += Hq * (2 * d * e + 4)
            tokens += K
    out["bytes_min"] = (out["kv_verify"] + out["kv_draft"] + out["index"] + out["qo"] +
                        out["topk_out"])
    out["bytes_method"] = out["bytes_min"] + out["logits_write"] + out["logits_read"]
    # what the attention launch itself must move: everything but the top-K stage
    out["attn_launch"] = (out["kv_verify"] + out["kv_draft"] + out["index"] + out["qo"] +
                          out["logits_write"])
    # with overlap, the verify and draft attention are separate launches
    out["attn_verify_launch"] = (out["kv_verify"] + out["index_verify"] + out["qo_verify"] +
                                 out["logits_write"])
    out["attn_draft_launch"] = out["attn_launch"] - out["attn_verify_launch"]
    out["attended_tokens"] = tokens
    return out


def mfma_flops(b) -> dict:
    """Dense multiply-add work of the attention launch's MFMA tiles, counted
    as 2 FLOPs per multiply-add: S = Q K^T and O = P V over every (row, query
    head, position) the method attends.  A verify request contributes
    4*(k+1)*H_q*d*L, a draft request 4*H_q*d*K (the bf16 path runs both on the
    MFMA tile; rows padded up to the 16-row MFMA tile are not counted)."""
    w = b.w
    Hq, d, k = w.num_qo_heads, w.head_dim, w.spec_k
    fv = sum(4 * (k + 1) * Hq * d * b.seq_lens[r] for r in range(b.B) if b.is_verify[r])
    fd = sum(4 * Hq * d * b.idx_count[r] for r in range(b.B) if not b.is_verify[r])
    return {"verify": fv, "draft": fd, "total": fv + fd}


# --------------------------------------------------------------------------- #
# counter-based traffic, valid only for the kernel source it was taken on
# --------------------------------------------------------------------------- #
# the sources that decide what the step's kernels do and move: the kernels,
# their parameter and plan layouts, and the host planning in api.cpp (the
# scheduler and the bandwidth probe are left out)
STEP_SOURCES = ("api.cpp", "kernels.hip", "spa_kernels.h", "spa_plan.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in STEP_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def recorded_mfma(workload: str):
    """MFMA counters of one attention launch (bf16 MFMA FLOPs issued, MFMA busy
    share of the SIMDs) from a committed summary, or None when none exists for
    this workload or the kernels changed since."""
    path = os.path.join(PROFILES, f"attn_kernel_{workload}_mfma.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"source_sha256:\s*([0-9a-f]+)", text)
    fl = re.search(r"mfma_flops_bf16_per_launch:\s*([0-9.eE+]+)", text)
    ut = re.search(r"mfma_util_pct:\s*([0-9.eE+]+)", text)
    if not src or not fl or not ut or src.group(1) != kernel_source_hash():
        return None
    return {"mfma_flops_issued_per_launch": float(fl.group(1)), "mfma_util_pct": float(ut.group(1))}


def recorded_traffic(workload: str):
    """HBM bytes per attention launch from a committed counter summary, or None
    when none exists for this workload or the kernels changed since."""
    path = os.path.join(PROFILES, f"attn_kernel_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"source_sha256:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


# --------------------------------------------------------------------------- #
# CPU baseline: the oracle on this machine's host cores
# --------------------------------------------------------------------------- #
def compact_for_oracle(b):
    """Host copies of exactly what the requests read: the pool rows their page
    tables reference, re-laid-out in page-table order (results do not depend on
    where a slot lives)."""
    lens = b.seq_lens
    stride = max(lens)
    flat = torch.cat([b.page_table[r, :lens[r]].long() for r in range(b.B)])
    kp = b.k_pool.index_select(0, flat).cpu()
    vp = b.v_pool.index_select(0, flat).cpu()
    pt = np.zeros((b.B, stride), np.int32)
    off = 0
    for r in range(b.B):
        pt[r, :lens[r]] = np.arange(off, off + lens[r], dtype=np.int32)
        off += lens[r]

    def host(t):
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    return dict(k=b.w.spec_k, Hq=b.w.num_qo_heads, Hkv=b.w.num_kv_heads,
                sm_scale=1.0 / np.sqrt(b.w.head_dim), is_verify=b.is_verify, seq_lens=lens,
                q_indptr=b.q_indptr, page_table=pt, q=host(b.q.cpu()), k_pool=host(kp),
                v_pool=host(vp), idx_count=b.idx_count, idx_off=b.idx_off,
                idx=host(b.idx.cpu()), logits_off=b.logits_off, logits_elems=b.logits_elems)


def cpu_baseline(b, repeats: int) -> dict:
    from oracle import Oracle  # the oracle is only ever used for this baseline leg
    orc = Oracle()
    inp = compact_for_oracle(b)
    cores = len(os.sched_getaffinity(0))
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        orc.step(**inp, nthreads=cores)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": 1.0 / t, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole step ({b.B} requests), median of {repeats} runs, "
                      f"{t:.2f} s each; fp64 C oracle, one thread per request",
            "seconds_per_step": t, "cpu": cpu_model}


# --------------------------------------------------------------------------- #
# extra measurements (not part of the one-line result)
# --------------------------------------------------------------------------- #
def _time_steps(fn, steps: int, warmup: int) -> float:
    """Mean microseconds per call of ``fn`` over ``steps`` back-to-back calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3


def launch_times(run, names, n: int) -> dict:
    """Mean microseconds of each named launch over n calls of run(opts), every
    call with its own timing events (recorded on the launch stream)."""
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    opts = [bd.Options(num_cus=props.multi_processor_count, timing=names) for _ in range(n)]
    for o in opts:
        run(o)
    torch.cuda.synchronize()
    out = {}
    for nm in names:
        out[nm] = float(np.mean([o.elapsed_ms(nm) for o in opts])) * 1e3
    return out


def sparsity_sweep(w, dev, steps: int, warmup: int):
    """Draft-only batches (every request a draft, the workload's shapes) at a
    range of sparsities: per-step time should fall close to proportionally to s."""
    from dataclasses import replace
    from fractions import Fraction
    L = w.lengths[1] if w.lengths[0] == "fixed" else 8192
    rows = []
    for s in (Fraction(1, 100), Fraction(1, 50), Fraction(1, 20), Fraction(1, 10), Fraction(1, 5),
              Fraction(1, 2), Fraction(1, 1)):
        ws = replace(w, sparsity=s, name=f"{w.name}-draft-only-s{float(s)}")
        b = synth.uniform_batch(ws, w.batch, L, [0] * w.batch, device=dev, seed=w.seed)
        bufs = bd.StepBuffers(b)
        # at least 50 warm-up and 200 timed steps: over a short window the
        # first tens of calls on a new batch, still slow, set the average of
        # steps this short
        us = _time_steps(bufs.step, max(steps, 200), max(warmup, 50))
        kern = {nm: round(v, 1) for nm, v in launch_times(bufs.step, ("attn",), 10).items()}
        alg = algorithmic_bytes(b)
        rows.append({"s": float(s), "K": b.idx_count[0], "us_per_step": round(us, 1), "kernel_us": kern,
                     "bytes_min": alg["bytes_min"],
                     "hbm_gbps_min": round(alg["bytes_min"] / (us * 1e-6) / 1e9, 1)})
        del bufs, b
        torch.cuda.empty_cache()
    t1 = rows[-1]["us_per_step"]
    for r in rows:
        r["t_over_t1"] = round(r["us_per_step"] / t1, 4)
    print(json.dumps({"sparsity_sweep": w.name, "batch": w.batch, "L": L, "rows": rows}))


def unified_vs_sequential(w, dev, steps: int, warmup: int):
    """The unified step against the three entry points called one after the
    other on the same batch (verify attention, PillarAttn top-K, draft attention)."""
    b = synth.make_batch(w, device=dev)
    bufs = bd.StepBuffers(b)
    k, Hq, Hkv, d = w.spec_k, w.num_qo_heads, w.num_kv_heads, w.head_dim
    lay = bufs.lay
    ver = [r for r in range(b.B) if b.is_verify[r]]
    dra = [r for r in range(b.B) if not b.is_verify[r]]
    qv = torch.cat([b.q[b.q_indptr[r]:b.q_indptr[r + 1]] for r in ver]).contiguous()
    ptv = torch.stack([b.page_table[r] for r in ver]).contiguous()
    lv = [b.seq_lens[r] for r in ver]
    loff = np.concatenate([[0], np.cumsum([(k + 1) * Hq * L for L in lv])[:-1]]).astype(np.int64)
    ov = torch.empty_like(qv)
    lsev = torch.empty((qv.shape[0], Hq), device=dev)
    lgv = torch.empty((int(sum((k + 1) * Hq * L for L in lv)),), device=dev)
    Kv = [b.idx_count[r] for r in ver]
    ioff = np.concatenate([[0], np.cumsum([Hkv * K for K in Kv])[:-1]]).astype(np.int64)
    idxv = torch.zeros((int(sum(Hkv * K for K in Kv)),), dtype=torch.int32, device=dev)
    qd = torch.stack([b.q[b.q_indptr[r]] for r in dra]).contiguous()
    ptd = torch.stack([b.page_table[r] for r in dra]).contiguous()
    ld = [b.seq_lens[r] for r in dra]
    Kd = [b.idx_count[r] for r in dra]
    doff = np.concatenate([[0], np.cumsum([Hkv * K for K in Kd])[:-1]]).astype(np.int64)
    idxd = torch.cat([b.idx[b.idx_off[r]:b.idx_off[r] + Hkv * b.idx_count[r]] for r in dra])
    od = torch.empty_like(qd)
    lsed = torch.empty((len(dra), Hq), device=dev)
    ws = bd.workspace(max(bd.workspace_bytes(lay, len(ver), k, [1] * len(ver), lv, Kv),
                          bd.workspace_bytes(lay, len(dra), 1, None, ld, Kd)), dev)

    def sequential():
        bd.verify_attn(lay, len(ver), k, lv, ptv, qv, b.k_pool, b.v_pool, ov, lsev, lgv, loff, ws)
        bd.pillar_topk(len(ver), k, Hq, Hkv, 1, k, lv, Kv, lgv, loff, lsev, idxv, ioff, ws)
        bd.draft_attn(lay, len(dra), ld, ptd, Kd, doff, idxd.contiguous(), qd, b.k_pool, b.v_pool,
                      od, lsed, ws)

    uni = _time_steps(bufs.step, steps, warmup)
    seq = _time_steps(sequential, steps, warmup)
    print(json.dumps({"unified_vs_sequential": w.name, "unified_us": round(uni, 1),
                      "sequential_us": round(seq, 1), "speedup": round(seq / uni, 3)}))


def recall_measure(w, dev, steps: int, warmup: int, n_sink: int, n_recent: int):
    """The recallable index on the workload's drafts: the index launch alone,
    and the unified step whose drafts read recalled lists (index launch + step)
    against the same step over the stored lists."""
    from dataclasses import replace
    b = synth.make_batch(w, device=dev)
    Hkv = w.num_kv_heads
    dra = [r for r in range(b.B) if not b.is_verify[r]]
    cnt = [bd.recall_length(b.seq_lens[r], b.idx_count[r], n_sink, n_recent) for r in dra]
    new_off, new_cnt = list(b.idx_off), list(b.idx_count)
    cur = b.idx_elems
    for r, c in zip(dra, cnt):
        new_off[r], new_cnt[r] = cur, c
        cur += Hkv * c
    idx = torch.cat([b.idx, torch.zeros((cur - b.idx_elems,), dtype=torch.int32, device=dev)])
    b2 = replace(b, idx=idx, idx_off=new_off, idx_count=new_cnt, idx_elems=cur)
    plain = bd.StepBuffers(b)
    recalled = bd.StepBuffers(b2)
    lens_d = np.asarray([b.seq_lens[r] for r in dra], np.int32)
    inc_d = np.asarray([b.idx_count[r] for r in dra], np.int32)
    inoff_d = np.asarray([b.idx_off[r] for r in dra], np.int64)
    outc_d = np.asarray(cnt, np.int32)
    outoff_d = np.asarray([new_off[r] for r in dra], np.int64)

    def recall():  # stored lists and recalled lists live in the step's own idx buffer
        bd.recall_index(len(dra), Hkv, lens_d, n_sink, n_recent, inc_d, inoff_d, recalled.idx,
                        outc_d, outoff_d, recalled.idx)

    def step_with_recall():
        recall()
        recalled.step()

    t_plain = _time_steps(plain.step, steps, warmup)
    t_recall = _time_steps(recall, steps, warmup)
    t_both = _time_steps(step_with_recall, steps, warmup)
    kern = {nm: round(v, 2) for nm, v in
            launch_times(recalled.step, ("attn", "post", "select"), 10).items()}
    # the index launch alone, between two events on the stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(10)]
    for a, z in ev:
        a.record()
        recall()
        z.record()
    torch.cuda.synchronize()
    kern["recall"] = round(float(np.mean([a.elapsed_time(z) for a, z in ev])) * 1e3, 2)
    # the index launch must read each stored list and write each output list once
    rec_bytes = int(sum(Hkv * (k_in + k_out) * 4 for k_in, k_out in zip(inc_d, cnt)))
    rec_us = kern.get("recall", float("nan"))
    gbps = rec_bytes / (rec_us * 1e-6) / 1e9
    print(json.dumps({
        "recall": w.name, "n_sink": n_sink, "n_recent": n_recent, "n_draft": len(dra),
        "stored_per_head": int(inc_d.mean()), "recalled_per_head": float(np.mean(cnt)),
        "step_us_stored_lists": round(t_plain, 1), "recall_launch_us_back_to_back": round(t_recall, 1),
        "step_us_with_recall": round(t_both, 1), "kernel_us_with_recall": kern,
        "recall_roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 5),
                            "algorithmic_bytes_per_launch": rec_bytes}}), flush=True)


def quality_measure(w, dev, steps: int, warmup: int, top_t: int):
    """How well index lists capture the drafts' exact attention: each draft
    query is scored over its whole context (spa_verify_attn, spec_k = 1, the
    query in row 1), then spa_list_quality measures the stored list (stale:
    the workload's pillar drift applies) and a fresh list (PillarAttn's top-K
    of the draft row itself, averaged over its GQA group, same K)."""
    b = synth.make_batch(w, device=dev)
    Hq, Hkv, d = w.num_qo_heads, w.num_kv_heads, w.head_dim
    dra = [r for r in range(b.B) if not b.is_verify[r]]
    nd = len(dra)
    q2 = torch.stack([torch.stack([b.q[b.q_indptr[r]], b.q[b.q_indptr[r]]]) for r in dra])
    q2 = q2.reshape(-1, Hq, d).contiguous()
    pt = torch.stack([b.page_table[r] for r in dra]).contiguous()
    lens = [b.seq_lens[r] for r in dra]
    K = [b.idx_count[r] for r in dra]
    loff = np.concatenate([[0], np.cumsum([2 * Hq * L for L in lens])[:-1]]).astype(np.int64)
    logits = torch.empty((int(sum(2 * Hq * L for L in lens)),), device=dev)
    lse = torch.empty((2 * nd, Hq), device=dev)
    o = torch.empty_like(q2)
    lay = bd.layout(Hq, Hkv, d, b.q.dtype, b.num_slots, b.stride)
    ws = bd.workspace(bd.workspace_bytes(lay, nd, 1, [1] * nd, lens, K), dev)
    ioff = np.concatenate([[0], np.cumsum([Hkv * k for k in K])[:-1]]).astype(np.int64)
    stale = torch.cat([b.idx[b.idx_off[r]:b.idx_off[r] + Hkv * b.idx_count[r]] for r in dra])
    fresh = torch.zeros_like(stale)
    qws = bd.workspace(bd.list_quality_workspace_bytes(nd, Hq, lens), dev)
    top = torch.empty((nd, Hq, top_t), dtype=torch.int32, device=dev)
    cov = torch.empty((nd, Hq), device=dev)
    rec = torch.empty((nd, Hq), device=dev)

    def score():
        bd.verify_attn(lay, nd, 1, lens, pt, q2, b.k_pool, b.v_pool, o, lse, logits, loff, ws)

    def quality(lists):
        bd.list_quality(nd, 1, Hq, Hkv, 1, top_t, lens, logits, loff, lse, K, ioff, lists, top, cov,
                        rec, qws)

    score()
    bd.pillar_topk(nd, 1, Hq, Hkv, 1, 1, lens, K, logits, loff, lse, fresh, ioff, ws)
    out = {"quality": w.name, "n_draft": nd, "top_t": top_t,
           "pillar_drift": w.pillar_drift, "mean_L": round(float(np.mean(lens)), 1),
           "mean_K": round(float(np.mean(K)), 1)}
    for name, lists in (("stale", stale), ("fresh", fresh)):
        quality(lists)
        torch.cuda.synchronize()
        out[name] = {"coverage_mean": round(float(cov.mean()), 4),
                     "coverage_p10": round(float(torch.quantile(cov.flatten(), 0.1)), 4),
                     f"recall@{top_t}_mean": round(float(rec.mean()), 4),
                     f"recall@{top_t}_p10": round(float(torch.quantile(rec.flatten(), 0.1)), 4)}
    out["score_launch_us_back_to_back"] = round(_time_steps(score, steps, warmup), 1)
    out["quality_launch_us_back_to_back"] = round(_time_steps(lambda: quality(stale), steps, warmup), 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(10)]
    for a, z in ev:
        a.record()
        quality(stale)
        z.record()
    torch.cuda.synchronize()
    q_us = float(np.mean([a.elapsed_time(z) for a, z in ev])) * 1e3  # incl. the release launch
    # the row's logits read once, its softmax written once and read back by the
    # selection, the lists read once; top-T, coverage and recall written
    qbytes = int(sum(Hq * L * 4 * 3 for L in lens) + sum(Hkv * k * 4 for k in K)
                 + nd * Hq * (top_t * 4 + 8))
    out["quality_launch_us"] = round(q_us, 2)
    out["quality_roofline"] = {"bound": "hbm", "achieved": round(qbytes / (q_us * 1e-6) / 1e9, 1),
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                               "frac": round(qbytes / (q_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                               "algorithmic_bytes_per_launch": qbytes}
    print(json.dumps(out), flush=True)


def stride_quality_measure(w, dev, sigmas, top_t: int = 10, n_req=None):
    """The verify's PillarAttn lists against the k drafts of the following
    stride (stride_quality.StrideRun): per stride position i = 1..k, the
    mean and 10th percentile over (request, query head) of attention coverage
    and recall@top_t, for the verify's lists and for a fresh top-K of each
    draft row (same K), at each query drift sigma."""
    from sparse_self_speculative_pillarattn_amd.stride_quality import StrideRun
    b, vlens = synth.stride_batch(w, device=dev, n_req=n_req)
    out = {"stride_quality": w.name, "requests": b.B, "spec_k": w.spec_k,
           "sparsity": str(w.sparsity), "top_t": top_t, "mean_L": round(float(np.mean(vlens)), 1),
           "sigmas": {}}

    def stats(x):
        x = x.flatten().float()
        return {"mean": round(float(x.mean()), 4), "p10": round(float(torch.quantile(x, 0.1)), 4)}

    for sigma in sigmas:
        print(f"[bench] stride quality {w.name} sigma={sigma}", file=sys.stderr, flush=True)
        res = StrideRun(b, vlens, sigma, seed=w.seed, top_t=top_t).run()
        per = []
        for i in sorted(res):
            row = {"i": i}
            for kind in ("pillar", "fresh"):
                cov, rec = res[i][kind]
                row[kind] = {"coverage": stats(cov), f"recall@{top_t}": stats(rec)}
            per.append(row)
        out["sigmas"][str(sigma)] = {"cos_q_i_vs_verify_row_k": [
            round(1.0 / float(np.sqrt(1 + i * sigma * sigma)), 4) for i in range(1, w.spec_k + 1)],
            "positions": per}
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def _mix_setup(w):
    """Tiles, stores per tile and pool size of the workload's attention launch
    for the probe (include/spa_probe.h)."""
    meta = synth.make_meta(w)
    Hkv = w.num_kv_heads
    chunks = 0
    for r in range(w.batch):
        n = meta.seq_lens[r] if meta.is_verify[r] else meta.idx_count[r]
        chunks += Hkv * (-(-n // 32))
    logits_bytes = sum((w.spec_k + 1) * w.num_qo_heads * meta.seq_lens[r] * 4
                       for r in range(w.batch) if meta.is_verify[r])
    wbytes = min(4096, (logits_bytes // chunks) // 16 * 16)
    return meta, chunks, wbytes


def mix_ceiling(w, dev, mixes, configs, reps: int = 20, settle: bool = True) -> dict:
    """Runs the probe over `mixes` (name -> (scattered, with_stores)) and
    `configs` ((depth, workgroups) pairs); returns per mix every run and the
    best."""
    assert w.head_dim == 128 and w.dtype == "bf16", "the probe replays 256-byte bf16 rows"
    meta, chunks, wbytes = _mix_setup(w)
    Hkv, nslots = w.num_kv_heads, meta.num_slots
    pool_bytes = nslots * Hkv * 256
    read_bytes = chunks * 2 * 32 * 256
    kp = torch.empty((pool_bytes,), dtype=torch.uint8, device=dev)
    vp = torch.empty_like(kp)
    out = torch.empty((max(wbytes, 16) * chunks,), dtype=torch.uint8, device=dev)
    sink = torch.zeros((4,), dtype=torch.int32, device=dev)
    if settle:  # loaded clocks first (see the settling copies of the main measurement)
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(150):
            dst.copy_(src)
        del src, dst
    res = {"tiles": chunks, "pool_bytes_each": pool_bytes, "read_bytes": read_bytes,
           "write_bytes_per_tile": wbytes, "write_bytes": wbytes * chunks, "reps": reps,
           "mixes": {}}
    for name, (rnd, stores) in mixes.items():
        wb = wbytes if stores else 0
        runs = []
        for depth, grid in configs:
            fn = lambda: bd.probe_ceiling(kp, vp, nslots, Hkv, chunks, rnd, depth,
                                          out if wb else None, wb, grid, sink)
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            runs.append({"depth": depth, "grid": grid, "us": round(us, 1),
                         "GB_s": round((read_bytes + wb * chunks) / (us * 1e-6) / 1e9, 1)})
        best = max(runs, key=lambda x: x["GB_s"])
        res["mixes"][name] = {"best": best, "frac_of_peak": round(best["GB_s"] / HBM_PEAK_GBPS, 4),
                              "runs": runs}
    del kp, vp, out
    torch.cuda.empty_cache()
    return res


MIXES = {"launch_mix": (True, True), "scattered_reads": (True, False),
         "sequential_mix": (False, True), "sequential_reads": (False, False)}


def ceiling_measure(w, dev, reps: int = 20):
    """Attainable bandwidth of the attention launch's own access mix
    (include/spa_probe.h): the workload's (request, KV head) tiles of 32
    positions, each reading the K and V rows (256 bytes each, non-temporal) of
    32 slots of a pool the workload's size, plus dependent sequential stores
    of the verify logits' total spread over the tiles (the launch's
    read:write ratio).  Four mixes -- scattered or consecutive slots, with or
    without the stores -- at 1, 2 and 4 tiles in flight per workgroup and
    1024 to 4096 workgroups; the best of each mix is its ceiling."""
    from types import SimpleNamespace
    meta, chunks, wbytes = _mix_setup(w)
    print(f"[bench] ceiling {w.name}: {chunks} tiles, {wbytes} B stored per tile",
          file=sys.stderr, flush=True)
    configs = [(d, g) for d in (1, 2, 4) for g in (1024, 2048, 4096)]
    res = {"ceiling": w.name, **mix_ceiling(w, dev, MIXES, configs, reps)}
    alg = algorithmic_bytes(SimpleNamespace(w=w, B=w.batch, is_verify=meta.is_verify,
                                            seq_lens=meta.seq_lens, idx_count=meta.idx_count))
    res["attn_launch_algorithmic_bytes"] = alg["attn_launch"]
    print(json.dumps(res), flush=True)


def offload_measure(w, dev, steps: int, warmup: int, mb_per_step=(0.52, 4.0, 18.9),
                    block_slots: int = 64, concurrent_only: bool = False):
    """Host-link traffic beside the step (include/spa_kvcache.h): per step,
    KV blocks leave the device for pinned host chunks and as many come back,
    on a copy stream, while the unified step runs back to back on the compute
    stream.  X is the MB moved per step, both directions together: 18.9 MB is the new KV of one
    decode step of the whole Qwen3-8B model at batch 128 (36 layers x 8 KV
    heads x 128 x 2 (K, V) x 2 bytes x 128 requests), the pages' ~18 MB per
    step; 0.52 MB is one layer's share of it.  Blocks of block_slots slots are
    moved in consecutive runs (one copy per pool per run) and, for the worst
    case, every other block (one copy per block).  Reports per X: the step
    time alone and with the copies running, the copies' GB/s alone and beside
    the step, and whether the copy stream kept up.  concurrent_only: only the
    consecutive runs beside the steps (for a trace of the overlap)."""
    b = synth.make_batch(w, device=dev)
    bufs = bd.StepBuffers(b)
    lay = bd.layout(w.num_qo_heads, w.num_kv_heads, w.head_dim, b.q.dtype, 4096 * block_slots,
                    b.stride)
    bb = bd.kv_block_bytes(lay, block_slots)
    nblk = 4096
    kp = torch.zeros((nblk * bb,), dtype=torch.uint8, device=dev)
    vp = torch.zeros_like(kp)
    ka = torch.zeros((nblk * bb,), dtype=torch.uint8, pin_memory=True)
    va = torch.zeros_like(ka, pin_memory=True)
    copy = torch.cuda.Stream(dev)
    comp = torch.cuda.current_stream(dev)

    def moves(i, n, scattered):
        # step i's blocks: a window that walks through the pool; offload the
        # first half, prefetch the second (different blocks and chunks)
        step = 2 if scattered else 1
        base = (i * 2 * n * step) % (nblk - 2 * n * step)
        ids = base + np.arange(2 * n) * step
        return ids[:n], ids[n:]

    def copies(i, n, scattered):
        off, pre = moves(i, n, scattered)
        if len(off):
            bd.kv_offload(lay, block_slots, off, off, kp, vp, ka, va, stream=copy)
        if len(pre):
            bd.kv_prefetch(lay, block_slots, pre, pre, ka, va, kp, vp, stream=copy)

    def timed(with_steps, with_copies, n, scattered):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        e0.record(comp)
        copy.wait_event(e0)
        for i in range(steps):
            if with_copies:
                copies(i, n, scattered)
            if with_steps:
                bufs.step()
        e1.record(comp)
        c1.record(copy)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3, e0.elapsed_time(c1) * 1e3

    for _ in range(warmup):
        bufs.step()
    copies(0, 4, False)
    torch.cuda.synchronize()
    base_us, _ = timed(True, False, 0, False)
    out = {"offload": w.name, "block_slots": block_slots, "block_bytes_per_pool": bb,
           "steps": steps, "step_us_alone": round(base_us / steps, 1), "runs": []}
    for mb in mb_per_step:
        # n blocks each way: 2 n blocks x 2 pools x bb bytes = mb * 1e6
        n = max(1, int(round(mb * 1e6 / (4 * bb))))
        moved = 4 * n * bb
        for scattered in ((False,) if concurrent_only else (False, True)):
            c_alone = float("nan") if concurrent_only else timed(False, True, n, scattered)[1]
            t_both, c_both = timed(True, True, n, scattered)
            out["runs"].append({
                "mb_per_step": round(moved / 1e6, 3), "blocks_each_way": n,
                "copies_per_step": 4 * (n if scattered else 1),
                "runs": "scattered" if scattered else "consecutive",
                "copy_gbps_alone": None if concurrent_only else
                round(moved * steps / (c_alone * 1e-6) / 1e9, 1),
                "step_us_with_copies": round(t_both / steps, 1),
                "step_slowdown": round(t_both / base_us - 1, 4),
                "copy_gbps_beside_steps": round(moved * steps / (c_both * 1e-6) / 1e9, 1),
                "copies_kept_up": bool(c_both <= t_both * 1.02)})
    print(json.dumps(out), flush=True)


def per_call(w, dev, n: int):
    """The first n calls on a freshly generated batch, each bracketed by its
    own events (whole call, and the attention, post-pass and selection
    launches): where the extra time of the first calls goes."""
    b = synth.make_batch(w, device=dev)
    bufs = bd.StepBuffers(b)
    props = torch.cuda.get_device_properties(dev)
    opts = [bd.Options(num_cus=props.multi_processor_count, timing=("attn", "post", "select"))
            for _ in range(n)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host = []
    for i in range(n):
        ev[i][0].record()
        bufs.step(opts[i])
        ev[i][1].record()
        host.append(time.perf_counter() - t0)
    torch.cuda.synchronize()
    rows = []
    for i in range(n):
        rows.append({"call": i + 1, "step_us": round(ev[i][0].elapsed_time(ev[i][1]) * 1e3, 1),
                     **{k: round(opts[i].elapsed_ms(k) * 1e3, 1) for k in ("attn", "post", "select")},
                     "host_issue_ms": round(host[i] * 1e3, 3)})
    print(json.dumps({"per_call": w.name, "calls": rows}), flush=True)


def clock_ramp(w, dev, n: int = 150, group: int = 5):
    """The same calls after the GPU sat idle and after it was kept busy with
    unrelated HBM copies: per-call time in groups of `group` calls (one event
    pair per group).  After an idle period the first tens of calls run slower
    while the GPU's clocks settle; after busy work they do not."""
    b = synth.make_batch(w, device=dev)
    bufs = bd.StepBuffers(b)
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    big2 = torch.empty_like(big)
    torch.cuda.synchronize()

    def groups():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n // group + 1)]
        ev[0].record()
        for i in range(n // group):
            for _ in range(group):
                bufs.step()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [round(ev[i].elapsed_time(ev[i + 1]) * 1e3 / group, 1) for i in range(n // group)]

    out = {"clock_ramp": w.name, "calls_per_group": group}
    groups()  # first use of the batch
    time.sleep(0.2)
    out["after_200ms_idle"] = groups()
    for _ in range(150):  # about 40 ms of 1 GiB device copies
        big2.copy_(big)
    out["after_40ms_of_copies"] = groups()
    out["back_to_back"] = groups()
    time.sleep(0.05)
    out["after_50ms_idle"] = groups()
    print(json.dumps(out), flush=True)


def scheduler_measure(w, dev, steps: int, warmup: int, modes=("plain", "delayed"),
                      output=(64, 1024)):
    """Decode steps under the phase-bucket scheduler (include/spa_sched.h),
    with and without delayed verification: w.batch slots, the workload's heads,
    k and s, prompts from its length recipe (a log-normal recipe is drawn
    uniformly over its clip range here), outputs uniform over `output` so that
    requests retire and new ones join during the run.  Each step is planned on
    the host (scheduler, initial lists of new requests), launched and
    committed.  Two host disciplines per mode: "host_waits" -- before planning
    a step the host waits for the step whose verify outcomes it needs (the one
    before, or with delayed verification the one before that), as a server
    that reads verify results back must; "run_ahead" -- the host never waits
    (the GPU-bound rate).  Reports steps/s over the timed steps and the
    per-step verify count and query rows against slots/C and (2k+1)/(k+1) B.
    Python's cyclic garbage collector is paused during the timed steps (a
    full collection in a process that has imported torch takes tens of ms)."""
    import gc
    from sparse_self_speculative_pillarattn_amd.sched_driver import SchedDriver
    kind = w.lengths[0]
    prompt = (w.lengths[1], w.lengths[1]) if kind == "fixed" else \
        (w.lengths[1], w.lengths[2]) if kind == "uniform" else (w.lengths[3], w.lengths[4])
    props = torch.cuda.get_device_properties(dev)
    out = {"scheduler": w.name, "slots": w.batch, "spec_k": w.spec_k,
           "sparsity": str(w.sparsity), "prompt": list(prompt), "output": list(output),
           "steps": steps, "warmup": warmup, "modes": {}}
    for mode in modes:
        delayed = mode == "delayed"
        print(f"[bench] scheduler {w.name} delayed={delayed}", file=sys.stderr, flush=True)
        drv = SchedDriver(w.batch, w.spec_k, w.num_qo_heads, w.num_kv_heads, w.head_dim,
                          w.sparsity, prompt, output, delayed=delayed, seed=w.seed, device=dev,
                          dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                          num_cus=props.multi_processor_count)
        res = {}
        for waits in (True, False):
            for _ in range(warmup):
                drv.step(dependent=waits)
            torch.cuda.synchronize()
            s0 = drv.sched.stats()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            rows, nv, kv = [], [], []
            gc.collect()
            gc.disable()
            wall0 = time.perf_counter()
            e0.record()
            for _ in range(steps):
                st = drv.step(dependent=waits)
                a = drv.last[1]
                rows.append(st.rows)
                nv.append(st.n_verify)
                kv.append(int(np.where(a["is_verify"] == 1, a["seq_lens"].astype(np.int64),
                                       a["idx_count"]).sum()))
            e1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - wall0
            gc.enable()
            gpu_ms = e0.elapsed_time(e1)
            s1 = drv.sched.stats()
            k, S = w.spec_k, w.batch
            C = k + 1 + int(delayed)
            rows_np = np.asarray(rows, np.float64)
            res["host_waits" if waits else "run_ahead"] = {
                "steps_per_s": round(steps / (gpu_ms * 1e-3), 1),
                "us_per_step": round(gpu_ms * 1e3 / steps, 1),
                "host_wall_us_per_step": round(wall * 1e6 / steps, 1),
                "verify_per_step": {"min": int(min(nv)), "max": int(max(nv)),
                                    "mean": round(float(np.mean(nv)), 3),
                                    "slots_over_C": round(S / C, 3)},
                "rows_per_step": {"min": int(rows_np.min()), "max": int(rows_np.max()),
                                  "mean": round(float(rows_np.mean()), 2),
                                  "cv": round(float(rows_np.std() / rows_np.mean()), 4),
                                  "2k+1_over_k+1_B": round((2 * k + 1) / (k + 1) * S, 2)},
                "attended_kv_tokens_per_s": round(float(np.sum(kv)) / (gpu_ms * 1e-3), 1),
                "tokens_committed_per_s": round((s1["committed"] - s0["committed"]) /
                                                (gpu_ms * 1e-3), 1),
                "accepted_per_verify": round((s1["accepted"] - s0["accepted"]) /
                                             max(1, s1["verifies"] - s0["verifies"]), 3),
                "new_requests": s1["retired"] - s0["retired"]}
        out["modes"]["delayed" if delayed else "plain"] = res
        del drv
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


# --------------------------------------------------------------------------- #
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # Steady state: over 10 warm-up and 50 timed steps the first calls on a
    # new batch, still slow, made the Qwen3-8B-shaped step 196 us instead of
    # the 191 us it keeps afterwards.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=synth.QWEN3_8B.name, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--settle-copies", type=int, default=150,
                    help="1 GiB device copies run at the end of the setup, before the warm-up, "
                         "so that the measured steps start from loaded clocks (0: none)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed one by one after a 512 MB cache-flushing write")
    ap.add_argument("--cpu-repeats", type=int, default=15,
                    help="oracle runs of the whole step (about 0.8 s each on 16 EPYC cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the access-mix ceiling measurement of the main line")
    ap.add_argument("--sparsity-sweep", action="store_true",
                    help="only run the draft-only sparsity sweep and print its JSON line")
    ap.add_argument("--unified-vs-sequential", action="store_true",
                    help="only compare the unified step with the three entry points in sequence")
    ap.add_argument("--recall", type=int, nargs=2, default=None, metavar=("SINKS", "RECENT"),
                    help="only measure the recallable index (SINKS sink tokens, RECENT recent "
                         "tokens) on the workload's drafts and print its JSON line")
    ap.add_argument("--quality", type=int, default=0, metavar="T",
                    help="only measure stale and fresh index lists against the drafts' exact "
                         "attention (coverage, recall of the top T) and print its JSON line")
    ap.add_argument("--per-call", type=int, default=0, metavar="N",
                    help="only time the first N calls on a fresh batch one by one and print "
                         "their JSON line")
    ap.add_argument("--clock-ramp", action="store_true",
                    help="only time calls after an idle period and after busy work (groups "
                         "of 5) and print their JSON line")
    ap.add_argument("--scheduler", nargs="?", const="both", default=None,
                    choices=("both", "plain", "delayed"),
                    help="only run decode steps under the phase-bucket scheduler (plain and/or "
                         "delayed verification; --steps timed after --warmup) and print their "
                         "JSON line")
    ap.add_argument("--stride-quality", type=float, nargs="+", default=None, metavar="SIGMA",
                    help="only measure the verify's PillarAttn lists against the next k drafts "
                         "(queries drifting by SIGMA per step) and print the JSON line")
    ap.add_argument("--stride-requests", type=int, default=None,
                    help="with --stride-quality: the first N requests of the workload")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the attainable bandwidth of the attention launch's access "
                         "mix (libspa_probe) on the workload and print its JSON line")
    ap.add_argument("--offload", type=float, nargs="*", default=None, metavar="MB",
                    help="only measure host offload/prefetch copies of MB per step (default "
                         "0.52 4 18.9) beside the step and print their JSON line")
    ap.add_argument("--offload-concurrent-only", action="store_true",
                    help="with --offload: only the consecutive-block runs beside the steps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (reference for the HBM "
                         "byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the step has no multi-GPU path; each GPU "
              "would run its own share of the batch (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones((n,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)  # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "copies": 5}))
        return
    bd.load()  # fails loudly when libspa.so is missing
    w = synth.WORKLOADS[args.workload]
    if args.sparsity_sweep:
        sparsity_sweep(w, dev, args.steps, args.warmup)
        return
    if args.unified_vs_sequential:
        unified_vs_sequential(w, dev, args.steps, args.warmup)
        return
    if args.recall:
        recall_measure(w, dev, args.steps, args.warmup, args.recall[0], args.recall[1])
        return
    if args.quality:
        quality_measure(w, dev, args.steps, args.warmup, args.quality)
        return
    if args.per_call:
        per_call(w, dev, args.per_call)
        return
    if args.clock_ramp:
        clock_ramp(w, dev)
        return
    if args.offload is not None:
        offload_measure(w, dev, args.steps, args.warmup, tuple(args.offload) or (0.52, 4.0, 18.9),
                        concurrent_only=args.offload_concurrent_only)
        return
    if args.ceiling:
        ceiling_measure(w, dev)
        return
    if args.stride_quality:
        stride_quality_measure(w, dev, args.stride_quality, n_req=args.stride_requests)
        return
    if args.scheduler:
        modes = ("plain", "delayed") if args.scheduler == "both" else (args.scheduler,)
        scheduler_measure(w, dev, args.steps, args.warmup, modes)
        return
    print(f"[bench] generating {w.name} on {dev}", file=sys.stderr, flush=True)
    b = synth.make_batch(w, device=dev)
    bufs = bd.StepBuffers(b)
    alg = algorithmic_bytes(b)

    # Clock settling, the last part of the setup: after an idle period (here
    # the host-side part of the batch generation) the GPU's clocks take about
    # 10 ms of load to settle, and calls made meanwhile run up to 10% slower
    # (--clock-ramp); after ~40 ms of plain device copies they do not.  A
    # serving loop keeps the GPU loaded between attention steps, so the
    # measured steps start from loaded clocks.  The copies are unrelated to
    # the step and end before the warm-up steps start.
    settle = None
    if args.settle_copies > 0:
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.settle_copies):
            dst.copy_(src)
        e1.record()
        del src, dst  # freed in stream order, after the copies

    # warm-up, queued right behind the settling copies
    for _ in range(args.warmup):
        bufs.step()
    torch.cuda.synchronize()
    if args.settle_copies > 0:
        settle = {"copies_of_1GiB": args.settle_copies, "ms": round(e0.elapsed_time(e1), 1)}

    # timed region: K steps back to back with nothing but the two bracketing
    # events (the library's per-launch events would add their own gaps)
    t_ev0 = torch.cuda.Event(enable_timing=True)
    t_ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_ev0.record()
    for _ in range(args.steps):
        bufs.step()
    t_ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_ev0.elapsed_time(t_ev1)
    ms_step = ms_total / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step * 1e3:.1f} us/step "
          f"(host wall {wall * 1e6 / args.steps:.1f} us/step)", file=sys.stderr, flush=True)

    # the same K steps again, now with the attention launch bracketed by HIP
    # events recorded on the stream it is launched on (each call its own pair)
    attn_us = launch_times(bufs.step, ("attn",), args.steps)["attn"]

    # per-kernel breakdown (separate pass, every kernel bracketed)
    breakdown = {nm: round(v, 2) for nm, v in
                 launch_times(bufs.step, ("attn", "post", "select"), 10).items()}

    # cold steps: a 512 MB write between steps evicts the 256 MB Infinity Cache
    cold = None
    if args.cold_steps > 0:
        scratch = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
        times = []
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        for i in range(args.cold_steps):
            scratch.fill_(i & 0xFF)
            e0.record()
            bufs.step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        del scratch
        times = np.array(times)
        cold = {"us_median": round(float(np.median(times)), 1),
                "us_p10": round(float(np.percentile(times, 10)), 1),
                "us_p90": round(float(np.percentile(times, 90)), 1),
                "hbm_gbps_method": round(alg["bytes_method"] / (np.median(times) * 1e-6) / 1e9, 1)}

    steps_per_s = 1e3 / ms_step
    gbps_method = alg["bytes_method"] / (ms_step * 1e-3) / 1e9
    gbps_min = alg["bytes_min"] / (ms_step * 1e-3) / 1e9
    # the dominant work is all attention of the step, one launch
    attn_bytes = alg["attn_launch"]
    attn_gbps = attn_bytes / (attn_us * 1e-6) / 1e9
    traffic = recorded_traffic(w.name)
    mf = mfma_flops(b)
    mfma = None
    if w.dtype == "bf16":
        # MFMA work of the same launch against the dense bf16 peak: the
        # contraction is real, but at 36-65 FLOP per KV byte the launch sits
        # far below the ridge (about 310 FLOP/B), so this stays small
        mfma = {"kernel": "attn_kernel", "dtype": "bf16",
                "algorithmic_flops_per_launch": mf["total"], "verify_flops": mf["verify"],
                "achieved_tflops": round(mf["total"] / (attn_us * 1e-6) / 1e12, 2),
                "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                "frac": round(mf["total"] / (attn_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                "counters": recorded_mfma(w.name),
                "counters_source": f"profiles/attn_kernel_{w.name}_mfma.md (recorded)"}

    # the attainable bandwidth of the launch's own access mix on this device,
    # measured now (libspa_probe; the two best settings of the full sweep)
    ceiling = None
    if w.dtype == "bf16" and w.head_dim == 128 and not args.no_ceiling:
        print("[bench] measuring the access-mix ceiling", file=sys.stderr, flush=True)
        cres = mix_ceiling(w, dev, {"launch_mix": MIXES["launch_mix"]}, [(4, 4096), (2, 4096)],
                           settle=False)
        cbest = cres["mixes"]["launch_mix"]["best"]
        ceiling = {"mix": "launch_mix", "GB_s": cbest["GB_s"], "depth": cbest["depth"],
                   "workgroups": cbest["grid"], "tiles": cres["tiles"],
                   "bytes": cres["read_bytes"] + cres["write_bytes"]}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        cpu = cpu_baseline(b, args.cpu_repeats)

    nv = sum(b.is_verify)
    line = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": b.B, "n_verify": nv, "n_draft": b.B - nv,
                   "seq_lens": "fixed" if len(set(b.seq_lens)) == 1 else "drawn",
                   "mean_seq_len": round(float(np.mean(b.seq_lens)), 1),
                   "num_qo_heads": w.num_qo_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "spec_k": w.spec_k,
                   "sparsity": f"{w.sparsity.numerator}/{w.sparsity.denominator}",
                   "page_size": 1, "pool_slots": b.num_slots},
        "attended_kv_tokens_per_s": round(alg["attended_tokens"] * steps_per_s, 1),
        "hbm_gbps_method": round(gbps_method, 1),
        "hbm_frac_method": round(gbps_method / HBM_PEAK_GBPS, 4),
        "hbm_gbps_min": round(gbps_min, 1),
        "bytes_method_per_step": alg["bytes_method"],
        "bytes_min_per_step": alg["bytes_min"],
        "kernel_us": breakdown,
        "clock_settle": settle,
        "cold": cold,
        "roofline": {"bound": "hbm", "kernel": "attn_kernel",
                     "achieved": round(attn_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     # where traffic comes from: recorded counter runs of these
                     # kernel sources (profiles/), not this run
                     "traffic_source": f"profiles/attn_kernel_{w.name}_traffic.md (recorded, "
                                       f"source {kernel_source_hash()})" if traffic else None,
                     # the bytes the launch really moves (counted), per second
                     "traffic_gbps": round(traffic / (attn_us * 1e-6) / 1e9, 1) if traffic else None,
                     "algorithmic_bytes_per_launch": attn_bytes,
                     "launch_us": round(attn_us, 2), "launches": args.steps,
                     # the same achieved rate against what this device attains for
                     # the launch's access mix (scattered 256-byte KV rows plus
                     # the logits stores, no arithmetic), measured in this run
                     "mix_ceiling": ceiling,
                     "frac_of_mix_ceiling": round(attn_gbps / ceiling["GB_s"], 4) if ceiling else None},
        "mfma": mfma,
        "cpu_baseline": cpu,
        "env": {"device": torch.cuda.get_device_name(dev),
                "gcn_arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
                "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
                "hip_runtime": torch.version.hip, "torch": torch.__version__,
                "seed": w.seed, "libspa_abi": bd.abi_version()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
