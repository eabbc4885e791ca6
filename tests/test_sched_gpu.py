"""Several decode steps chained under the scheduler, against the oracle step by
step -- needs an MI355X.

Each step's inputs are what the earlier steps left on the device: the lists
that a verify selected are the ones its request's following drafts read
(list persistence across a speculation stride), new requests get their
initial lists, and the batch mixes phases as the buckets dictate.  Every step
is compared with the oracle on the same inputs (O, LSE, logits, top-K), and
the lists are followed across steps: a draft reads exactly the list its
request's last verify wrote.  Cases span at least two strides, with and
without delayed verification, and include retirements (short outputs)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import to_np
import parity
from sparse_self_speculative_pillarattn_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def batch_of(drv, st, a, idx_before, dtype):
    """The step as a synth.Batch: host metadata plus host copies of what it reads."""
    w = synth.Workload(name="sched", batch=st.B, num_qo_heads=drv.Hq, num_kv_heads=drv.Hkv,
                       head_dim=drv.d, dtype=dtype, spec_k=drv.k, sparsity=Fraction(1, 1),
                       lengths=("fixed", 1))
    slots = torch.from_numpy(a["slot"].astype(np.int64)).to(DEV)
    lo = a["logits_off"].tolist()
    return synth.Batch(
        w=w, B=st.B, seq_lens=a["seq_lens"].tolist(), is_verify=[bool(v) for v in a["is_verify"]],
        q_indptr=a["q_indptr"].tolist(), idx_count=a["idx_count"].tolist(),
        idx_off=a["idx_off"].tolist(),
        logits_off=[o if v else -1 for o, v in zip(lo, a["is_verify"])], pillar_pos=[],
        q=drv.q[:st.rows].cpu(), k_pool=drv.k_pool.cpu(), v_pool=drv.v_pool.cpu(),
        page_table=drv.page_table.index_select(0, slots).cpu(), idx=idx_before,
        num_slots=drv.num_slots, stride=drv.max_len, logits_elems=int(st.logits_elems),
        idx_elems=int(drv.idx.numel()))


CASES = [
    # slots, k, H_q, H_kv, d, dtype, delayed, prompt, output, steps
    (7, 3, 8, 2, 128, "bf16", False, (40, 200), (6, 14), 12),
    (7, 3, 8, 2, 128, "bf16", True, (40, 200), (6, 14), 15),
    (9, 4, 16, 8, 128, "bf16", True, (60, 400), (10, 30), 18),
    (5, 2, 4, 2, 64, "f32", False, (10, 120), (3, 8), 12),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{c[0]}k{c[1]}h{c[2]}kv{c[3]}{c[5]}"
                         + ("-delayed" if c[6] else ""))
def test_chained_steps_match_the_oracle(oracle, case):
    from sparse_self_speculative_pillarattn_amd.sched_driver import SchedDriver
    S, k, Hq, Hkv, d, dtype, delayed, prompt, output, steps = case
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    drv = SchedDriver(S, k, Hq, Hkv, d, Fraction(1, 10), prompt, output, delayed=delayed, seed=11,
                      device=DEV, dtype=tdt)
    written = {}  # slot -> (K, lists [H_kv][K]) its last verify selected
    C = k + 1 + int(delayed)
    verifies = drafts_checked = 0
    for t in range(steps):
        st, a = drv.plan(fresh_q=True)
        torch.cuda.synchronize()
        for s in a["new_slots"].tolist():
            written.pop(int(s), None)
        idx_before = drv.idx.cpu()
        b = batch_of(drv, st, a, idx_before, dtype)
        print(f"[step] {t} B={st.B} rows={st.rows} verify={st.n_verify} new={st.n_new} "
              f"lens={b.seq_lens}", flush=True)
        drv.o.fill_(float("nan"))
        drv.lse.fill_(float("nan"))
        drv.logits.fill_(float("nan"))
        drv.launch()
        torch.cuda.synchronize()
        ref = oracle.step(**parity.oracle_inputs(b))
        gpu = {"o": drv.o[:st.rows], "lse": drv.lse[:st.rows],
               "logits": drv.logits[:max(st.logits_elems, 1)], "idx": drv.idx}
        if st.logits_elems == 0:
            gpu["logits"] = drv.logits[:0]
        parity.compare_step(oracle, b, gpu, ref)
        idx_after = to_np(drv.idx)
        for r in range(st.B):
            s, off, K = int(a["slot"][r]), int(a["idx_off"][r]), int(a["idx_count"][r])
            seg = idx_after[off:off + Hkv * K].reshape(Hkv, K)
            if a["is_verify"][r]:
                written[s] = (K, seg.copy())
                verifies += 1
            elif s in written:
                Kw, lists = written[s]
                assert K == Kw and np.array_equal(seg, lists), f"step {t} slot {s}: stale list"
                drafts_checked += 1
        drv.commit()
    assert steps >= 2 * C and verifies >= S and drafts_checked > 0
    assert drv.sched.stats()["verifies"] == verifies
