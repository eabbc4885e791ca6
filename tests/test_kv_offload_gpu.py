"""A step whose KV partly came back from host memory -- needs an MI355X.

The batch's K and V rows move into block-structured pools (kv_offload.BlockKV);
a step runs and is checked against the oracle; then half of the requests are
offloaded to pinned host chunks on the copy stream, every free device block
is overwritten, the requests are prefetched back into other blocks, their
page-table rows are rewritten, and the step runs again.  The second step must
equal the first bit for bit (the kernels' work split does not depend on where
a position's slot lives) and match the oracle.  Meanwhile an unrelated
request is offloaded on the copy stream, so copies and attention overlap."""
from dataclasses import replace
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import to_np
import parity
from sparse_self_speculative_pillarattn_amd import binding as bd
from sparse_self_speculative_pillarattn_amd import synth
from sparse_self_speculative_pillarattn_amd.kv_offload import BlockKV

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_step(b):
    bufs = bd.StepBuffers(b)
    for t in (bufs.o, bufs.lse, bufs.logits):
        t.fill_(float("nan"))
    bufs.step()
    return {"o": bufs.o, "lse": bufs.lse, "logits": bufs.logits, "idx": bufs.idx}


@pytest.mark.parametrize("dtype,bs", [("bf16", 64), ("f32", 16)])
def test_step_after_offload_and_prefetch(oracle, dtype, bs):
    w = synth.Workload(name=f"kv-offload-{dtype}", batch=6, num_qo_heads=8, num_kv_heads=2,
                       head_dim=128, dtype=dtype, spec_k=4, sparsity=Fraction(1, 20),
                       lengths=("uniform", 100, 3000), seed=61)
    b = synth.make_batch(w, device=DEV)
    B, lens = b.B, b.seq_lens
    tdt = b.k_pool.dtype
    need = sum(-(-L // bs) for L in lens)
    spare_len = 5 * bs
    kv = BlockKV(w.num_qo_heads, w.num_kv_heads, w.head_dim, tdt, dev_blocks=2 * need + 8,
                 host_chunks=need + 8, block_slots=bs, max_requests=B + 1, max_len=b.stride)
    print(f"[kv-offload] {dtype} block_slots={bs} lens={lens} blocks={need}", flush=True)
    for r in range(B):
        rows = b.page_table[r, :lens[r]].long()
        assert kv.write(r, b.k_pool.index_select(0, rows), b.v_pool.index_select(0, rows))
    # a request outside the batch, moved while the second step runs
    g = torch.Generator(device=DEV).manual_seed(3)
    spare_k = torch.randn((spare_len, 2, 128), generator=g, device=DEV).to(tdt)
    spare_v = torch.randn((spare_len, 2, 128), generator=g, device=DEV).to(tdt)
    assert kv.write(B, spare_k, spare_v)
    all_lens = dict(enumerate(lens))
    all_lens[B] = spare_len
    pt_a = kv.page_rows(range(B), lens, b.stride)
    ba = replace(b, page_table=pt_a, k_pool=kv.k_pool, v_pool=kv.v_pool, num_slots=kv.slots)
    out_a = run_step(ba)
    torch.cuda.synchronize()
    ref = oracle.step(**parity.oracle_inputs(b))
    parity.compare_step(oracle, b, out_a, ref)
    out_a = {k: v.clone() for k, v in out_a.items()}

    # offload the odd requests (the batch's newest first), keeping the even ones
    odd = [r for r in range(B) if r % 2]
    keep = [r for r in range(B) if r % 2 == 0] + [B]
    reqs, done, moved = kv.offload(need_free=kv.slots // bs, keep=keep)
    assert sorted(reqs.tolist()) == odd and list(reqs) == sorted(odd, reverse=True)
    assert moved == sum(-(-lens[r] // bs) for r in odd)
    # once they are on the host, overwrite every block nobody holds
    cur = torch.cuda.current_stream()
    cur.wait_event(done)
    free = kv.free_blocks(all_lens)
    slots = torch.from_numpy((free[:, None] * bs + np.arange(bs)).reshape(-1)).to(DEV)
    junk = torch.full((slots.numel(), 2, 128), 1e4, dtype=tdt, device=DEV)
    kv.k_pool.index_copy_(0, slots, junk)
    kv.v_pool.index_copy_(0, slots, -junk)
    rows_before = {r: kv.kvm.where(r) for r in odd}
    assert all(v == 2 for v in rows_before.values())
    back, done2, moved2 = kv.prefetch()          # waits for the overwrite
    assert list(back) == list(reqs) and moved2 == moved
    cur.wait_event(done2)
    pt_b = kv.page_rows(range(B), lens, b.stride)
    changed = [r for r in odd if not torch.equal(pt_a[r, :lens[r]], pt_b[r, :lens[r]])]
    assert changed == odd                        # they came back into other blocks
    for r in keep[:-1]:
        assert torch.equal(pt_a[r], pt_b[r])
    # the unrelated request leaves while the step runs
    ev = torch.cuda.Event()
    ev.record()
    spare, done3, _ = kv.offload(need_free=kv.slots // bs, keep=list(range(B)), after=ev)
    assert list(spare) == [B]
    out_b = run_step(replace(ba, page_table=pt_b))
    torch.cuda.synchronize()
    done3.synchronize()
    for name in ("o", "lse", "logits", "idx"):
        assert torch.equal(out_a[name].view(torch.uint8), out_b[name].view(torch.uint8)), name
    parity.compare_step(oracle, b, out_b, ref)
    st = kv.kvm.stats()
    assert st["offloads"] == len(odd) + 1 and st["prefetches"] == len(odd)
    # the unrelated request's rows arrived in its host chunks intact
    _, chunks = kv.last_moves
    ka = kv.k_arena.view(tdt).view(-1, bs, 2, 128)
    va = kv.v_arena.view(tdt).view(-1, bs, 2, 128)
    idx = torch.from_numpy(chunks.astype(np.int64))
    assert torch.equal(ka[idx].reshape(-1, 2, 128)[:spare_len], spare_k.cpu())
    assert torch.equal(va[idx].reshape(-1, 2, 128)[:spare_len], spare_v.cpu())
