"""The KV block manager and the host-side checks of the block copies of
include/spa_kvcache.h -- CPU only.

The manager's rules (review of SparseSpec, 核心方法 / "Dynamic KV-Cache
manager"): requests are admitted while device blocks last; offload victims
are the resident requests admitted last (the oldest keep their memory),
skipping the ones about to run; offloaded requests come back first in, first
out, each only while its blocks fit.  Invariants over random operation
sequences: no device block or host chunk is held twice, the free counts
match, and page-table rows follow the blocks."""
import ctypes as C
import os

import numpy as np
import pytest

from sparse_self_speculative_pillarattn_amd import binding as bd

FAKE = C.c_void_p(0x1000)


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from sparse_self_speculative_pillarattn_amd import build
        build.build()
    return bd.load()


def test_reserve_admits_in_block_order_and_reports_full():
    m = bd.KVManager(dev_blocks=10, host_chunks=6, block_slots=4, max_requests=5, max_blocks=8)
    assert m.reserve(0, 9)                      # 3 blocks: 0, 1, 2
    assert list(m.page_row(0, 9)) == list(range(9))
    assert m.reserve(0, 12) and m.stats()["free_dev_blocks"] == 7   # same 3 blocks
    assert m.reserve(0, 13)                     # a 4th block: 3
    assert list(m.page_row(0, 13)[12:]) == [12]
    assert not m.reserve(1, 4 * 7)              # 7 blocks > 6 free: nothing changes
    assert m.where(1) == 0 and m.stats()["free_dev_blocks"] == 6
    assert m.reserve(1, 24) and m.where(1) == 1
    with pytest.raises(bd.SpaError):
        m.reserve(2, 4 * 9)                     # beyond max_blocks
    with pytest.raises(bd.SpaError):
        m.page_row(0, 17)                       # beyond the request's blocks
    m.release(0)
    assert m.where(0) == 0 and m.stats()["free_dev_blocks"] == 4
    assert m.stats()["resident"] == 1


def test_offload_takes_the_newest_and_prefetch_returns_fifo():
    m = bd.KVManager(dev_blocks=12, host_chunks=12, block_slots=2, max_requests=6, max_blocks=6)
    for r, L in ((0, 4), (1, 4), (2, 4), (3, 4), (4, 4), (5, 4)):
        assert m.reserve(r, L)
    assert m.stats()["free_dev_blocks"] == 0
    blocks, chunks, reqs = m.plan_offload(need_free=5, keep=[4])
    assert list(reqs) == [5, 3, 2]              # newest first, request 4 kept
    assert len(blocks) == 6 and len(set(chunks.tolist())) == 6
    assert m.stats()["free_dev_blocks"] == 6 and m.stats()["offloaded"] == 3
    for r in reqs:
        assert m.where(r) == 2
        with pytest.raises(bd.SpaError):
            m.page_row(r, 4)
        with pytest.raises(bd.SpaError):
            m.reserve(r, 6)                     # offloaded requests do not grow
    # a new request takes 3 of the 6 free blocks; prefetch keeps 1 free
    assert m.reserve(4, 8)                      # request 4 grows by 2 blocks
    ch, bl, back = m.plan_prefetch(keep_free=1)
    assert list(back) == [5]                    # first offloaded first; 3 would leave 0 free
    ch2, bl2, back2 = m.plan_prefetch(keep_free=0)
    assert list(back2) == [3]
    assert sorted(np.concatenate([ch, ch2]).tolist()) == sorted(chunks[:4].tolist())
    assert not set(np.concatenate([bl, bl2]).tolist()) & set(
        (m.page_row(4, 8) // 2).tolist())       # they land in blocks nobody holds
    assert list(m.plan_prefetch()[2]) == []     # request 2 needs 2 blocks, 0 free
    m.release(0)
    assert list(m.plan_prefetch()[2]) == [2] and m.stats()["offloaded"] == 0


def test_offload_respects_cap_and_host_chunks():
    m = bd.KVManager(dev_blocks=8, host_chunks=3, block_slots=1, max_requests=4, max_blocks=8)
    assert m.reserve(0, 2) and m.reserve(1, 2) and m.reserve(2, 4)
    b, c, reqs = m.plan_offload(need_free=8)
    assert list(reqs) == []                     # request 2 needs 4 chunks, 3 free: stop
    b, c, reqs = m.plan_offload(need_free=8, keep=[2])
    assert list(reqs) == [1]                    # then request 0 needs 2 more, 1 left
    b, c, reqs = m.plan_offload(need_free=8, cap=1)
    assert list(reqs) == []


@pytest.mark.parametrize("seed", range(4))
def test_random_operations_keep_the_books(seed):
    rng = np.random.default_rng(seed)
    R, D, H, bs = 24, 40, 30, 3
    m = bd.KVManager(D, H, bs, R, 20)
    lens = {r: 0 for r in range(R)}
    for _ in range(600):
        op = rng.integers(0, 5)
        r = int(rng.integers(0, R))
        if op == 0 and m.where(r) != 2:
            L = lens[r] + int(rng.integers(1, 10))
            if L <= 20 * bs and m.reserve(r, L):
                lens[r] = L
        elif op == 1:
            m.release(r)
            lens[r] = 0
        elif op == 2:
            keep = rng.choice(R, size=3, replace=False)
            _, _, reqs = m.plan_offload(int(rng.integers(0, D + 1)), keep=keep)
            assert not set(reqs.tolist()) & set(keep.tolist())
        elif op == 3:
            m.plan_prefetch(int(rng.integers(0, 5)))
        # books: resident blocks distinct, counts consistent
        held = []
        st = m.stats()
        res = [q for q in range(R) if m.where(q) == 1]
        off = [q for q in range(R) if m.where(q) == 2]
        for q in res:
            if lens[q]:
                row = m.page_row(q, lens[q])
                assert np.array_equal(row % bs, np.arange(lens[q]) % bs)
                held += sorted(set((row // bs).tolist()))
        assert len(held) == len(set(held)) and all(0 <= b < D for b in held)
        assert st["resident"] == len(res) and st["offloaded"] == len(off)
        assert st["free_dev_blocks"] == D - len(held)
        held_chunks = sum(-(-lens[q] // bs) for q in off)
        assert st["free_host_chunks"] == H - held_chunks


def _lay():
    return bd.SpaLayout(num_qo_heads=8, num_kv_heads=2, head_dim=128, sm_scale=0.0, dtype=0,
                        num_slots=64, page_table_stride=64)


@pytest.mark.parametrize("blocks,chunks,arena,msg", [
    ([0, 8], [0, 1], 4 * 4096, b"outside"),       # 64 slots / 8 = 8 blocks
    ([0, 1], [0, 4], 4 * 4096, b"outside"),       # arena holds 4 chunks
    ([2, 2], [0, 1], 4 * 4096, b"twice"),
    ([1, 2], [3, 3], 4 * 4096, b"twice"),
    ([-1], [0], 4 * 4096, b"outside"),
])
def test_block_copies_reject_bad_moves(lib, blocks, chunks, arena, msg):
    b = np.asarray(blocks, np.int32)
    c = np.asarray(chunks, np.int32)
    lay = _lay()
    assert lib.spa_kv_block_bytes(C.byref(lay), 8) == 8 * 2 * 128 * 2
    rc = lib.spa_kv_offload(C.byref(lay), 8, len(b), b.ctypes.data_as(C.c_void_p),
                            c.ctypes.data_as(C.c_void_p), FAKE, FAKE, FAKE, FAKE, arena, None,
                            None, None)
    assert rc == bd.SPA_ERR_INVALID_ARG and msg in lib.spa_last_error()
    rc = lib.spa_kv_prefetch(C.byref(lay), 8, len(b), c.ctypes.data_as(C.c_void_p),
                             b.ctypes.data_as(C.c_void_p), FAKE, FAKE, arena, FAKE, FAKE, None,
                             None, None)
    assert rc == bd.SPA_ERR_INVALID_ARG and msg in lib.spa_last_error()


def test_block_copies_reject_pageable_arenas_and_bad_layouts(lib):
    lay = _lay()
    b = np.asarray([0], np.int32)
    host = np.zeros(8192, np.uint8)   # ordinary (pageable) memory
    rc = lib.spa_kv_offload(C.byref(lay), 8, 1, b.ctypes.data_as(C.c_void_p),
                            b.ctypes.data_as(C.c_void_p), FAKE, FAKE,
                            host.ctypes.data_as(C.c_void_p), host.ctypes.data_as(C.c_void_p),
                            8192, None, None, None)
    assert rc == bd.SPA_ERR_INVALID_ARG and b"pinned" in lib.spa_last_error()
    assert lib.spa_kv_block_bytes(C.byref(lay), 0) == 0
    bad = bd.SpaLayout(num_qo_heads=8, num_kv_heads=2, head_dim=96, sm_scale=0.0, dtype=0,
                       num_slots=64, page_table_stride=64)
    assert lib.spa_kv_offload(C.byref(bad), 8, 0, None, None, None, None, None, None, 0, None,
                              None, None) == bd.SPA_ERR_INVALID_ARG
    # nothing to move: a no-op
    assert lib.spa_kv_offload(C.byref(lay), 8, 0, None, None, None, None, None, None, 0, None,
                              None, None) == bd.SPA_OK


@pytest.mark.parametrize("cfg", [dict(dev_blocks=0), dict(block_slots=0), dict(max_requests=0),
                                 dict(max_blocks=0), dict(host_chunks=-1)])
def test_manager_rejects_bad_configs(cfg):
    kw = dict(dev_blocks=4, host_chunks=4, block_slots=4, max_requests=4, max_blocks=4)
    kw.update(cfg)
    with pytest.raises(bd.SpaError):
        bd.KVManager(**kw)
