"""ctypes front of the fp64 C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline leg of the benchmark, never by the HIP library or its binding.

Arrays are numpy; bf16 data is passed as its raw uint16 bits (dtype code 0),
fp32 as float32 (dtype code 1).  Outputs are float64.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_LIBS: dict = {}

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def _load(mutant: int = 0):
    if mutant in _LIBS:
        return _LIBS[mutant]
    path = _build.lib_path(mutant)
    if mutant or not os.path.exists(path) or (
            os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
        _build.build(mutant)
    lib = C.CDLL(path)
    vp = C.c_void_p
    lib.oracle_verify_request.argtypes = [C.c_int, C.c_int, C.c_int, C.c_double, C.c_int, C.c_int,
                                          C.c_int, vp, vp, vp, _i32p, _f64p, _f64p, _f64p]
    lib.oracle_verify_request.restype = None
    lib.oracle_average.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                   _f64p, _f64p, _f64p]
    lib.oracle_average.restype = None
    lib.oracle_topk.argtypes = [C.c_int, C.c_int, _f64p, _i32p]
    lib.oracle_topk.restype = C.c_int
    lib.oracle_draft_request.argtypes = [C.c_int, C.c_int, C.c_int, C.c_double, C.c_int, C.c_int,
                                         vp, vp, vp, _i32p, C.c_int, _i32p, _f64p, _f64p]
    lib.oracle_draft_request.restype = None
    lib.oracle_step.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_double, C.c_int,
                                C.c_int, C.c_int, _u8p, _i32p, _i32p, _i32p, C.c_int64,
                                vp, vp, vp, _i32p, _i64p, _i32p, _f64p, _f64p, _f64p, _i64p,
                                vp, C.c_int]
    lib.oracle_step.restype = C.c_int
    lib.oracle_recall_index.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, _i32p, C.c_int,
                                        _i32p]
    lib.oracle_recall_index.restype = C.c_int
    lib.oracle_list_quality.argtypes = [C.c_int, C.c_int, C.c_int, _f64p, _f64p, C.c_int, _i32p,
                                        C.c_int, _i32p, _f64p, _f64p]
    lib.oracle_list_quality.restype = C.c_int
    lib.oracle_mutant_id.restype = C.c_int
    _LIBS[mutant] = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 0
    if a.dtype == np.float32:
        return 1
    raise TypeError(f"oracle inputs are bf16 bits (uint16) or float32, got {a.dtype}")


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


class Oracle:
    """One loaded oracle library (``mutant`` > 0 loads a deliberately broken build)."""

    def __init__(self, mutant: int = 0):
        self.mutant = mutant
        self.lib = _load(mutant)

    # -- single-request pieces ------------------------------------------------
    def verify_request(self, q, k_pool, v_pool, pt_row, L, k, Hq, Hkv, sm_scale):
        """q [(k+1)][Hq][d]; returns logits [(k+1)][Hq][L], lse [(k+1)][Hq], o [(k+1)][Hq][d]."""
        dt = _dtype_code(q)
        assert _dtype_code(k_pool) == dt and _dtype_code(v_pool) == dt
        d = q.shape[-1]
        q = np.ascontiguousarray(q)
        logits = np.empty(((k + 1), Hq, L), np.float64)
        lse = np.empty(((k + 1), Hq), np.float64)
        o = np.empty(((k + 1), Hq, d), np.float64)
        self.lib.oracle_verify_request(Hq, Hkv, d, float(sm_scale), dt, int(L), int(k), _ptr(q),
                                       _ptr(k_pool), _ptr(v_pool),
                                       np.ascontiguousarray(pt_row, np.int32), logits, lse, o)
        return logits, lse, o

    def average(self, logits, lse, Hkv, row_begin, row_count):
        """logits [(k+1)][Hq][L] (any float), lse [(k+1)][Hq] -> pbar [Hkv][L]."""
        logits = np.ascontiguousarray(logits, np.float64)
        lse = np.ascontiguousarray(lse, np.float64)
        rows, Hq, L = logits.shape
        pbar = np.empty((Hkv, L), np.float64)
        self.lib.oracle_average(Hq, Hkv, L, rows - 1, int(row_begin), int(row_count), logits, lse,
                                pbar)
        return pbar

    def topk(self, score, K):
        score = np.ascontiguousarray(score, np.float64)
        out = np.empty((K,), np.int32)
        rc = self.lib.oracle_topk(score.shape[0], int(K), score, out)
        if rc:
            raise ValueError(f"oracle_topk failed ({rc})")
        return out

    def draft_request(self, q, k_pool, v_pool, pt_row, L, idx, Hkv, sm_scale):
        """q [Hq][d]; idx [Hkv][n]; returns o [Hq][d], lse [Hq]."""
        dt = _dtype_code(q)
        Hq, d = q.shape
        idx = np.ascontiguousarray(idx, np.int32).reshape(Hkv, -1)
        q = np.ascontiguousarray(q)
        o = np.empty((Hq, d), np.float64)
        lse = np.empty((Hq,), np.float64)
        self.lib.oracle_draft_request(Hq, Hkv, d, float(sm_scale), dt, int(L), _ptr(q),
                                      _ptr(k_pool), _ptr(v_pool),
                                      np.ascontiguousarray(pt_row, np.int32), idx.shape[1], idx,
                                      o, lse)
        return o, lse

    def recall_index(self, L, n_sink, n_recent, stored, cap):
        """stored [n] positions of one KV head -> (out [cap], u): the ascending
        union of sinks, valid stored positions and recent positions, then -1."""
        stored = np.ascontiguousarray(stored, np.int32).reshape(-1)
        out = np.empty((max(int(cap), 1),), np.int32)
        u = self.lib.oracle_recall_index(int(L), int(n_sink), int(n_recent), stored.shape[0],
                                         stored, int(cap), out)
        if u < 0:
            raise ValueError(f"oracle_recall_index failed ({u})")
        return out[:int(cap)], u

    def list_quality(self, logits, lse, lists, T):
        """logits [Hq][L] and lse [Hq] of one query row; lists [Hkv][n].
        Returns (top [Hq][T] ascending, coverage [Hq], recall [Hq])."""
        logits = np.ascontiguousarray(logits, np.float64)
        lse = np.ascontiguousarray(lse, np.float64).reshape(-1)
        Hq, L = logits.shape
        lists = np.ascontiguousarray(lists, np.int32)
        Hkv = lists.shape[0]
        n = lists.shape[1] if lists.ndim == 2 else 0
        lists = lists.reshape(-1) if lists.size else np.zeros((1,), np.int32)
        top = np.empty((Hq, int(T)), np.int32)
        cov = np.empty((Hq,), np.float64)
        rec = np.empty((Hq,), np.float64)
        rc = self.lib.oracle_list_quality(Hq, Hkv, L, logits, lse, n, lists, int(T), top.reshape(-1),
                                          cov, rec)
        if rc:
            raise ValueError(f"oracle_list_quality failed ({rc})")
        return top, cov, rec

    # -- whole batch --------------------------------------------------------------
    def step(self, *, k, Hq, Hkv, sm_scale, is_verify, seq_lens, q_indptr, page_table, q,
             k_pool, v_pool, idx_count, idx_off, idx, logits_off, logits_elems,
             row_begin=1, row_count=None, selected=None, nthreads=None):
        """Run the unified step; returns dict(o, lse, logits, idx)."""
        dt = _dtype_code(q)
        assert _dtype_code(k_pool) == dt and _dtype_code(v_pool) == dt
        B = len(seq_lens)
        d = q.shape[-1]
        rows = int(q_indptr[-1])
        row_count = k if row_count is None else row_count
        if nthreads is None:
            nthreads = len(os.sched_getaffinity(0))
        o = np.zeros((rows, Hq, d), np.float64)
        lse = np.zeros((rows, Hq), np.float64)
        logits = np.zeros((max(int(logits_elems), 1),), np.float64)
        idx_io = np.ascontiguousarray(idx, np.int32).copy()
        sel = None
        if selected is not None:
            sel = np.ascontiguousarray(selected, np.uint8)
        pt = np.ascontiguousarray(page_table, np.int32)
        rc = self.lib.oracle_step(
            B, int(k), Hq, Hkv, d, float(sm_scale), dt, int(row_begin), int(row_count),
            np.ascontiguousarray(is_verify, np.uint8), np.ascontiguousarray(seq_lens, np.int32),
            np.ascontiguousarray(q_indptr, np.int32), pt, pt.shape[1] if pt.ndim == 2 else 0,
            _ptr(np.ascontiguousarray(q)), _ptr(k_pool), _ptr(v_pool),
            np.ascontiguousarray(idx_count, np.int32), np.ascontiguousarray(idx_off, np.int64),
            idx_io, o, lse, logits,
            np.ascontiguousarray([max(x, 0) for x in logits_off], np.int64),
            _ptr(sel) if sel is not None else None, int(nthreads))
        if rc:
            raise RuntimeError(f"oracle_step failed ({rc})")
        return {"o": o, "lse": lse, "logits": logits, "idx": idx_io, "nthreads": nthreads}
