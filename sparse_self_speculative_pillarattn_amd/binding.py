"""ctypes binding of libspa (include/spa.h): argument marshalling only.

Device buffers are PyTorch tensors on the current HIP device; host metadata are
Python sequences or numpy arrays; plan buffers are pinned host tensors
(``plan_buffer``).  Every call enqueues on the current PyTorch stream of the
tensors' device and returns without synchronising.  The library must be built
(``python -m sparse_self_speculative_pillarattn_amd.build``); there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import threading
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspa.so")

SPA_OK = 0
SPA_ERR_INVALID_ARG = 1
SPA_ERR_UNSUPPORTED = 2
SPA_ERR_WORKSPACE_TOO_SMALL = 3
SPA_ERR_HIP = 4
SPA_ERR_PLAN_TOO_SMALL = 5
SPA_ERR_KV_FULL = 6
SPA_BF16 = 0
SPA_F32 = 1
ABI_VERSION = 2

STATIC_WORKSPACE_BYTES = 32 << 20  # SPA_STATIC_WORKSPACE_BYTES

EXPORTED = ("spa_abi_version", "spa_last_error", "spa_workspace_bytes", "spa_plan_bytes",
            "spa_verify_attn", "spa_pillar_topk", "spa_draft_attn", "spa_unified_step",
            "spa_unified_step_static",
            "spa_recall_index", "spa_recall_plan_bytes", "spa_list_quality",
            "spa_list_quality_workspace_bytes", "spa_list_quality_plan_bytes")
# include/spa_sched.h
SCHED_EXPORTED = ("spa_sched_bytes", "spa_sched_capacity", "spa_sched_init", "spa_sched_next",
                  "spa_sched_commit", "spa_sched_stats_read", "spa_sched_buckets")
KV_EXPORTED = ("spa_kv_block_bytes", "spa_kv_offload", "spa_kv_prefetch", "spa_kvm_bytes",
               "spa_kvm_init", "spa_kvm_reserve", "spa_kvm_release", "spa_kvm_plan_offload",
               "spa_kvm_plan_prefetch", "spa_kvm_page_row", "spa_kvm_where", "spa_kvm_stats_read")
# per-token acceptance probability whose leading-run mean over k = 8 drafts is
# 6.16 accepted tokens (the review's PillarAttn acceptance, 实验与结果)
ACCEPT_PROB_6_16_OF_8 = 0.9415853644089122

# indices into SpaOptions.timing: begin/end event pairs of each launch
TIMING = {"attn": (0, 1), "post": (2, 3), "select": (4, 5), "attn_draft": (6, 7)}


class SpaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libspa status {status}: {msg}")
        self.status = status


class SpaLayout(C.Structure):
    _fields_ = [("num_qo_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("sm_scale", C.c_float), ("dtype", C.c_int32),
                ("num_slots", C.c_int64), ("page_table_stride", C.c_int32)]


class SpaOptions(C.Structure):
    _fields_ = [("verify_chunk", C.c_int32), ("draft_chunk", C.c_int32), ("num_cus", C.c_int32),
                ("overlap", C.c_int32), ("side_stream", C.c_void_p), ("fork_event", C.c_void_p),
                ("join_event", C.c_void_p), ("timing", C.c_void_p * 8),
                ("page_table_rows", C.c_void_p), ("page_table_row_count", C.c_int32)]


class SpaSchedConfig(C.Structure):
    _fields_ = [("slots", C.c_int32), ("spec_k", C.c_int32), ("delayed", C.c_int32),
                ("num_qo_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("sparsity_num", C.c_int32), ("sparsity_den", C.c_int32),
                ("prompt_min", C.c_int32), ("prompt_max", C.c_int32),
                ("output_min", C.c_int32), ("output_max", C.c_int32), ("max_len", C.c_int32),
                ("accept_prob", C.c_float), ("seed", C.c_uint64)]


class SpaSchedStep(C.Structure):
    _fields_ = [("step", C.c_int64), ("B", C.c_int32), ("rows", C.c_int32),
                ("n_verify", C.c_int32), ("n_draft", C.c_int32), ("n_waiting", C.c_int32),
                ("n_new", C.c_int32), ("is_verify", C.c_void_p), ("seq_lens", C.c_void_p),
                ("q_indptr", C.c_void_p), ("idx_count", C.c_void_p), ("idx_off", C.c_void_p),
                ("logits_off", C.c_void_p), ("slot", C.c_void_p), ("new_slots", C.c_void_p),
                ("new_len", C.c_void_p), ("new_count", C.c_void_p), ("logits_elems", C.c_int64)]


class SpaSchedStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("steps", "verifies", "drafts", "waits", "drafted",
                                         "accepted", "committed", "retired", "rows")]


class SpaKvmConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("dev_blocks", "host_chunks", "block_slots",
                                         "max_requests", "max_blocks")]


class SpaKvmStats(C.Structure):
    _fields_ = ([(n, C.c_int32) for n in ("resident", "offloaded", "free_dev_blocks",
                                          "free_host_chunks")] +
                [(n, C.c_int64) for n in ("offloads", "prefetches", "blocks_offloaded",
                                          "blocks_prefetched")])


_lib = None


def load(path: str = LIB_PATH):
    """Load libspa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m sparse_self_speculative_pillarattn_amd.build`")
    lib = C.CDLL(path)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    L = C.POINTER(SpaLayout)
    O = C.POINTER(SpaOptions)
    lib.spa_abi_version.restype = i32
    lib.spa_last_error.restype = C.c_char_p
    for name in ("spa_workspace_bytes", "spa_plan_bytes"):
        f = getattr(lib, name)
        f.argtypes = [L, i32, i32, vp, vp, vp, O]
        f.restype = sz
    lib.spa_verify_attn.argtypes = [L, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                    sz, O, vp]
    lib.spa_verify_attn.restype = i32
    lib.spa_pillar_topk.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                    sz, vp, sz, O, vp]
    lib.spa_pillar_topk.restype = i32
    lib.spa_draft_attn.argtypes = [L, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz,
                                   O, vp]
    lib.spa_draft_attn.restype = i32
    lib.spa_unified_step.argtypes = [L, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, i32, i32, vp, sz, vp, sz, O, vp]
    lib.spa_unified_step.restype = i32
    lib.spa_unified_step_static.argtypes = [L, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp, vp, vp, vp, i32, i32, vp, sz, O, vp]
    lib.spa_unified_step_static.restype = i32
    lib.spa_recall_index.argtypes = [i32, i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spa_recall_index.restype = i32
    lib.spa_recall_plan_bytes.argtypes = [i32]
    lib.spa_recall_plan_bytes.restype = sz
    lib.spa_list_quality.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp, sz, vp, sz, vp]
    lib.spa_list_quality.restype = i32
    lib.spa_list_quality_workspace_bytes.argtypes = [i32, i32, vp]
    lib.spa_list_quality_workspace_bytes.restype = sz
    lib.spa_list_quality_plan_bytes.argtypes = [i32]
    lib.spa_list_quality_plan_bytes.restype = sz
    SC = C.POINTER(SpaSchedConfig)
    lib.spa_sched_bytes.argtypes = [SC]
    lib.spa_sched_bytes.restype = sz
    lib.spa_sched_capacity.argtypes = [SC, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                       C.POINTER(C.c_int32)]
    lib.spa_sched_capacity.restype = i32
    lib.spa_sched_init.argtypes = [vp, sz, SC]
    lib.spa_sched_init.restype = i32
    lib.spa_sched_next.argtypes = [vp, C.POINTER(SpaSchedStep)]
    lib.spa_sched_next.restype = i32
    lib.spa_sched_commit.argtypes = [vp]
    lib.spa_sched_commit.restype = i32
    lib.spa_sched_stats_read.argtypes = [vp, C.POINTER(SpaSchedStats)]
    lib.spa_sched_stats_read.restype = i32
    lib.spa_sched_buckets.argtypes = [vp, C.POINTER(C.c_int32), i32]
    lib.spa_sched_buckets.restype = i32
    KC = C.POINTER(SpaKvmConfig)
    pi = C.POINTER(C.c_int32)
    lib.spa_kv_block_bytes.argtypes = [L, i32]
    lib.spa_kv_block_bytes.restype = sz
    lib.spa_kv_offload.argtypes = [L, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.spa_kv_offload.restype = i32
    lib.spa_kv_prefetch.argtypes = [L, i32, i32, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp]
    lib.spa_kv_prefetch.restype = i32
    lib.spa_kvm_bytes.argtypes = [KC]
    lib.spa_kvm_bytes.restype = sz
    lib.spa_kvm_init.argtypes = [vp, sz, KC]
    lib.spa_kvm_init.restype = i32
    lib.spa_kvm_reserve.argtypes = [vp, i32, i32]
    lib.spa_kvm_reserve.restype = i32
    lib.spa_kvm_release.argtypes = [vp, i32]
    lib.spa_kvm_release.restype = i32
    lib.spa_kvm_plan_offload.argtypes = [vp, i32, vp, i32, i32, vp, vp, pi, vp, pi]
    lib.spa_kvm_plan_offload.restype = i32
    lib.spa_kvm_plan_prefetch.argtypes = [vp, i32, i32, vp, vp, pi, vp, pi]
    lib.spa_kvm_plan_prefetch.restype = i32
    lib.spa_kvm_page_row.argtypes = [vp, i32, i32, vp]
    lib.spa_kvm_page_row.restype = i32
    lib.spa_kvm_where.argtypes = [vp, i32]
    lib.spa_kvm_where.restype = i32
    lib.spa_kvm_stats_read.argtypes = [vp, C.POINTER(SpaKvmStats)]
    lib.spa_kvm_stats_read.restype = i32
    _lib = lib
    return lib


def _check(rc: int):
    if rc != SPA_OK:
        raise SpaError(rc, load().spa_last_error().decode())


class _Host:
    """Keeps host arrays alive for the duration of one call."""

    def __init__(self):
        self.keep = []

    def arr(self, seq, dtype):
        if seq is None:
            return None
        if isinstance(seq, np.ndarray) and seq.dtype == dtype and seq.flags.c_contiguous:
            a = seq
        else:
            a = np.ascontiguousarray(np.asarray(seq, dtype=dtype))
        self.keep.append(a)
        return C.c_void_p(a.ctypes.data)


def _dptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device buffers must be GPU tensors")
    if not t.is_contiguous():
        raise ValueError("device buffers must be contiguous")
    return C.c_void_p(t.data_ptr())


def _hptr(t: torch.Tensor):
    """Address of a pinned host buffer (plan buffer, KV arena)."""
    if t.is_cuda or not t.is_pinned():
        raise ValueError("plan buffers and KV arenas must be pinned host tensors")
    return C.c_void_p(t.data_ptr())


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _opts(o: Optional["Options"]):
    return None if o is None else C.byref(o.c)


def layout(num_qo_heads: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
           num_slots: int, page_table_stride: int, sm_scale: float = 0.0) -> SpaLayout:
    code = {torch.bfloat16: SPA_BF16, torch.float32: SPA_F32}.get(dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {dtype}")
    return SpaLayout(num_qo_heads, num_kv_heads, head_dim, float(sm_scale), code, int(num_slots),
                     int(page_table_stride))


class Options:
    """spa_options for one or more calls.  Streams and events are PyTorch
    objects; they are kept alive here for as long as the options are."""

    def __init__(self, verify_chunk: int = 0, draft_chunk: int = 0, num_cus: int = 0,
                 overlap: bool = False, side_stream: Optional[torch.cuda.Stream] = None,
                 timing: Optional[dict] = None, page_table_rows=None,
                 page_table_row_count: int = 0):
        self.c = SpaOptions()
        if page_table_rows is not None:
            self.rows = np.ascontiguousarray(page_table_rows, dtype=np.int32)
            self.c.page_table_rows = self.rows.ctypes.data
            self.c.page_table_row_count = int(page_table_row_count)
        self.c.verify_chunk = int(verify_chunk)
        self.c.draft_chunk = int(draft_chunk)
        self.c.num_cus = int(num_cus)
        self.c.overlap = 1 if overlap else 0
        self.keep = []
        if overlap:
            side = side_stream if side_stream is not None else torch.cuda.Stream()
            fork, join = _event(False), _event(False)
            self.keep += [side, fork, join]
            self.c.side_stream = side.cuda_stream
            self.c.fork_event = fork._as_parameter_.value
            self.c.join_event = join._as_parameter_.value
        self.timing = {}
        for name in (timing or {}):
            a, b = TIMING[name]
            ea, eb = _event(True), _event(True)
            self.timing[name] = (ea, eb)
            self.c.timing[a] = ea._as_parameter_.value
            self.c.timing[b] = eb._as_parameter_.value

    def elapsed_ms(self, name: str) -> float:
        """Milliseconds between the last recorded begin and end of a timed launch."""
        ea, eb = self.timing[name]
        eb.synchronize()
        return ea.elapsed_time(eb)


def _event(timing: bool) -> torch.cuda.Event:
    """A created (recorded once) PyTorch event, so that its handle exists."""
    ev = torch.cuda.Event(enable_timing=timing)
    ev.record()
    return ev


def default_options(device=None) -> Options:
    """Options with the device's compute-unit count for the automatic verify chunk."""
    props = torch.cuda.get_device_properties(device if device is not None else
                                             torch.cuda.current_device())
    return Options(num_cus=props.multi_processor_count)


def abi_version() -> int:
    return load().spa_abi_version()


def workspace_bytes(lay: SpaLayout, B: int, spec_k: int, is_verify: Optional[Sequence],
                    seq_lens: Sequence, idx_count: Optional[Sequence],
                    opts: Optional[Options] = None) -> int:
    h = _Host()
    n = load().spa_workspace_bytes(C.byref(lay), int(B), int(spec_k), h.arr(is_verify, np.uint8),
                                   h.arr(seq_lens, np.int32), h.arr(idx_count, np.int32),
                                   _opts(opts))
    if n == 0 and B > 0:
        raise SpaError(SPA_ERR_INVALID_ARG, load().spa_last_error().decode())
    return int(n)


def plan_bytes(lay: SpaLayout, B: int, spec_k: int, is_verify: Optional[Sequence],
               seq_lens: Sequence, idx_count: Optional[Sequence],
               opts: Optional[Options] = None) -> int:
    h = _Host()
    n = load().spa_plan_bytes(C.byref(lay), int(B), int(spec_k), h.arr(is_verify, np.uint8),
                              h.arr(seq_lens, np.int32), h.arr(idx_count, np.int32), _opts(opts))
    if n == 0 and B > 0:
        raise SpaError(SPA_ERR_INVALID_ARG, load().spa_last_error().decode())
    return int(n)


def workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of at least ``nbytes``, zero-filled (its first 256 bytes are
    work counters that must start at zero; calls leave them zero)."""
    return torch.zeros((max(int(nbytes), 256),), dtype=torch.uint8, device=device)


def plan_buffer(nbytes: int) -> torch.Tensor:
    """A pinned host plan buffer of at least ``nbytes``, 64-byte aligned."""
    raw = torch.empty((max(int(nbytes), 256) + 64,), dtype=torch.uint8, pin_memory=True)
    skip = (-raw.data_ptr()) % 64
    return raw[skip:skip + max(int(nbytes), 256)]


_tls = threading.local()


def _plan_for(nbytes: int) -> torch.Tensor:
    """A plan buffer of at least ``nbytes`` from this thread's own ring, for
    calls made without one.  A ring that is too small is replaced after the
    device has drained (the GPU may still read the old buffers until then)."""
    ring = getattr(_tls, "ring", None)
    if ring is None or ring.nbytes < nbytes:
        if ring is not None:
            torch.cuda.synchronize()
        ring = PlanRing(max(int(nbytes), 1 << 16))
        _tls.ring = ring
    return ring.next()


def verify_attn(lay, B, spec_k, seq_lens, page_table, q, k_pool, v_pool, o, lse, logits,
                logits_off, ws: torch.Tensor, plan: Optional[torch.Tensor] = None,
                opts: Optional[Options] = None):
    """plan: a pinned plan buffer (plan_buffer), or None for this thread's ring."""
    if plan is None:
        plan = _plan_for(plan_bytes(lay, B, spec_k, [1] * int(B), seq_lens, [1] * int(B), opts))
    h = _Host()
    _check(load().spa_verify_attn(
        C.byref(lay), int(B), int(spec_k), h.arr(seq_lens, np.int32), _dptr(page_table), _dptr(q),
        _dptr(k_pool), _dptr(v_pool), _dptr(o), _dptr(lse), _dptr(logits),
        h.arr(logits_off, np.int64), _dptr(ws), _nbytes(ws), _hptr(plan), _nbytes(plan),
        _opts(opts), _stream(q)))


def pillar_topk(B, spec_k, num_qo_heads, num_kv_heads, avg_row_begin, avg_row_count, seq_lens,
                topk, logits, logits_off, lse, idx, idx_off, ws: torch.Tensor,
                plan: Optional[torch.Tensor] = None, opts: Optional[Options] = None):
    if plan is None:
        lay = layout(num_qo_heads, num_kv_heads, 128, torch.bfloat16, 1, max(seq_lens))
        plan = _plan_for(plan_bytes(lay, B, spec_k, [1] * int(B), seq_lens, topk, opts))
    h = _Host()
    _check(load().spa_pillar_topk(
        int(B), int(spec_k), int(num_qo_heads), int(num_kv_heads), int(avg_row_begin),
        int(avg_row_count), h.arr(seq_lens, np.int32), h.arr(topk, np.int32), _dptr(logits),
        h.arr(logits_off, np.int64), _dptr(lse), _dptr(idx), h.arr(idx_off, np.int64), _dptr(ws),
        _nbytes(ws), _hptr(plan), _nbytes(plan), _opts(opts), _stream(logits)))


def draft_attn(lay, B, seq_lens, page_table, idx_count, idx_off, idx, q, k_pool, v_pool, o, lse,
               ws: torch.Tensor, plan: Optional[torch.Tensor] = None,
               opts: Optional[Options] = None):
    if plan is None:
        plan = _plan_for(plan_bytes(lay, B, 1, None, seq_lens, idx_count, opts))
    h = _Host()
    _check(load().spa_draft_attn(
        C.byref(lay), int(B), h.arr(seq_lens, np.int32), _dptr(page_table),
        h.arr(idx_count, np.int32), h.arr(idx_off, np.int64), _dptr(idx), _dptr(q),
        _dptr(k_pool), _dptr(v_pool), _dptr(o), _dptr(lse), _dptr(ws), _nbytes(ws), _hptr(plan),
        _nbytes(plan), _opts(opts), _stream(q)))


def unified_step(lay, B, spec_k, is_verify, seq_lens, q_indptr, page_table, q, k_pool, v_pool,
                 idx_count, idx_off, idx, o, lse, logits, logits_off, ws: torch.Tensor,
                 plan: Optional[torch.Tensor] = None, avg_row_begin: int = 1,
                 avg_row_count: Optional[int] = None, opts: Optional[Options] = None):
    if plan is None:
        plan = _plan_for(plan_bytes(lay, B, spec_k, is_verify, seq_lens, idx_count, opts))
    h = _Host()
    avg_row_count = spec_k if avg_row_count is None else avg_row_count
    _check(load().spa_unified_step(
        C.byref(lay), int(B), int(spec_k), h.arr(is_verify, np.uint8), h.arr(seq_lens, np.int32),
        h.arr(q_indptr, np.int32), _dptr(page_table), _dptr(q), _dptr(k_pool), _dptr(v_pool),
        h.arr(idx_count, np.int32), h.arr(idx_off, np.int64), _dptr(idx), _dptr(o), _dptr(lse),
        _dptr(logits), h.arr(logits_off, np.int64), int(avg_row_begin), int(avg_row_count),
        _dptr(ws), _nbytes(ws), _hptr(plan), _nbytes(plan), _opts(opts), _stream(q)))


def unified_step_static(lay, B, spec_k, is_verify, seq_lens, q_indptr, page_table, q, k_pool,
                        v_pool, idx_count, idx_off, idx, o, lse, logits, logits_off,
                        plan: Optional[torch.Tensor] = None, avg_row_begin: int = 1,
                        avg_row_count: Optional[int] = None, opts: Optional[Options] = None):
    """spa_unified_step_static: the unified step with the library's static
    device workspace (no workspace argument; nothing is allocated)."""
    if plan is None:
        plan = _plan_for(plan_bytes(lay, B, spec_k, is_verify, seq_lens, idx_count, opts))
    h = _Host()
    avg_row_count = spec_k if avg_row_count is None else avg_row_count
    _check(load().spa_unified_step_static(
        C.byref(lay), int(B), int(spec_k), h.arr(is_verify, np.uint8), h.arr(seq_lens, np.int32),
        h.arr(q_indptr, np.int32), _dptr(page_table), _dptr(q), _dptr(k_pool), _dptr(v_pool),
        h.arr(idx_count, np.int32), h.arr(idx_off, np.int64), _dptr(idx), _dptr(o), _dptr(lse),
        _dptr(logits), h.arr(logits_off, np.int64), int(avg_row_begin), int(avg_row_count),
        _hptr(plan), _nbytes(plan), _opts(opts), _stream(q)))


def recall_length(L: int, stored: int, n_sink: int, n_recent: int) -> int:
    """Smallest output length spa_recall_index accepts for one request."""
    s = min(n_sink, L)
    rec = L - max(s, L - min(n_recent, L))
    return max(1, min(L, s + rec + stored))


def recall_plan_bytes(B: int) -> int:
    return int(load().spa_recall_plan_bytes(int(B)))


def recall_index(B, num_kv_heads, seq_lens, n_sink, n_recent, in_count, in_off,
                 idx_in: Optional[torch.Tensor], out_count, out_off, idx_out: torch.Tensor,
                 plan: Optional[torch.Tensor] = None):
    if plan is None:
        plan = _plan_for(recall_plan_bytes(B))
    h = _Host()
    _check(load().spa_recall_index(
        int(B), int(num_kv_heads), h.arr(seq_lens, np.int32), int(n_sink), int(n_recent),
        h.arr(in_count, np.int32), h.arr(in_off, np.int64), _dptr(idx_in),
        h.arr(out_count, np.int32), h.arr(out_off, np.int64), _dptr(idx_out), _hptr(plan),
        _nbytes(plan), _stream(idx_out)))


def list_quality_workspace_bytes(B, num_qo_heads, seq_lens) -> int:
    h = _Host()
    return int(load().spa_list_quality_workspace_bytes(int(B), int(num_qo_heads),
                                                       h.arr(seq_lens, np.int32)))


def list_quality_plan_bytes(B: int) -> int:
    return int(load().spa_list_quality_plan_bytes(int(B)))


def list_quality(B, spec_k, num_qo_heads, num_kv_heads, row, top_t, seq_lens, logits, logits_off,
                 lse, list_count, list_off, lists: Optional[torch.Tensor], top: torch.Tensor,
                 coverage: torch.Tensor, recall: torch.Tensor, ws: torch.Tensor,
                 plan: Optional[torch.Tensor] = None):
    if plan is None:
        plan = _plan_for(list_quality_plan_bytes(B))
    h = _Host()
    _check(load().spa_list_quality(
        int(B), int(spec_k), int(num_qo_heads), int(num_kv_heads), int(row), int(top_t),
        h.arr(seq_lens, np.int32), _dptr(logits), h.arr(logits_off, np.int64), _dptr(lse),
        h.arr(list_count, np.int32), h.arr(list_off, np.int64), _dptr(lists), _dptr(top),
        _dptr(coverage), _dptr(recall), _dptr(ws), _nbytes(ws), _hptr(plan), _nbytes(plan),
        _stream(logits)))


def kv_block_bytes(lay: SpaLayout, block_slots: int) -> int:
    return int(load().spa_kv_block_bytes(C.byref(lay), int(block_slots)))


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, np.int32))
    return a, a.ctypes.data_as(C.c_void_p)


def kv_offload(lay, block_slots, dev_blocks, host_chunks, k_pool, v_pool, k_arena, v_arena,
               stream=None, wait_event=None, done_event=None):
    """Device blocks -> host chunks of the pinned arenas, on `stream`
    (a torch.cuda.Stream; None: the current stream)."""
    b, bp = _i32(dev_blocks)
    c, cp = _i32(host_chunks)
    assert len(b) == len(c)
    st = (stream or torch.cuda.current_stream(k_pool.device)).cuda_stream
    _check(load().spa_kv_offload(
        C.byref(lay), int(block_slots), len(b), bp, cp, _dptr(k_pool), _dptr(v_pool),
        _hptr(k_arena), _hptr(v_arena), _nbytes(k_arena),
        None if wait_event is None else C.c_void_p(wait_event.cuda_event),
        None if done_event is None else C.c_void_p(done_event.cuda_event), C.c_void_p(st)))


def kv_prefetch(lay, block_slots, host_chunks, dev_blocks, k_arena, v_arena, k_pool, v_pool,
                stream=None, wait_event=None, done_event=None):
    """Host chunks of the pinned arenas -> device blocks, on `stream`."""
    c, cp = _i32(host_chunks)
    b, bp = _i32(dev_blocks)
    assert len(b) == len(c)
    st = (stream or torch.cuda.current_stream(k_pool.device)).cuda_stream
    _check(load().spa_kv_prefetch(
        C.byref(lay), int(block_slots), len(b), cp, bp, _hptr(k_arena), _hptr(v_arena),
        _nbytes(k_arena), _dptr(k_pool), _dptr(v_pool),
        None if wait_event is None else C.c_void_p(wait_event.cuda_event),
        None if done_event is None else C.c_void_p(done_event.cuda_event), C.c_void_p(st)))


class KVManager:
    """The block manager of include/spa_kvcache.h over a host state buffer
    owned here."""

    def __init__(self, dev_blocks, host_chunks, block_slots, max_requests, max_blocks):
        self.cfg = SpaKvmConfig(int(dev_blocks), int(host_chunks), int(block_slots),
                                int(max_requests), int(max_blocks))
        lib = load()
        n = lib.spa_kvm_bytes(C.byref(self.cfg))
        if n == 0:
            raise SpaError(SPA_ERR_INVALID_ARG, lib.spa_last_error().decode())
        raw = np.zeros(n + 64, np.uint8)
        skip = (-raw.ctypes.data) % 64
        self._raw = raw
        self.ptr = C.c_void_p(raw[skip:].ctypes.data)
        _check(lib.spa_kvm_init(self.ptr, n, C.byref(self.cfg)))
        R = int(max_requests)
        self._reqs = np.zeros(R, np.int32)
        self._cap = 0
        self._a = self._b = np.zeros(0, np.int32)

    def reserve(self, req, length) -> bool:
        """True when the request now holds blocks for `length` positions;
        False when the device blocks ran out (nothing changed)."""
        rc = load().spa_kvm_reserve(self.ptr, int(req), int(length))
        if rc == SPA_ERR_KV_FULL:
            return False
        _check(rc)
        return True

    def release(self, req):
        _check(load().spa_kvm_release(self.ptr, int(req)))

    def _moves(self, cap):
        if cap > self._cap:
            self._cap = cap
            self._a = np.zeros(cap, np.int32)
            self._b = np.zeros(cap, np.int32)
        return self._a, self._b

    def plan_offload(self, need_free, keep=(), cap=1 << 16):
        """(dev_blocks, host_chunks, requests) to move off the device."""
        a, b = self._moves(cap)
        kp = np.ascontiguousarray(np.asarray(keep, np.int32))
        nm, nr = C.c_int32(), C.c_int32()
        _check(load().spa_kvm_plan_offload(
            self.ptr, int(need_free), kp.ctypes.data_as(C.c_void_p) if kp.size else None,
            int(kp.size), int(cap), a.ctypes.data_as(C.c_void_p), b.ctypes.data_as(C.c_void_p),
            C.byref(nm), self._reqs.ctypes.data_as(C.c_void_p), C.byref(nr)))
        return a[:nm.value].copy(), b[:nm.value].copy(), self._reqs[:nr.value].copy()

    def plan_prefetch(self, keep_free=0, cap=1 << 16):
        """(host_chunks, dev_blocks, requests) to bring back."""
        a, b = self._moves(cap)
        nm, nr = C.c_int32(), C.c_int32()
        _check(load().spa_kvm_plan_prefetch(
            self.ptr, int(keep_free), int(cap), a.ctypes.data_as(C.c_void_p),
            b.ctypes.data_as(C.c_void_p), C.byref(nm), self._reqs.ctypes.data_as(C.c_void_p),
            C.byref(nr)))
        return a[:nm.value].copy(), b[:nm.value].copy(), self._reqs[:nr.value].copy()

    def page_row(self, req, length) -> np.ndarray:
        out = np.zeros(max(int(length), 1), np.int32)
        _check(load().spa_kvm_page_row(self.ptr, int(req), int(length),
                                       out.ctypes.data_as(C.c_void_p)))
        return out[:int(length)]

    def where(self, req) -> int:
        return int(load().spa_kvm_where(self.ptr, int(req)))

    def stats(self) -> dict:
        st = SpaKvmStats()
        _check(load().spa_kvm_stats_read(self.ptr, C.byref(st)))
        return {n: int(getattr(st, n)) for n, _ in SpaKvmStats._fields_}


_probe = None
PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspa_probe.so")


def load_probe():
    """libspa_probe.so (include/spa_probe.h); raises if it was not built."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: run "
                               "`python -m sparse_self_speculative_pillarattn_amd.build`")
        lib = C.CDLL(PROBE_LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        lib.spa_probe_ceiling.argtypes = [vp, vp, i64, i32, i64, i32, i32, vp, i64, i32, i32, vp, vp]
        lib.spa_probe_ceiling.restype = i32
        _probe = lib
    return _probe


def probe_ceiling(k_pool, v_pool, num_slots, num_kv_heads, chunks, random, depth, out,
                  write_bytes_per_chunk, grid, sink):
    rc = load_probe().spa_probe_ceiling(
        _dptr(k_pool), _dptr(v_pool), int(num_slots), int(num_kv_heads), int(chunks),
        1 if random else 0, int(depth), _dptr(out), 0 if out is None else _nbytes(out),
        int(write_bytes_per_chunk), int(grid), _dptr(sink), _stream(k_pool))
    if rc:
        raise SpaError(SPA_ERR_INVALID_ARG if rc == 1 else SPA_ERR_HIP,
                       f"spa_probe_ceiling failed ({rc})")


class PlanRing:
    """A few pinned plan buffers used in turn, so the host can queue that many
    calls ahead of the GPU (a call waits only for the buffer's previous use)."""

    def __init__(self, nbytes: int, n: int = 4):
        self.bufs = [plan_buffer(nbytes) for _ in range(n)]
        self.args = [(_hptr(b), _nbytes(b)) for b in self.bufs]
        self.i = 0

    @property
    def nbytes(self) -> int:
        return _nbytes(self.bufs[0])

    def next(self) -> torch.Tensor:
        b = self.bufs[self.i]
        self.i = (self.i + 1) % len(self.bufs)
        return b

    def next_args(self):
        """(address, bytes) of the next buffer, as ctypes arguments."""
        a = self.args[self.i]
        self.i = (self.i + 1) % len(self.bufs)
        return a


# --------------------------------------------------------------------------- #
# convenience: run one synthetic batch through the unified step
# --------------------------------------------------------------------------- #
class StepBuffers:
    """Output, workspace and plan buffers for one synthetic batch (see synth.Batch)."""

    def __init__(self, batch, avg_row_begin: int = 1, avg_row_count: Optional[int] = None,
                 opts: Optional[Options] = None, n_plans: int = 4):
        w = batch.w
        dev = batch.q.device
        self.batch = batch
        self.opts = opts if opts is not None else default_options(dev)
        self.lay = layout(w.num_qo_heads, w.num_kv_heads, w.head_dim, batch.q.dtype,
                          batch.num_slots, batch.stride)
        self.o = torch.empty_like(batch.q)
        self.lse = torch.empty((batch.rows, w.num_qo_heads), dtype=torch.float32, device=dev)
        self.logits = torch.empty((batch.logits_elems,), dtype=torch.float32, device=dev)
        self.idx = batch.idx.clone()
        self.avg_row_begin = avg_row_begin
        self.avg_row_count = w.spec_k if avg_row_count is None else avg_row_count
        sizes = (self.lay, batch.B, w.spec_k, batch.is_verify, batch.seq_lens, batch.idx_count,
                 self.opts)
        self.ws = workspace(workspace_bytes(*sizes), dev)
        self.plans = PlanRing(plan_bytes(*sizes), n_plans)
        # host metadata typed once, so a step only marshals pointers
        self.h_is_verify = np.ascontiguousarray(batch.is_verify, dtype=np.uint8)
        self.h_seq_lens = np.ascontiguousarray(batch.seq_lens, dtype=np.int32)
        self.h_q_indptr = np.ascontiguousarray(batch.q_indptr, dtype=np.int32)
        self.h_idx_count = np.ascontiguousarray(batch.idx_count, dtype=np.int32)
        self.h_idx_off = np.ascontiguousarray(batch.idx_off, dtype=np.int64)
        self.h_logits_off = np.ascontiguousarray(np.maximum(batch.logits_off, 0), dtype=np.int64)

        self._key = None
        self._args = None

    def _marshal(self):
        """The ctypes arguments of one call before the plan buffer, rebuilt only
        when an output, index or workspace buffer has moved or resized."""
        key = (self.idx.data_ptr(), self.o.data_ptr(), self.lse.data_ptr(),
               self.logits.data_ptr(), self.ws.data_ptr(), _nbytes(self.ws))
        if key != self._key:
            b = self.batch
            host = [np.ascontiguousarray(a) for a in (self.h_is_verify, self.h_seq_lens,
                                                       self.h_q_indptr, self.h_idx_count,
                                                       self.h_idx_off, self.h_logits_off)]
            self._host = host
            hp = [C.c_void_p(a.ctypes.data) for a in host]
            self._args = (C.byref(self.lay), int(b.B), int(b.w.spec_k), hp[0], hp[1], hp[2],
                          _dptr(b.page_table), _dptr(b.q), _dptr(b.k_pool), _dptr(b.v_pool),
                          hp[3], hp[4], _dptr(self.idx), _dptr(self.o), _dptr(self.lse),
                          _dptr(self.logits), hp[5], int(self.avg_row_begin),
                          int(self.avg_row_count), _dptr(self.ws), _nbytes(self.ws))
            self._key = key
        return self._args

    def step(self, opts: Optional[Options] = None):
        """One unified step on the current stream (opts: instead of the buffers' own)."""
        _check(load().spa_unified_step(*self._marshal(), *self.plans.next_args(),
                                       _opts(self.opts if opts is None else opts),
                                       _stream(self.batch.q)))


# --------------------------------------------------------------------------- #
# the scheduler of include/spa_sched.h
# --------------------------------------------------------------------------- #
class Scheduler:
    """Phase buckets and delayed verification over ``slots`` batch slots; the
    state lives in a host buffer owned here.  next() plans a step (numpy views
    of the scheduler's arrays, valid until the following call), commit()
    applies it."""

    def __init__(self, slots, spec_k, num_qo_heads, num_kv_heads, sparsity, prompt, output,
                 max_len, delayed=False, accept_prob=ACCEPT_PROB_6_16_OF_8, seed=0):
        from fractions import Fraction
        s = Fraction(str(sparsity)) if isinstance(sparsity, float) else Fraction(sparsity)
        self.cfg = SpaSchedConfig(int(slots), int(spec_k), 1 if delayed else 0, int(num_qo_heads),
                                  int(num_kv_heads), s.numerator, s.denominator, int(prompt[0]),
                                  int(prompt[1]), int(output[0]), int(output[1]), int(max_len),
                                  float(accept_prob), int(seed))
        lib = load()
        n = lib.spa_sched_bytes(C.byref(self.cfg))
        if n == 0:
            raise SpaError(SPA_ERR_INVALID_ARG, lib.spa_last_error().decode())
        raw = np.zeros(n + 64, np.uint8)
        skip = (-raw.ctypes.data) % 64
        self._raw = raw
        self.state = raw[skip:skip + n]
        self.ptr = C.c_void_p(self.state.ctypes.data)
        _check(lib.spa_sched_init(self.ptr, n, C.byref(self.cfg)))
        ie, le, rw = C.c_int64(), C.c_int64(), C.c_int32()
        _check(lib.spa_sched_capacity(C.byref(self.cfg), C.byref(ie), C.byref(le), C.byref(rw)))
        self.idx_elems, self.logits_elems, self.max_rows = int(ie.value), int(le.value), int(rw.value)
        self.cycle = int(spec_k) + 1 + (1 if delayed else 0)
        self.step_c = SpaSchedStep()

    def next(self) -> SpaSchedStep:
        """Plans the next step; returns the step record (ctypes, pointers into the state)."""
        _check(load().spa_sched_next(self.ptr, C.byref(self.step_c)))
        return self.step_c

    def commit(self):
        _check(load().spa_sched_commit(self.ptr))

    def stats(self) -> dict:
        st = SpaSchedStats()
        _check(load().spa_sched_stats_read(self.ptr, C.byref(st)))
        return {n: int(getattr(st, n)) for n, _ in SpaSchedStats._fields_}

    def buckets(self) -> np.ndarray:
        out = np.zeros(self.cycle, np.int32)
        _check(load().spa_sched_buckets(self.ptr, out.ctypes.data_as(C.POINTER(C.c_int32)),
                                        self.cycle))
        return out

    @staticmethod
    def view(ptr, n, dtype):
        """numpy copy-free view of n elements of a scheduler array."""
        if n == 0:
            return np.zeros(0, dtype)
        ct = {np.uint8: C.c_uint8, np.int32: C.c_int32, np.int64: C.c_int64}[dtype]
        return np.ctypeslib.as_array(C.cast(ptr, C.POINTER(ct)), shape=(n,))

    def arrays(self, st: SpaSchedStep) -> dict:
        """The step's arrays as numpy views."""
        v = self.view
        return {"is_verify": v(st.is_verify, st.B, np.uint8), "seq_lens": v(st.seq_lens, st.B, np.int32),
                "q_indptr": v(st.q_indptr, st.B + 1, np.int32),
                "idx_count": v(st.idx_count, st.B, np.int32), "idx_off": v(st.idx_off, st.B, np.int64),
                "logits_off": v(st.logits_off, st.B, np.int64), "slot": v(st.slot, st.B, np.int32),
                "new_slots": v(st.new_slots, st.n_new, np.int32),
                "new_len": v(st.new_len, st.n_new, np.int32),
                "new_count": v(st.new_count, st.n_new, np.int32)}
