"""libspa loads, exports what include/spa.h declares, and rejects bad
arguments on the host before anything is enqueued -- CPU only (no device
pointer is dereferenced on these paths, so fake non-null addresses stand in)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from sparse_self_speculative_pillarattn_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = C.c_void_p(0x1000)  # never dereferenced on the paths below


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):  # a fresh checkout: cross-compile it (no GPU needed)
        from sparse_self_speculative_pillarattn_amd import build
        build.build()
    return bd.load()


def declared_symbols(header="spa.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spa_[a-z_]+)\s*\(", src)))


@pytest.mark.parametrize("header,exported", [("spa.h", bd.EXPORTED),
                                             ("spa_sched.h", bd.SCHED_EXPORTED),
                                             ("spa_kvcache.h", bd.KV_EXPORTED)])
def test_exports_every_declared_symbol(lib, header, exported):
    names = declared_symbols(header)
    assert set(names) == set(exported), names
    for n in names:
        assert hasattr(lib, n), n


def test_scheduler_structs_match_the_header():
    """Field counts and sizes of the ctypes mirrors of include/spa_sched.h."""
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "spa_sched.h")).read(),
                 flags=re.S)
    for name, cls in (("spa_sched_config", bd.SpaSchedConfig), ("spa_sched_step", bd.SpaSchedStep),
                      ("spa_sched_stats", bd.SpaSchedStats)):
        body = re.search(r"typedef struct \{([^{}]*)\}\s*" + name + ";", src, flags=re.S).group(1)
        fields = []
        for decl in body.split(";"):
            decl = decl.strip()
            if decl:
                fields += [f.strip().lstrip("*") for f in decl.split(None, 1)[1].split(",")]
        if name == "spa_sched_step":  # pointer declarators carry the type's const
            fields = [f.split()[-1].lstrip("*") for f in fields]
        assert [f for f, _ in cls._fields_] == fields, name


def test_abi_version(lib):
    assert lib.spa_abi_version() == bd.ABI_VERSION == 2


def _lay(**kw):
    d = dict(num_qo_heads=8, num_kv_heads=2, head_dim=128, sm_scale=0.0, dtype=0,
             num_slots=4096, page_table_stride=512)
    d.update(kw)
    return bd.SpaLayout(**d)


def _arr(a, dt):
    a = np.ascontiguousarray(np.asarray(a, dtype=dt))
    return a, a.ctypes.data_as(C.c_void_p)


def _unified(lib, lay, B=2, k=4, ver=(1, 0), lens=(100, 50), indptr=(0, 5, 6), counts=(5, 3),
             ioff=(0, 10), loff=(0, 0), ws_bytes=1 << 30, avg=(1, 4), null=(), plan=FAKE,
             plan_bytes=1 << 30, opts=None):
    ver_a, ver_p = _arr(ver, np.uint8)
    len_a, len_p = _arr(lens, np.int32)
    ind_a, ind_p = _arr(indptr, np.int32)
    cnt_a, cnt_p = _arr(counts, np.int32)
    io_a, io_p = _arr(ioff, np.int64)
    lo_a, lo_p = _arr(loff, np.int64)
    args = dict(ver=ver_p, lens=len_p, indptr=ind_p, pt=FAKE, q=FAKE, kp=FAKE, vp=FAKE,
                cnt=cnt_p, ioff=io_p, idx=FAKE, o=FAKE, lse=FAKE, logits=FAKE, loff=lo_p,
                ws=FAKE, plan=plan)
    for n in null:
        args[n] = None
    return lib.spa_unified_step(C.byref(lay), B, k, args["ver"], args["lens"], args["indptr"],
                                args["pt"], args["q"], args["kp"], args["vp"], args["cnt"],
                                args["ioff"], args["idx"], args["o"], args["lse"], args["logits"],
                                args["loff"], avg[0], avg[1], args["ws"], ws_bytes, args["plan"],
                                plan_bytes, None if opts is None else C.byref(opts), None)


def test_valid_arguments_reach_workspace_check(lib):
    rc = _unified(lib, _lay(), ws_bytes=0)
    assert rc == bd.SPA_ERR_WORKSPACE_TOO_SMALL
    assert b"workspace" in lib.spa_last_error()


def test_empty_batch_is_a_noop(lib):
    assert _unified(lib, _lay(), B=0, ws_bytes=0) == bd.SPA_OK


_PT_KEEP = []


def _pt_rows(rows, count):
    """Options that map request r to page-table row rows[r] (of `count`)."""
    a = np.asarray(rows, np.int32)
    _PT_KEEP.append(a)
    return bd.SpaOptions(page_table_rows=a.ctypes.data,
                         page_table_row_count=count)


@pytest.mark.parametrize("kw,code", [
    (dict(lay=dict(num_qo_heads=6, num_kv_heads=4)), bd.SPA_ERR_INVALID_ARG),
    (dict(lay=dict(num_kv_heads=0)), bd.SPA_ERR_INVALID_ARG),
    (dict(lay=dict(head_dim=96)), bd.SPA_ERR_UNSUPPORTED),
    (dict(lay=dict(dtype=7)), bd.SPA_ERR_UNSUPPORTED),
    (dict(lay=dict(num_slots=0)), bd.SPA_ERR_INVALID_ARG),
    (dict(lay=dict(page_table_stride=64)), bd.SPA_ERR_INVALID_ARG),   # L exceeds stride
    (dict(lay=dict(sm_scale=-1.0)), bd.SPA_ERR_INVALID_ARG),
    (dict(B=-1), bd.SPA_ERR_INVALID_ARG),
    (dict(k=0), bd.SPA_ERR_INVALID_ARG),
    (dict(lens=(3, 50)), bd.SPA_ERR_INVALID_ARG),          # verify shorter than k+1
    (dict(lens=(100, 0)), bd.SPA_ERR_INVALID_ARG),         # empty context
    (dict(counts=(0, 3)), bd.SPA_ERR_INVALID_ARG),         # K_r < 1
    (dict(counts=(101, 3)), bd.SPA_ERR_INVALID_ARG),       # K_r > L_r
    (dict(counts=(5, 0)), bd.SPA_ERR_INVALID_ARG),         # empty draft list
    (dict(indptr=(0, 4, 5)), bd.SPA_ERR_INVALID_ARG),      # verify must own k+1 rows
    (dict(indptr=(0, 5, 7)), bd.SPA_ERR_INVALID_ARG),      # draft must own 1 row
    (dict(ioff=(0, 5)), bd.SPA_ERR_INVALID_ARG),           # overlapping idx segments
    (dict(ioff=(-2, 10)), bd.SPA_ERR_INVALID_ARG),         # negative offset
    (dict(loff=(-1, 0)), bd.SPA_ERR_INVALID_ARG),          # negative logits offset
    (dict(avg=(0, 6)), bd.SPA_ERR_INVALID_ARG),            # rows beyond k
    (dict(avg=(1, 0)), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("q",)), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("ws",), ws_bytes=1 << 30), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("logits",)), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("plan",)), bd.SPA_ERR_INVALID_ARG),
    (dict(plan=C.c_void_p(0x1010)), bd.SPA_ERR_INVALID_ARG),  # plan buffer not 64-byte aligned
    (dict(plan_bytes=256), bd.SPA_ERR_PLAN_TOO_SMALL),
    (dict(opts=bd.SpaOptions(verify_chunk=-1)), bd.SPA_ERR_INVALID_ARG),
    (dict(opts=bd.SpaOptions(draft_chunk=2049)), bd.SPA_ERR_INVALID_ARG),
    (dict(opts=bd.SpaOptions(num_cus=-4)), bd.SPA_ERR_INVALID_ARG),
    (dict(opts=bd.SpaOptions(overlap=1)), bd.SPA_ERR_INVALID_ARG),  # no side stream or events
    (dict(opts=_pt_rows((0, 2), 2)), bd.SPA_ERR_INVALID_ARG),       # row index past the count
    (dict(opts=_pt_rows((-1, 0), 2)), bd.SPA_ERR_INVALID_ARG),      # negative row index
    (dict(opts=_pt_rows((0, 1), 0)), bd.SPA_ERR_INVALID_ARG),       # rows given, count 0
    (dict(lay=dict(num_qo_heads=192, num_kv_heads=8), ioff=(0, 100)),
     bd.SPA_ERR_UNSUPPORTED),  # (k+1) G = 120 rows exceed the 112-row MFMA budget
])
def test_unified_step_rejects(lib, kw, code):
    lay = _lay(**kw.pop("lay", {}))
    assert _unified(lib, lay, **kw) == code
    assert lib.spa_last_error()


def test_two_verifies_need_disjoint_logits(lib):
    rc = _unified(lib, _lay(), ver=(1, 1), indptr=(0, 5, 10), counts=(5, 3), loff=(0, 100),
                  lens=(100, 50))
    assert rc == bd.SPA_ERR_INVALID_ARG
    assert b"logits" in lib.spa_last_error()


def _sizes(lib, lay, B, k, ver, lens, cnt, opts=None):
    v, l, c = (np.ascontiguousarray(np.asarray(a, t)) for a, t in
               ((ver, np.uint8), (lens, np.int32), (cnt, np.int32)))
    args = (C.byref(lay), B, k, v.ctypes.data_as(C.c_void_p), l.ctypes.data_as(C.c_void_p),
            c.ctypes.data_as(C.c_void_p), None if opts is None else C.byref(opts))
    return lib.spa_workspace_bytes(*args), lib.spa_plan_bytes(*args)


def test_workspace_bytes_matches_call_requirement(lib):
    lay = _lay()
    need, plan = _sizes(lib, lay, 2, 4, [1, 0], [100, 50], [5, 3])
    assert need > 256 and plan > 256
    assert _unified(lib, lay, ws_bytes=need - 1) == bd.SPA_ERR_WORKSPACE_TOO_SMALL
    assert _unified(lib, lay, ws_bytes=need, plan_bytes=plan - 1) == bd.SPA_ERR_PLAN_TOO_SMALL


def test_sizes_are_pure_functions_of_their_arguments(lib):
    """Workspace and plan sizes depend on the batch and the options only: the
    same arguments give the same sizes, the CU count the automatic verify
    chunk plans for is an option, and invalid options give 0."""
    lay = _lay(page_table_stride=8192)
    args = (2, 4, [1, 1], [8000, 6000], [400, 300])
    first = _sizes(lib, lay, *args)
    assert first == _sizes(lib, lay, *args) == _sizes(lib, lay, *args, opts=bd.SpaOptions())
    # 14000 positions x 2 KV heads on 256 CUs: a light load, 512-position
    # chunks; planned for 2 CUs (four resident workgroups), 2048-position
    # chunks (14 items, at least two per workgroup) and far fewer partials
    few = _sizes(lib, lay, *args, opts=bd.SpaOptions(num_cus=2))
    assert few[0] < first[0] and few[1] < first[1]
    assert _sizes(lib, lay, *args, opts=bd.SpaOptions(num_cus=256)) == first
    # an explicit chunk is used as given
    assert _sizes(lib, lay, *args, opts=bd.SpaOptions(verify_chunk=2048)) == few
    assert _sizes(lib, lay, *args, opts=bd.SpaOptions(verify_chunk=4096)) == (0, 0)
    assert b"verify_chunk" in lib.spa_last_error()


def test_workspace_holds_a_histogram_per_selected_row(lib):
    """Turning a draft into a verify request adds, besides its averaged
    scores, one 2048-bin uint32 score histogram per KV head to the workspace
    (the post-pass counts into it, the selection starts from it)."""
    lay = _lay()
    lens = np.array([100, 100], np.int32)
    cnt = np.array([5, 5], np.int32)

    def need(ver):
        return _sizes(lib, lay, 2, 4, ver, lens, cnt)[0]
    assert need([1, 1]) - need([1, 0]) >= lay.num_kv_heads * 2048 * 4


@pytest.mark.parametrize("lens,want", [
    ([8192] * 14, 512),          # 14 x 16 x 8 = 1792 items at 512, 896 at 1024 (< 2 x 512)
    ([80558, 126350], 1536),     # 1088 items at 1536 (>= 1024), 816 at 2048
    ([13500] * 20, 2048),        # 7 x 20 x 8 = 1120 items at 2048 with one workgroup per CU
])
def test_automatic_verify_chunk(lib, lens, want):
    """The automatic verify chunk is the longest of 2048, 1536 and 1024 that
    gives at least two verify items per resident attention workgroup (two per
    CU up to 48 query rows per KV head, one above), else 512: the workspace
    equals the one planned with that chunk given explicitly."""
    G = 5 if want == 2048 else 4    # (k+1) G = 45 rows or more: one workgroup per CU
    k = 12 if want == 2048 else 8
    lay = _lay(num_qo_heads=8 * G, num_kv_heads=8, page_table_stride=1 << 17)
    B = len(lens)
    args = (B, k, [1] * B, lens, [max(1, L // 20) for L in lens])
    auto = _sizes(lib, lay, *args)
    assert auto[0] > 0, lib.spa_last_error()
    assert auto == _sizes(lib, lay, *args, opts=bd.SpaOptions(verify_chunk=want))
    for other in (512, 1024, 1536, 2048):
        if other != want:
            assert _sizes(lib, lay, *args, opts=bd.SpaOptions(verify_chunk=other)) != auto, other


def test_draft_packing_beside_verify_items(lib):
    """Short draft lists go two KV heads to an item while the draft items
    still number one per CU beside verify items, or two per CU in a
    draft-only call (Qwen3-8B shape: 114 drafts x 8 KV heads of 13-tile
    lists; 64-byte records)."""
    lay = _lay(num_qo_heads=32, num_kv_heads=8, page_table_stride=8192)
    nv, nd = 14, 114
    ver = [1] * nv + [0] * nd
    lens = [8192] * (nv + nd)
    cnt = [410] * (nv + nd)
    mixed = _sizes(lib, lay, nv + nd, 8, ver, lens, cnt)[1]
    verify_only = _sizes(lib, lay, nv, 8, ver[:nv], lens[:nv], cnt[:nv])[1]
    draft_only = _sizes(lib, lay, nd, 8, ver[nv:], lens[nv:], cnt[nv:])[1]
    empty = _sizes(lib, lay, 0, 8, [], [], [])[1]
    drafts_beside_verify = (mixed - verify_only) // 64
    drafts_alone = (draft_only - empty) // 64
    assert abs(drafts_beside_verify - nd * 8 // 2) <= 4, drafts_beside_verify   # 456 items
    assert abs(drafts_alone - nd * 8) <= 4, drafts_alone                        # 912 items


def test_light_verify_load_with_a_very_long_request_is_planned(lib):
    """A light verify load gets 512-position chunks, but not so many that one
    request needs more than the 256 split-K chunks a merge takes: a lone
    140,000-token verify request is still planned (longer chunks)."""
    lay = _lay(page_table_stride=1 << 20)
    for L in (131072, 140000, 1 << 19):
        ver = np.array([1], np.uint8)
        lens = np.array([L], np.int32)
        cnt = np.array([L // 20], np.int32)
        need = _sizes(lib, lay, 1, 4, ver, lens, cnt)[0]
        assert need > 0, (L, lib.spa_last_error())


def test_verify_row_beyond_the_split_k_limit_is_refused(lib):
    """524,288 positions (256 split-K chunks of 2048) is the longest verify
    row; one position more is refused before anything is enqueued."""
    lay = _lay(page_table_stride=1 << 20)
    ver = np.array([1], np.uint8)
    for L, ok in ((1 << 19, True), ((1 << 19) + 1, False)):
        lens = np.array([L], np.int32)
        cnt = np.array([L // 50], np.int32)
        need = _sizes(lib, lay, 1, 4, ver, lens, cnt)[0]
        assert (need > 0) == ok, (L, lib.spa_last_error())
    assert b"256 split-K chunks" in lib.spa_last_error()


def test_unpinned_plan_buffer_is_rejected(lib):
    """A plan buffer the device cannot read (ordinary host memory) is refused
    before anything is enqueued."""
    buf = np.zeros(1 << 16, np.uint8)
    addr = (buf.ctypes.data + 63) // 64 * 64
    rc = _unified(lib, _lay(), plan=C.c_void_p(addr), plan_bytes=(1 << 16) - 64)
    assert rc == bd.SPA_ERR_INVALID_ARG
    assert b"pinned" in lib.spa_last_error()
    assert not buf.any(), "the rejected buffer was written"


def test_other_entry_points_validate(lib):
    # work chunks of 512 positions / 256 list entries
    opts = C.byref(bd.SpaOptions(verify_chunk=512, draft_chunk=256))
    P, PB = FAKE, 1 << 30
    lay = _lay(page_table_stride=2048)
    # lengths above one work chunk, so that every call below needs workspace
    lens, lp = _arr([1000, 800], np.int32)
    lo, lop = _arr([0, 5 * 8 * 1000], np.int64)
    # verify-only: k+1 rows per request, L >= k+1
    assert lib.spa_verify_attn(C.byref(lay), 2, 0, lp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               lop, FAKE, 0, P, PB, opts, None) == bd.SPA_ERR_INVALID_ARG
    assert lib.spa_verify_attn(C.byref(lay), 2, 4, lp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               lop, FAKE, 0, P, PB, opts, None) == bd.SPA_ERR_WORKSPACE_TOO_SMALL
    # top-K: K within [1, L], rows within [0, k]
    kk, kp = _arr([5, 801], np.int32)
    io, iop = _arr([0, 4000], np.int64)
    assert lib.spa_pillar_topk(2, 4, 8, 2, 1, 4, lp, kp, FAKE, lop, FAKE, FAKE, iop, FAKE, 0,
                               P, PB, opts, None) == bd.SPA_ERR_INVALID_ARG
    kk, kp = _arr([5, 8], np.int32)
    assert lib.spa_pillar_topk(2, 4, 8, 2, 1, 5, lp, kp, FAKE, lop, FAKE, FAKE, iop, FAKE, 0,
                               P, PB, opts, None) == bd.SPA_ERR_INVALID_ARG
    assert lib.spa_pillar_topk(2, 4, 8, 3, 1, 4, lp, kp, FAKE, lop, FAKE, FAKE, iop, FAKE, 0,
                               P, PB, opts, None) == bd.SPA_ERR_INVALID_ARG
    assert lib.spa_pillar_topk(2, 4, 8, 2, 1, 4, lp, kp, FAKE, lop, FAKE, FAKE, iop, FAKE, 0,
                               P, PB, opts, None) == bd.SPA_ERR_WORKSPACE_TOO_SMALL
    # draft-only: non-empty lists, disjoint segments
    cnt, cp = _arr([4, 0], np.int32)
    assert lib.spa_draft_attn(C.byref(lay), 2, lp, FAKE, cp, iop, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, 0, P, PB, opts, None) == bd.SPA_ERR_INVALID_ARG
    cnt, cp = _arr([1500, 4], np.int32)
    io, iop = _arr([0, 4000], np.int64)
    assert lib.spa_draft_attn(C.byref(lay), 2, lp, FAKE, cp, iop, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, 0, P, PB, opts, None) == bd.SPA_ERR_WORKSPACE_TOO_SMALL


# --------------------------------------------------------------------------- #
# spa_recall_index argument checks
# --------------------------------------------------------------------------- #
def _recall(lib, B=2, Hkv=2, lens=(100, 50), S=4, W=8, inc=(10, 5), inoff=(0, 100),
            outc=None, outoff=(1000, 2000), in_ptr=0x10000, out_ptr=0x10000, null=(),
            plan_bytes=1 << 20):
    if outc is None:
        outc = [bd.recall_length(L, n, S, W) for L, n in zip(lens, inc)]
    len_a, len_p = _arr(lens, np.int32)
    inc_a, inc_p = _arr(inc, np.int32)
    ino_a, ino_p = _arr(inoff, np.int64)
    outc_a, outc_p = _arr(outc, np.int32)
    outo_a, outo_p = _arr(outoff, np.int64)
    args = dict(lens=len_p, inc=inc_p, inoff=ino_p, idx_in=C.c_void_p(in_ptr), outc=outc_p,
                outoff=outo_p, idx_out=C.c_void_p(out_ptr), plan=FAKE)
    for n in null:
        args[n] = None
    return lib.spa_recall_index(B, Hkv, args["lens"], S, W, args["inc"], args["inoff"],
                                args["idx_in"], args["outc"], args["outoff"], args["idx_out"],
                                args["plan"], plan_bytes, None)


def test_recall_length_formula():
    assert bd.recall_length(100, 10, 4, 8) == 22
    assert bd.recall_length(100, 95, 4, 8) == 100       # never more than L
    assert bd.recall_length(10, 0, 50, 0) == 10          # sinks cover everything
    assert bd.recall_length(10, 0, 6, 6) == 10           # sinks and window overlap
    assert bd.recall_length(1, 0, 0, 0) == 1             # at least one entry


@pytest.mark.parametrize("kw,code", [
    (dict(S=-1), bd.SPA_ERR_INVALID_ARG),
    (dict(W=-2), bd.SPA_ERR_INVALID_ARG),
    (dict(Hkv=0), bd.SPA_ERR_INVALID_ARG),
    (dict(B=-1), bd.SPA_ERR_INVALID_ARG),
    (dict(lens=(0, 50)), bd.SPA_ERR_INVALID_ARG),
    (dict(lens=((1 << 20) + 1, 50)), bd.SPA_ERR_UNSUPPORTED),
    (dict(inc=(-1, 5)), bd.SPA_ERR_INVALID_ARG),
    (dict(outc=(21, 17)), bd.SPA_ERR_INVALID_ARG),            # first needs 22
    (dict(inoff=(-4, 100)), bd.SPA_ERR_INVALID_ARG),
    (dict(outoff=(1000, 1030)), bd.SPA_ERR_INVALID_ARG),      # output lists overlap
    (dict(outoff=(90, 2000)), bd.SPA_ERR_INVALID_ARG),        # output over a stored list
    (dict(null=("idx_in",)), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("outc",)), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("idx_out",)), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("plan",)), bd.SPA_ERR_INVALID_ARG),
    (dict(plan_bytes=256 + 32), bd.SPA_ERR_PLAN_TOO_SMALL),   # two 32-byte records
])
def test_recall_invalid_arguments(lib, kw, code):
    assert _recall(lib, **kw) == code
    assert lib.spa_last_error()


def test_recall_empty_batch_is_a_noop(lib):
    assert _recall(lib, B=0) == bd.SPA_OK


# --------------------------------------------------------------------------- #
# spa_list_quality argument checks
# --------------------------------------------------------------------------- #
def _quality(lib, B=2, k=1, Hq=8, Hkv=2, row=1, T=10, lens=(100, 50), loff=(0, 1600),
             cnt=(5, 3), coff=(0, 10), ws_bytes=1 << 30, ws=0x10000, null=(), plan_bytes=1 << 20):
    len_a, len_p = _arr(lens, np.int32)
    lo_a, lo_p = _arr(loff, np.int64)
    c_a, c_p = _arr(cnt, np.int32)
    co_a, co_p = _arr(coff, np.int64)
    args = dict(lens=len_p, logits=FAKE, loff=lo_p, lse=FAKE, cnt=c_p, coff=co_p, lst=FAKE,
                top=FAKE, cov=FAKE, rec=FAKE, ws=C.c_void_p(ws), plan=FAKE)
    for n in null:
        args[n] = None
    return lib.spa_list_quality(B, k, Hq, Hkv, row, T, args["lens"], args["logits"], args["loff"],
                                args["lse"], args["cnt"], args["coff"], args["lst"], args["top"],
                                args["cov"], args["rec"], args["ws"], ws_bytes, args["plan"],
                                plan_bytes, None)


def test_list_quality_workspace_formula(lib):
    assert bd.list_quality_workspace_bytes(2, 8, [100, 50]) == 8 * 4 * (100 + 52)
    assert bd.list_quality_workspace_bytes(0, 8, [100]) == 0


def test_plan_bytes_of_recall_and_quality(lib):
    assert lib.spa_recall_plan_bytes(3) == 256 + 3 * 32
    assert lib.spa_list_quality_plan_bytes(3) == 256 + 3 * 40
    assert lib.spa_recall_plan_bytes(-1) == 0 and lib.spa_list_quality_plan_bytes(-1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), bd.SPA_ERR_INVALID_ARG),
    (dict(k=0), bd.SPA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), bd.SPA_ERR_INVALID_ARG),
    (dict(row=2), bd.SPA_ERR_INVALID_ARG),
    (dict(row=-1), bd.SPA_ERR_INVALID_ARG),
    (dict(T=0), bd.SPA_ERR_INVALID_ARG),
    (dict(T=51), bd.SPA_ERR_INVALID_ARG),                     # above the second request's L
    (dict(lens=(1, 50), T=1), bd.SPA_ERR_INVALID_ARG),        # L < spec_k + 1
    (dict(lens=((1 << 20) + 1, 50)), bd.SPA_ERR_UNSUPPORTED),
    (dict(cnt=(-1, 3)), bd.SPA_ERR_INVALID_ARG),
    (dict(loff=(0, 1000)), bd.SPA_ERR_INVALID_ARG),           # logits segments overlap
    (dict(coff=(-2, 10)), bd.SPA_ERR_INVALID_ARG),
    (dict(ws_bytes=100), bd.SPA_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=0x10004), bd.SPA_ERR_INVALID_ARG),               # workspace not 16-byte aligned
    (dict(null=("lst",)), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("top",)), bd.SPA_ERR_INVALID_ARG),
    (dict(null=("plan",)), bd.SPA_ERR_INVALID_ARG),
    (dict(plan_bytes=256 + 40), bd.SPA_ERR_PLAN_TOO_SMALL),   # two 40-byte records
])
def test_list_quality_invalid_arguments(lib, kw, code):
    assert _quality(lib, **kw) == code
    assert lib.spa_last_error()


def test_list_quality_empty_batch_is_a_noop(lib):
    assert _quality(lib, B=0) == bd.SPA_OK


def test_probe_library_exports_and_rejects():
    """libspa_probe exports what include/spa_probe.h declares and rejects bad
    arguments before launching anything."""
    if not os.path.exists(bd.PROBE_LIB_PATH):
        from sparse_self_speculative_pillarattn_amd import build
        build.build()
    lib = bd.load_probe()
    assert declared_symbols("spa_probe.h") == ["spa_probe_ceiling"]
    f = lib.spa_probe_ceiling
    ok = dict(k=FAKE, v=FAKE, ns=1024, h=8, ch=10, rnd=1, dep=2, out=FAKE, ob=3200, wb=320,
              grid=64, sink=FAKE)
    for bad in (dict(k=None), dict(ns=0), dict(h=0), dict(ch=-1), dict(dep=3), dict(wb=8),
                dict(wb=4112), dict(ob=3000), dict(out=None), dict(grid=0), dict(sink=None)):
        a = dict(ok, **bad)
        assert f(a["k"], a["v"], a["ns"], a["h"], a["ch"], a["rnd"], a["dep"], a["out"], a["ob"],
                 a["wb"], a["grid"], a["sink"], None) == 1, bad
    a = dict(ok, ch=0)  # nothing to do: returns before any launch
    assert f(a["k"], a["v"], a["ns"], a["h"], a["ch"], a["rnd"], a["dep"], a["out"], a["ob"],
             a["wb"], a["grid"], a["sink"], None) == 0
