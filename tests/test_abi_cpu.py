"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects invalid arguments before any HIP call (so no GPU is needed here).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("ltopk.h", "ltopk_debug.h")]
LIB = os.path.join(ROOT, "topk_index_selection_amd", "libltopk.so")

LT_OK, LT_EINVAL, LT_ENOSPC, LT_EHIP = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from topk_index_selection_amd import build_lib
        build_lib.build()
    L = ctypes.CDLL(LIB)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.lt_topk_run.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    L.lt_topk_run.restype = ctypes.c_int
    L.lt_topk_blocks.argtypes = [vp, i64, vp, i32, i32, i32, i32, vp, vp, sz, vp]
    L.lt_topk_blocks.restype = ctypes.c_int
    L.lt_topk_two_stage.argtypes = [vp, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    L.lt_topk_two_stage.restype = ctypes.c_int
    L.lt_topk_workspace_bytes.argtypes = [i32, i32, i32]
    L.lt_topk_workspace_bytes.restype = sz
    L.lt_topk_order.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp]
    L.lt_topk_order.restype = ctypes.c_int
    L.lt_gather_rows.argtypes = [vp, i64, i64, i64, i32, vp, i32, i32, vp, vp]
    L.lt_gather_rows.restype = ctypes.c_int
    L.lt_status_str.argtypes = [ctypes.c_int]
    L.lt_status_str.restype = ctypes.c_char_p
    return L


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(lt_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"lt_topk_run", "lt_topk_blocks", "lt_topk_workspace_bytes", "lt_status_str",
            "lt_topk_order", "lt_gather_rows"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (LT_OK, LT_EINVAL, LT_ENOSPC, LT_EHIP, 99):
        s = lib.lt_status_str(code)
        assert s and len(s) > 3


def test_workspace_bytes_is_pure_arithmetic(lib):
    assert lib.lt_topk_workspace_bytes(0, 262144, 512) == 0
    assert lib.lt_topk_workspace_bytes(64, 1024, 512) == 0       # one workgroup per row
    one = lib.lt_topk_workspace_bytes(1, 262144, 512)
    assert one > 0 and one % 256 == 0
    assert lib.lt_topk_workspace_bytes(64, 32768, 512) == 64 * one
    # capped: never more rows than one launch can hold
    assert lib.lt_topk_workspace_bytes(8192, 262144, 512) == lib.lt_topk_workspace_bytes(1024, 262144, 512)


@pytest.mark.parametrize("n_max", [1025, 1500, 2048, 4096])
def test_workspace_needed_past_the_smallest_split_chunk(lib, n_max):
    """A block stage with block_size 1 splits rows of more than 1024 blocks over
    workgroups, so every n_max above 1024 needs a workspace; 1024 and below fit
    one workgroup in every form."""
    assert lib.lt_topk_workspace_bytes(1, 1024, 512) == 0
    assert lib.lt_topk_workspace_bytes(1, n_max, 512) == lib.lt_topk_workspace_bytes(1, 262144, 512)


LT_MAX_SPLIT_BLOCKS = 4194304
LT_MAX_SPLIT_SLOTS = 8388608
STREAM_ROW_MAX = 536866816


def test_header_split_limits():
    text = open(HEADERS[0]).read()
    assert "#define LT_MAX_SPLIT_BLOCKS %d" % LT_MAX_SPLIT_BLOCKS in text
    assert "#define LT_MAX_SPLIT_SLOTS %d" % LT_MAX_SPLIT_SLOTS in text


@pytest.mark.parametrize("bs,n_max,ok", [
    (1, LT_MAX_SPLIT_BLOCKS, True), (1, LT_MAX_SPLIT_BLOCKS + 1, False),
    (2, 2 * LT_MAX_SPLIT_BLOCKS, True), (2, 2 * LT_MAX_SPLIT_BLOCKS + 1, False),
    (8, 2 ** 31 - 4, True),          # block size 8 streams: no split limit
    (16, 16 * LT_MAX_SPLIT_BLOCKS + 1, False),
])
def test_blocks_split_limit(lib, bs, n_max, ok):
    """Rejected on the host before any launch; B = 0 so an accepted call is a no-op."""
    stride = n_max + (-n_max) % 4
    rc = lib.lt_topk_blocks(ALIGNED, stride, ALIGNED, 0, n_max, bs, 16, ALIGNED, None, 0, None)
    assert rc == (LT_OK if ok else LT_EINVAL)


@pytest.mark.parametrize("n_blocks,bs,n_max,ok", [
    (LT_MAX_SPLIT_SLOTS, 1, 4096, True), (LT_MAX_SPLIT_SLOTS + 1, 1, 4096, False),
    (LT_MAX_SPLIT_SLOTS // 4, 4, 4096, True), (LT_MAX_SPLIT_SLOTS // 4 + 1, 4, 4096, False),
    (LT_MAX_SPLIT_SLOTS, 8, 4096, True),                     # block size 8 streams
    (LT_MAX_SPLIT_SLOTS // 8 + 1, 8, STREAM_ROW_MAX, True),
    (LT_MAX_SPLIT_SLOTS // 8 + 1, 8, STREAM_ROW_MAX + 4, False),  # row too long to stream
])
def test_candidate_split_limit(lib, n_blocks, bs, n_max, ok):
    c = _Cand(ALIGNED, n_blocks, bs)
    rc = lib.lt_topk_run(ALIGNED, n_max, ALIGNED, 0, n_max, 16, ctypes.byref(c), ALIGNED, None, 0,
                         None)
    assert rc == (LT_OK if ok else LT_EINVAL)


# A fake "device" pointer: validation must reject before dereferencing anything.
ALIGNED = 1 << 20


class _Cand(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_void_p), ("n_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32)]


@pytest.mark.parametrize("args", [
    dict(scores=None),
    dict(lengths=None),
    dict(out=None),
    dict(B=-1),
    dict(n_max=-1),
    dict(k=0),
    dict(k=4097),
    dict(row_stride=100, n_max=101),
    dict(row_stride=102, n_max=100),
    dict(scores=ALIGNED + 4),
    dict(cand=_Cand(None, 4, 8)),
    dict(cand=_Cand(ALIGNED, 0, 8)),
    dict(cand=_Cand(ALIGNED, 4, 0)),
    dict(ws=ALIGNED + 8),
])
def test_run_rejects_invalid_arguments(lib, args):
    a = dict(scores=ALIGNED, row_stride=128, lengths=ALIGNED, B=1, n_max=128, k=16, cand=None,
             out=ALIGNED, ws=None, ws_bytes=0)
    a.update(args)
    cand = ctypes.byref(a["cand"]) if a["cand"] is not None else None
    rc = lib.lt_topk_run(a["scores"], a["row_stride"], a["lengths"], a["B"], a["n_max"], a["k"],
                         cand, a["out"], a["ws"], a["ws_bytes"], None)
    assert rc == LT_EINVAL


@pytest.mark.parametrize("args", [
    dict(scores=None), dict(out=None), dict(B=-3), dict(bs=0), dict(kb=0), dict(kb=5000),
    dict(row_stride=126), dict(scores=ALIGNED + 8),
])
def test_blocks_rejects_invalid_arguments(lib, args):
    a = dict(scores=ALIGNED, row_stride=128, lengths=ALIGNED, B=1, n_max=128, bs=8, kb=16,
             out=ALIGNED)
    a.update(args)
    rc = lib.lt_topk_blocks(a["scores"], a["row_stride"], a["lengths"], a["B"], a["n_max"], a["bs"],
                            a["kb"], a["out"], None, 0, None)
    assert rc == LT_EINVAL


@pytest.mark.parametrize("args", [
    dict(scores=None), dict(lengths=None), dict(blocks=None), dict(out=None), dict(B=-3),
    dict(bs=0), dict(kb=0), dict(kb=5000), dict(k=0), dict(k=4097), dict(row_stride=126),
    dict(scores=ALIGNED + 8), dict(ws=ALIGNED + 8),
    # a block stage past LT_MAX_SPLIT_BLOCKS blocks with a block size other than 8
    dict(bs=3, kb=4096, n_max=2 ** 31 - 4, row_stride=2 ** 31),
])
def test_two_stage_rejects_invalid_arguments(lib, args):
    a = dict(scores=ALIGNED, row_stride=128, lengths=ALIGNED, B=1, n_max=128, bs=8, kb=16, k=4,
             blocks=ALIGNED, out=ALIGNED, ws=None)
    a.update(args)
    rc = lib.lt_topk_two_stage(a["scores"], a["row_stride"], a["lengths"], a["B"], a["n_max"],
                               a["bs"], a["kb"], a["k"], a["blocks"], a["out"], a["ws"], 0, None)
    assert rc == LT_EINVAL


@pytest.mark.parametrize("args", [
    dict(idx=None), dict(B=-1), dict(n_max=-1), dict(k=0), dict(k=4097), dict(order=3),
    dict(order=-1), dict(order=2, scores=None), dict(vals=ALIGNED, scores=None),
    dict(order=2, row_stride=10, n_max=11), dict(order=0, vals=ALIGNED, row_stride=3, n_max=4),
])
def test_order_rejects_invalid_arguments(lib, args):
    a = dict(scores=ALIGNED, row_stride=128, B=2, n_max=128, k=16, order=1, idx=ALIGNED,
             vals=None)
    a.update(args)
    rc = lib.lt_topk_order(a["scores"], a["row_stride"], a["B"], a["n_max"], a["k"], a["order"],
                           a["idx"], a["vals"], None)
    assert rc == LT_EINVAL


@pytest.mark.parametrize("args", [
    dict(kv=None), dict(idx=None), dict(out=None), dict(B=-1), dict(k=0), dict(k=4097),
    dict(n_kv=-1), dict(row_bytes=8), dict(row_bytes=24), dict(row_bytes=(1 << 20) + 16),
    dict(kv_stride=16), dict(kv_stride=40), dict(kv_batch_stride=-16), dict(kv_batch_stride=8),
    dict(kv=ALIGNED + 8), dict(out=ALIGNED + 4),
])
def test_gather_rejects_invalid_arguments(lib, args):
    a = dict(kv=ALIGNED, kv_stride=64, kv_batch_stride=0, n_kv=100, row_bytes=32, idx=ALIGNED,
             B=2, k=16, out=ALIGNED)
    a.update(args)
    rc = lib.lt_gather_rows(a["kv"], a["kv_stride"], a["kv_batch_stride"], a["n_kv"],
                            a["row_bytes"], a["idx"], a["B"], a["k"], a["out"], None)
    assert rc == LT_EINVAL


def test_output_calls_with_nothing_to_do(lib):
    assert lib.lt_topk_order(ALIGNED, 128, 0, 128, 16, 2, ALIGNED, None, None) == LT_OK  # B = 0
    assert lib.lt_topk_order(None, 0, 4, 128, 16, 0, ALIGNED, None, None) == LT_OK   # as-is, no values
    assert lib.lt_gather_rows(ALIGNED, 64, 0, 100, 32, ALIGNED, 0, 16, ALIGNED, None) == LT_OK


def test_empty_batch_is_a_no_op(lib):
    assert lib.lt_topk_run(ALIGNED, 128, ALIGNED, 0, 128, 16, None, ALIGNED, None, 0, None) == LT_OK
    assert lib.lt_topk_blocks(ALIGNED, 128, ALIGNED, 0, 128, 8, 16, ALIGNED, None, 0, None) == LT_OK
    assert lib.lt_topk_two_stage(ALIGNED, 128, ALIGNED, 0, 128, 8, 16, 4, ALIGNED, ALIGNED, None, 0,
                                 None) == LT_OK


def test_binding_refuses_cpu_tensors():
    import torch
    import topk_index_selection_amd as ltk
    with pytest.raises(TypeError):
        ltk.lt_topk_run(torch.zeros(1, 8), torch.zeros(1, dtype=torch.int32), 4)
