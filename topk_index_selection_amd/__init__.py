"""Python binding for ``libltopk.so``: CSA indexer top-k selection on MI355X.

The functions keep the C entry points' names (``lt_topk_run``,
``lt_topk_blocks``, ``lt_topk_workspace_bytes``, ``lt_topk_order``,
``lt_gather_rows``, ``lt_status_str``) and only marshal arguments: every step
runs in the HIP kernels of ``csrc/ltopk_kernels.hip`` (the selection) and
``csrc/ltopk_output.hip`` (its output variants). PyTorch supplies device memory (tensors) and the
stream (``torch.cuda.current_stream()``); there is no CPU fallback, and a
missing library is an error.

What is computed (see ``include/ltopk.h`` for the full contract): for each row,
the indices of the top-k scores among the row's valid positions, highest first,
lower index first among equal scores, at most k of them (k = 512 per
index-source layer, 2048 eight-position blocks for the shared-candidate layer:
"SGLang 与 Miles 为 DeepSeek-V4.1 提供首日支持", xhh.club, Q&A on cross-layer
sharing). Output slots [0, m) hold the selection in no particular order, the
rest -1.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libltopk.so")

LT_OK, LT_EINVAL, LT_ENOSPC, LT_EHIP = 0, 1, 2, 3
LT_K_MAX = 4096
LT_NOALLOC_SPLIT_ROWS = 64
LT_ORDER_ASIS, LT_ORDER_INDEX, LT_ORDER_RANK = 0, 1, 2

_lib = None
_lib_lock = threading.Lock()


class LtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, lt_status_str(status)))


class _Cand(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_void_p), ("n_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32)]


def load_library():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libltopk.so is not built (%s); run "
                                   "`python -m topk_index_selection_amd.build_lib`" % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            lib.lt_topk_workspace_bytes.argtypes = [i32, i32, i32]
            lib.lt_topk_workspace_bytes.restype = sz
            lib.lt_topk_run.argtypes = [vp, i64, vp, i32, i32, i32, ctypes.POINTER(_Cand), vp, vp,
                                        sz, vp]
            lib.lt_topk_run.restype = ctypes.c_int
            lib.lt_topk_run_noalloc.argtypes = [vp, i64, vp, i32, i32, i32, ctypes.POINTER(_Cand),
                                                vp, vp]
            lib.lt_topk_run_noalloc.restype = ctypes.c_int
            lib.lt_topk_blocks.argtypes = [vp, i64, vp, i32, i32, i32, i32, vp, vp, sz, vp]
            lib.lt_topk_blocks.restype = ctypes.c_int
            lib.lt_topk_two_stage.argtypes = [vp, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp,
                                              sz, vp]
            lib.lt_topk_two_stage.restype = ctypes.c_int
            lib.lt_topk_order.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp]
            lib.lt_topk_order.restype = ctypes.c_int
            lib.lt_gather_rows.argtypes = [vp, i64, i64, i64, i32, vp, i32, i32, vp, vp]
            lib.lt_gather_rows.restype = ctypes.c_int
            lib.lt_status_str.argtypes = [ctypes.c_int]
            lib.lt_status_str.restype = ctypes.c_char_p
            lib.lt_debug_force_path.argtypes = [ctypes.c_int]
            lib.lt_debug_force_path.restype = ctypes.c_int
            lib.lt_debug_force_fallback.argtypes = [ctypes.c_int]
            lib.lt_debug_force_fallback.restype = ctypes.c_int
            lib.lt_debug_force_sample.argtypes = [ctypes.c_int]
            lib.lt_debug_force_sample.restype = ctypes.c_int
            lib.lt_debug_empty_launch.argtypes = [i32, i32, i32, vp]
            lib.lt_debug_empty_launch.restype = ctypes.c_int
            pi = ctypes.POINTER(i32)
            lib.lt_debug_launch_shape.argtypes = [i32, i32, pi, pi, pi]
            lib.lt_debug_launch_shape.restype = ctypes.c_int
            _lib = lib
    return _lib


def lt_status_str(status: int) -> str:
    return load_library().lt_status_str(int(status)).decode()


def lt_topk_workspace_bytes(B: int, n_max: int, k: int) -> int:
    return int(load_library().lt_topk_workspace_bytes(int(B), int(n_max), int(k)))


# test hooks (include/ltopk_debug.h)

PATH_AUTO, PATH_SPLIT, PATH_STREAM, PATH_ROW = 0, 1, 2, 3


def lt_debug_force_path(path: int) -> int:
    return int(load_library().lt_debug_force_path(int(path)))


def lt_debug_force_fallback(on: bool) -> int:
    return int(load_library().lt_debug_force_fallback(1 if on else 0))


SAMPLE_AUTO, SAMPLE_NEVER, SAMPLE_ALWAYS = 0, 1, 2


def lt_debug_force_sample(mode: int) -> int:
    return int(load_library().lt_debug_force_sample(int(mode)))


def lt_debug_launch_shape(B: int, n_max: int):
    """(kernel, (grid_x, grid_y), block) of the first launch of lt_topk_run for
    B rows of n_max scores without candidates; kernel is "split", "stream" or
    "row"."""
    gx, gy, bl = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    r = load_library().lt_debug_launch_shape(int(B), int(n_max), ctypes.byref(gx),
                                             ctypes.byref(gy), ctypes.byref(bl))
    if r < 0:
        raise RuntimeError("lt_debug_launch_shape failed")
    return ("split", "stream", "row")[r], (gx.value, gy.value), bl.value


def lt_debug_empty_launch(grid_x: int, grid_y: int = 1, block: int = 256) -> None:
    """Empty kernel on the current stream (launch-floor measurements)."""
    stream = torch.cuda.current_stream()
    if load_library().lt_debug_empty_launch(int(grid_x), int(grid_y), int(block),
                                            stream.cuda_stream) != 0:
        raise RuntimeError("lt_debug_empty_launch failed")


# ------------------------------------------------------------------ workspace

_ws_cache: Dict[Tuple[int, int], torch.Tensor] = {}
_ws_lock = threading.Lock()


def workspace(nbytes: int, device: torch.device, stream: Optional[torch.cuda.Stream] = None):
    """A zero-filled workspace of at least ``nbytes`` for (device, stream).

    The kernels return it to zero after every call, so it is allocated and
    cleared once and then reused by every call on that stream.
    """
    if nbytes == 0:
        return None
    dev = torch.device(device)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), s.cuda_stream)
    with _ws_lock:
        t = _ws_cache.get(key)
        if t is None or t.numel() < nbytes:
            t = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
            _ws_cache[key] = t
        return t


def _check_scores(scores: torch.Tensor) -> Tuple[int, int, int]:
    if not isinstance(scores, torch.Tensor) or not scores.is_cuda:
        raise TypeError("scores must be a GPU tensor (no CPU path exists)")
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    if scores.dim() == 1:
        scores = scores.unsqueeze(0)
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be [B, n_max] with unit column stride")
    B, n_max = scores.shape
    row_stride = scores.stride(0) if B > 1 else max(n_max + (-n_max) % 4, 0)
    return B, n_max, row_stride


def _check_i32(t: torch.Tensor, name: str, numel: Optional[int] = None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32:
        raise TypeError("%s must be an int32 GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must have %d elements" % (name, numel))


def lt_topk_run(scores: torch.Tensor, lengths: torch.Tensor, k: int,
                cand: Optional[Tuple[torch.Tensor, int]] = None,
                out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k positions per row -> int32 [B, k] (slots past min(k, |V|) are -1).

    scores : float32 [B, n_max] (or [n_max]) on the GPU, unit column stride
    lengths: int32 [B] on the GPU
    cand   : optional (blocks int32 [B, n_blocks], block_size) restriction
    """
    lib = load_library()
    B, n_max, row_stride = _check_scores(scores)
    _check_i32(lengths, "lengths", B)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    _check_i32(out, "out", B * k)
    cptr = None
    ws_n = n_max
    if cand is not None:
        blocks, block_size = cand
        _check_i32(blocks, "cand blocks")
        if blocks.dim() != 2 or blocks.shape[0] != B:
            raise ValueError("cand blocks must be [B, n_blocks]")
        c = _Cand(blocks.data_ptr(), int(blocks.shape[1]), int(block_size))
        cptr = ctypes.byref(c)
        ws_n = max(n_max, int(blocks.shape[1]) * int(block_size))
    need = lt_topk_workspace_bytes(B, ws_n, k)
    stream = torch.cuda.current_stream(scores.device)
    if ws is None:
        ws = workspace(need, scores.device, stream)
    rc = lib.lt_topk_run(scores.data_ptr(), row_stride, lengths.data_ptr(), B, n_max, int(k), cptr,
                         out.data_ptr(), ws.data_ptr() if ws is not None else None,
                         ws.numel() if ws is not None else 0, stream.cuda_stream)
    if rc != LT_OK:
        raise LtError(rc, "lt_topk_run")
    return out


def lt_topk_run_noalloc(scores: torch.Tensor, lengths: torch.Tensor, k: int,
                        cand: Optional[Tuple[torch.Tensor, int]] = None,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lt_topk_run through the library's built-in workspace (no workspace
    argument, nothing allocated by the call). Split rows are limited to
    LT_NOALLOC_SPLIT_ROWS per call (LtError LT_ENOSPC beyond). Pass ``out``
    to allocate nothing at all."""
    lib = load_library()
    B, n_max, row_stride = _check_scores(scores)
    _check_i32(lengths, "lengths", B)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    _check_i32(out, "out", B * k)
    cptr = None
    if cand is not None:
        blocks, block_size = cand
        _check_i32(blocks, "cand blocks")
        if blocks.dim() != 2 or blocks.shape[0] != B:
            raise ValueError("cand blocks must be [B, n_blocks]")
        c = _Cand(blocks.data_ptr(), int(blocks.shape[1]), int(block_size))
        cptr = ctypes.byref(c)
    stream = torch.cuda.current_stream(scores.device)
    rc = lib.lt_topk_run_noalloc(scores.data_ptr(), row_stride, lengths.data_ptr(), B, n_max,
                                 int(k), cptr, out.data_ptr(), stream.cuda_stream)
    if rc != LT_OK:
        raise LtError(rc, "lt_topk_run_noalloc")
    return out


def lt_topk_blocks(scores: torch.Tensor, lengths: torch.Tensor, block_size: int, kb: int,
                   out: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-kb blocks of ``block_size`` positions per row, scored by their max -> int32 [B, kb]."""
    lib = load_library()
    B, n_max, row_stride = _check_scores(scores)
    _check_i32(lengths, "lengths", B)
    if out is None:
        out = torch.empty((B, kb), dtype=torch.int32, device=scores.device)
    _check_i32(out, "out", B * kb)
    need = lt_topk_workspace_bytes(B, n_max, kb)
    stream = torch.cuda.current_stream(scores.device)
    if ws is None:
        ws = workspace(need, scores.device, stream)
    rc = lib.lt_topk_blocks(scores.data_ptr(), row_stride, lengths.data_ptr(), B, n_max,
                            int(block_size), int(kb), out.data_ptr(),
                            ws.data_ptr() if ws is not None else None,
                            ws.numel() if ws is not None else 0, stream.cuda_stream)
    if rc != LT_OK:
        raise LtError(rc, "lt_topk_blocks")
    return out


def lt_topk_two_stage(scores: torch.Tensor, lengths: torch.Tensor, block_size: int, kb: int,
                      k: int, out_blocks: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Both stages of a shared-candidate layer: the top-kb blocks of ``block_size``
    positions (int32 [B, kb]) and the top-k positions inside them (int32 [B, k])."""
    lib = load_library()
    B, n_max, row_stride = _check_scores(scores)
    _check_i32(lengths, "lengths", B)
    if out_blocks is None:
        out_blocks = torch.empty((B, kb), dtype=torch.int32, device=scores.device)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    _check_i32(out_blocks, "out_blocks", B * kb)
    _check_i32(out, "out", B * k)
    need = lt_topk_workspace_bytes(B, n_max, k)
    stream = torch.cuda.current_stream(scores.device)
    if ws is None:
        ws = workspace(need, scores.device, stream)
    rc = lib.lt_topk_two_stage(scores.data_ptr(), row_stride, lengths.data_ptr(), B, n_max,
                               int(block_size), int(kb), int(k), out_blocks.data_ptr(),
                               out.data_ptr(), ws.data_ptr() if ws is not None else None,
                               ws.numel() if ws is not None else 0, stream.cuda_stream)
    if rc != LT_OK:
        raise LtError(rc, "lt_topk_two_stage")
    return out_blocks, out


def two_stage(scores: torch.Tensor, lengths: torch.Tensor, k: int = 512, kb: int = 2048,
              block_size: int = 8) -> Tuple[torch.Tensor, torch.Tensor]:
    """Shared-candidate selection: top-kb blocks, then top-k restricted to them."""
    return lt_topk_two_stage(scores, lengths, block_size, kb, k)


def lt_topk_order(idx: torch.Tensor, order: int, scores: Optional[torch.Tensor] = None,
                  vals: bool = False, out_vals: Optional[torch.Tensor] = None,
                  n_max: Optional[int] = None):
    """Reorder a selection's slots in place (LT_ORDER_ASIS / _INDEX / _RANK) and
    optionally return the score at each slot (-inf for empty slots).

    idx    : int32 [B, k] on the GPU, rewritten in place
    scores : float32 [B, n_max] the indices refer to (needed for LT_ORDER_RANK
             and for values)
    n_max  : indices at or above it count as empty (default: scores' width,
             or no limit without scores)
    Returns idx, or (idx, values float32 [B, k]) when vals is true.
    """
    lib = load_library()
    _check_i32(idx, "idx")
    if idx.dim() != 2:
        raise ValueError("idx must be [B, k]")
    B, k = idx.shape
    sptr, row_stride, width = None, 0, 2 ** 31 - 1
    if scores is not None:
        Bs, width, row_stride = _check_scores(scores)
        if Bs != B:
            raise ValueError("scores and idx must have the same rows")
        sptr = scores.data_ptr()
    if n_max is None:
        n_max = width
    elif scores is not None and n_max > width:
        raise ValueError("n_max exceeds the scores' width")
    if vals and out_vals is None:
        out_vals = torch.empty((B, k), dtype=torch.float32, device=idx.device)
    if out_vals is not None:
        if not out_vals.is_cuda or out_vals.dtype != torch.float32 or not out_vals.is_contiguous() \
                or out_vals.numel() != B * k:
            raise TypeError("out_vals must be a contiguous float32 GPU tensor of B*k elements")
    stream = torch.cuda.current_stream(idx.device)
    rc = lib.lt_topk_order(sptr, row_stride, B, n_max, k, int(order), idx.data_ptr(),
                           out_vals.data_ptr() if out_vals is not None else None,
                           stream.cuda_stream)
    if rc != LT_OK:
        raise LtError(rc, "lt_topk_order")
    return (idx, out_vals) if out_vals is not None else idx


def lt_gather_rows(kv: torch.Tensor, idx: torch.Tensor, per_row: bool = False,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The cache rows a selection names -> [B, k, *row] (zeros for empty slots).

    kv  : GPU tensor [n_kv, ...] shared by every row, or [B, n_kv, ...] with
          per_row; each cache row must be contiguous, 16-byte multiples
    idx : int32 [B, k] on the GPU
    """
    lib = load_library()
    _check_i32(idx, "idx")
    if idx.dim() != 2:
        raise ValueError("idx must be [B, k]")
    if not isinstance(kv, torch.Tensor) or not kv.is_cuda:
        raise TypeError("kv must be a GPU tensor")
    B, k = idx.shape
    lead = 2 if per_row else 1
    if kv.dim() < lead + 1:
        raise ValueError("kv must have a row dimension")
    if per_row and kv.shape[0] != B:
        raise ValueError("per-row kv must have B caches")
    row_shape = tuple(kv.shape[lead:])
    row_elems = 1
    for d in row_shape:
        row_elems *= d
    expect = 1
    for d in range(kv.dim() - 1, lead - 1, -1):
        if kv.shape[d] > 1 and kv.stride(d) != expect:
            raise ValueError("each cache row must be contiguous")
        expect *= kv.shape[d]
    es = kv.element_size()
    row_bytes = row_elems * es
    kv_stride = kv.stride(lead - 1) * es
    kv_batch_stride = kv.stride(0) * es if per_row else 0
    n_kv = kv.shape[lead - 1]
    if out is None:
        out = torch.empty((B, k) + row_shape, dtype=kv.dtype, device=kv.device)
    if not out.is_contiguous() or out.dtype != kv.dtype or out.numel() != B * k * row_elems:
        raise ValueError("out must be a contiguous [B, k, *row] tensor of kv's dtype")
    stream = torch.cuda.current_stream(kv.device)
    rc = lib.lt_gather_rows(kv.data_ptr(), kv_stride, kv_batch_stride, n_kv, row_bytes,
                            idx.data_ptr(), B, k, out.data_ptr(), stream.cuda_stream)
    if rc != LT_OK:
        raise LtError(rc, "lt_gather_rows")
    return out
