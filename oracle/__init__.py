"""CPU oracle for CSA indexer top-k index selection -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package. The product path (``topk_index_selection_amd``) never
imports, links or calls it, and the two share no code.

The arithmetic lives in ``ltopk_oracle.c`` (plain C, built with gcc, no
``-ffast-math``); this module only builds and loads it and marshals numpy
arrays. See the C file's header for the definition it implements and the
passages of the pages it follows:

* "SGLang 与 Miles 为 DeepSeek-V4.1 提供首日支持" (xhh.club), Q&A on cross-layer
  sharing: index-source layers keep at most 512 compressed positions; the
  candidate layer publishes at most 2048 blocks of eight positions and later
  layers restrict their top-512 to them.
* AICon 2026 Shenzhen speaker page (aicon.infoq.cn), abstract and outline 一.1:
  CSA = 4:1 KV compression plus top-k sparse selection.

Readings the pages leave open (tie rule, NaN/+-0 order, short rows, how a block
is scored) are stated in the C header and listed in the design doc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ltopk_oracle.c")
_LIB = os.path.join(_HERE, "libltopk_oracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle into ``oracle/libltopk_oracle.so`` with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-std=c11", "-D_GNU_SOURCE", "-fPIC",
               "-shared", "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.lt_oracle_topk.argtypes = [f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                       i32p, ctypes.c_int32, ctypes.c_int32, i32p]
        lib.lt_oracle_topk.restype = ctypes.c_int
        lib.lt_oracle_blocks.argtypes = [f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, i32p]
        lib.lt_oracle_blocks.restype = ctypes.c_int
        lib.lt_oracle_topk_batch.argtypes = [f32p, ctypes.c_int64, i32p, ctypes.c_int32,
                                             ctypes.c_int64, ctypes.c_int32, i32p, ctypes.c_int32,
                                             ctypes.c_int32, i32p, ctypes.c_int]
        lib.lt_oracle_topk_batch.restype = ctypes.c_int
        lib.lt_oracle_blocks_batch.argtypes = [f32p, ctypes.c_int64, i32p, ctypes.c_int32,
                                               ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                               i32p, ctypes.c_int]
        lib.lt_oracle_blocks_batch.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _i32(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _rows(scores: np.ndarray):
    scores = np.asarray(scores)
    if scores.dtype != np.float32:
        raise TypeError("scores must be float32")
    if scores.ndim == 1:
        scores = scores[None, :]
    if scores.ndim != 2 or scores.strides[1] != 4:
        raise ValueError("scores must be [B, n_max] with unit column stride")
    return scores


def topk(scores: np.ndarray, lengths, k: int, cand: Optional[np.ndarray] = None,
         bs: int = 1, nthreads: int = 1) -> np.ndarray:
    """Top-k indices per row: [B, k] int32, selection order, -1 padded.

    ``cand`` (optional) is [B, n_cand] int32 block ids of ``bs`` positions each.
    """
    lib = _load()
    s = _rows(scores)
    B, n_max = s.shape
    row_stride = s.strides[0] // 4 if B > 1 else n_max
    lens = np.ascontiguousarray(np.broadcast_to(np.asarray(lengths, dtype=np.int32), (B,)))
    out = np.empty((B, k), dtype=np.int32)
    if cand is not None:
        c = np.ascontiguousarray(np.asarray(cand, dtype=np.int32).reshape(B, -1))
        n_cand = c.shape[1]
        cptr = _i32(c)
    else:
        c = None
        n_cand = 0
        cptr = None
    rc = lib.lt_oracle_topk_batch(_f32(s), row_stride, _i32(lens), B, n_max, k, cptr, n_cand,
                                  bs, _i32(out), int(nthreads))
    if rc != 0:
        raise ValueError("lt_oracle_topk_batch rejected its arguments")
    return out


def topk_blocks(scores: np.ndarray, lengths, bs: int, kb: int, nthreads: int = 1) -> np.ndarray:
    """Top-kb block ids per row: [B, kb] int32, selection order, -1 padded."""
    lib = _load()
    s = _rows(scores)
    B, n_max = s.shape
    row_stride = s.strides[0] // 4 if B > 1 else n_max
    lens = np.ascontiguousarray(np.broadcast_to(np.asarray(lengths, dtype=np.int32), (B,)))
    out = np.empty((B, kb), dtype=np.int32)
    rc = lib.lt_oracle_blocks_batch(_f32(s), row_stride, _i32(lens), B, n_max, bs, kb, _i32(out),
                                    int(nthreads))
    if rc != 0:
        raise ValueError("lt_oracle_blocks_batch rejected its arguments")
    return out


def topk_row(row: np.ndarray, length: int, k: int, cand: Optional[np.ndarray] = None,
             bs: int = 1) -> np.ndarray:
    """One row (the single-row entry point, no threads)."""
    lib = _load()
    r = np.ascontiguousarray(row, dtype=np.float32)
    out = np.empty(k, dtype=np.int32)
    if cand is not None:
        c = np.ascontiguousarray(cand, dtype=np.int32)
        rc = lib.lt_oracle_topk(_f32(r), r.shape[0], int(length), k, _i32(c), c.shape[0], bs,
                                _i32(out))
    else:
        rc = lib.lt_oracle_topk(_f32(r), r.shape[0], int(length), k, None, 0, 1, _i32(out))
    if rc != 0:
        raise ValueError("lt_oracle_topk rejected its arguments")
    return out
