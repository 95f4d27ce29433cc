"""Output variants of a selection -- TEST INFRASTRUCTURE ONLY (plain numpy).

Only the tests and the benchmark's checks import this module; the product path
never does, and it shares no code with the HIP library.

What a selection feeds is CSA's sparse attention over the selected compressed
positions (AICon 2026 Shenzhen speaker page, aicon.infoq.cn: abstract and
outline 一.1, CSA = 4:1 KV compression plus top-k selection). The pages give no
layout for what the consumer receives, so the variants take the plainest
reading of "indices, possibly ordered, possibly with their scores, possibly as
the selected cache rows themselves":

* ``order_index``: a row's selected indices in ascending order, empty slots
  (-1) after them;
* ``order_rank``: the selected indices in selection order -- higher score
  first, equal scores lower index first, -0.0 equal to +0.0, every NaN below
  -inf (the same total order the selection itself uses);
* ``values``: the score at each slot's index, -inf in empty slots;
* ``gather_rows``: the cache row of each slot's index, zero bytes in empty
  slots.

An index outside [0, n) counts as an empty slot. Repeated indices are kept as
they are (a selection never repeats one).
"""
from __future__ import annotations

import numpy as np

ORDER_ASIS, ORDER_INDEX, ORDER_RANK = 0, 1, 2


def _valid(row: np.ndarray, n: int) -> np.ndarray:
    return row[(row >= 0) & (row < n)]


def order(scores: np.ndarray, idx: np.ndarray, how: int, n_max: int) -> np.ndarray:
    """Reordered copy of idx [B, k] (ORDER_ASIS returns it unchanged)."""
    idx = np.asarray(idx, np.int32)
    if how == ORDER_ASIS:
        return idx.copy()
    out = np.full_like(idx, -1)
    for r in range(idx.shape[0]):
        sel = _valid(idx[r], n_max)
        if how == ORDER_INDEX:
            sel = np.sort(sel, kind="stable")
        elif how == ORDER_RANK:
            s = scores[r, sel].astype(np.float64)
            nan = np.isnan(s)
            # ascending -s is descending s; adding +0.0 makes -0.0 and +0.0 one value
            neg = np.where(nan, 0.0, -s) + 0.0
            # lexsort: last key first -- non-NaN before NaN, then -s, then index
            sel = sel[np.lexsort((sel, neg, nan))]
        else:
            raise ValueError("unknown order %r" % how)
        out[r, :len(sel)] = sel
    return out


def values(scores: np.ndarray, idx: np.ndarray, n_max: int) -> np.ndarray:
    """scores[r, idx[r, j]] per slot, -inf where the slot is empty."""
    idx = np.asarray(idx, np.int32)
    out = np.full(idx.shape, -np.inf, np.float32)
    for r in range(idx.shape[0]):
        ok = (idx[r] >= 0) & (idx[r] < n_max)
        out[r, ok] = scores[r, idx[r, ok]]
    return out


def gather_rows(kv: np.ndarray, idx: np.ndarray, n_kv: int, per_row: bool = False) -> np.ndarray:
    """Cache rows selected by idx [B, k]: out[r, j] = kv[idx[r, j]] (per_row:
    kv[r, idx[r, j]]), zero bytes where the slot is empty. kv is [n_kv, D] (or
    [B, n_kv, D]) of any dtype; the result is [B, k, D] of the same dtype."""
    idx = np.asarray(idx, np.int32)
    B, k = idx.shape
    D = kv.shape[-1]
    out = np.zeros((B, k, D), kv.dtype)
    for r in range(B):
        ok = (idx[r] >= 0) & (idx[r] < n_kv)
        src = kv[r] if per_row else kv
        out[r, ok] = src[idx[r, ok]]
    return out
