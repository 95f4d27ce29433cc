"""Brute-force selection by rank counting (independent of the oracle's sort).

Position i of a row is selected iff it is valid and fewer than k valid
positions come before it, where j comes before i when s_j ranks above s_i, or
the two scores tie and j < i. Ranking: real-number order, -0.0 equal to +0.0,
+inf highest, -inf lowest non-NaN, every NaN below -inf and NaNs tied.

Everything is vectorised over many rows at once: O(n^2) per row, so only for
short rows.
"""
from __future__ import annotations

import numpy as np


def ranks(rows: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """rank[r, i] = number of valid j that come before i in row r (int64).

    rows: [R, n] float; valid: [R, n] bool. Ranks of invalid positions are
    meaningless.
    """
    a = rows[:, :, None]          # s_j along axis 1
    b = rows[:, None, :]          # s_i along axis 2
    a_nan = np.isnan(a)
    b_nan = np.isnan(b)
    with np.errstate(invalid="ignore"):
        above = (~a_nan) & (b_nan | (a > b))
        tie = (a_nan & b_nan) | (a == b)
    n = rows.shape[1]
    j_lt_i = np.arange(n)[:, None] < np.arange(n)[None, :]
    before = above | (tie & j_lt_i[None, :, :])
    before &= valid[:, :, None]
    return before.sum(axis=1)


def select(rows: np.ndarray, valid: np.ndarray, k: int):
    """Return (selected mask [R, n], rank [R, n])."""
    r = ranks(rows, valid)
    return valid & (r < k), r


def ordered(rows: np.ndarray, valid: np.ndarray, k: int) -> np.ndarray:
    """[R, k] indices in selection order, -1 padded (from ranks)."""
    sel, r = select(rows, valid, k)
    R, n = rows.shape
    out = np.full((R, k), -1, dtype=np.int64)
    rr, ii = np.nonzero(sel)
    out[rr, r[rr, ii]] = ii
    return out


def block_scores(rows: np.ndarray, length: np.ndarray, bs: int):
    """Per block: the score of the block's best valid position (NaN lowest).

    Returns (scores [R, nb], valid [R, nb]) with nb = ceil(n / bs). Computed
    with an explicit scan, independent of the oracle.
    """
    R, n = rows.shape
    nb = -(-n // bs)
    out = np.full((R, nb), np.nan, dtype=rows.dtype)
    valid = np.zeros((R, nb), dtype=bool)
    for r in range(R):
        L = int(length[r])
        for b in range(nb):
            best = None
            for i in range(b * bs, min(b * bs + bs, L)):
                v = rows[r, i]
                if best is None:
                    best = v
                elif np.isnan(best) and not np.isnan(v):
                    best = v
                elif not np.isnan(v) and v > best:
                    best = v
            if best is not None:
                out[r, b] = best
                valid[r, b] = True
    return out, valid
