"""Pin of the oracle's batch entry points when rows are split across threads.

The batch calls (``oracle.topk`` / ``oracle.topk_blocks`` with ``nthreads``)
give each thread a contiguous range of rows. The selection of a row does not
depend on which thread computes it, so every thread count must reproduce the
single-thread output exactly, element by element (the oracle writes its
selection in selection order, so even the slot order must agree). The
single-thread path is itself pinned by the brute-force, closed-form and
library-reduction tests; this ties the threaded path to it.

The cases cover the plain, block and candidate variants, batch sizes that the
thread count does not divide, and thread counts above the batch size.
"""
import numpy as np
import pytest

import oracle
import workloads

THREADS = [2, 3, 7, 16, 64]


def _batch(B, n, seed):
    """Rows of mixed shape: normal scores, bf16 ties, -inf runs, ragged lengths."""
    rng = np.random.default_rng(seed)
    s = np.empty((B, n), np.float32)
    for r in range(B):
        row = workloads.normal_row(90 + seed, r, n)
        if r % 3 == 1:
            row = workloads.round_to_bf16(row)
        if r % 5 == 2:
            row[rng.choice(n, n // 2, replace=False)] = -np.inf
        s[r] = row
    lengths = rng.integers(0, n + 1, size=B).astype(np.int32)
    lengths[0] = n
    if B > 1:
        lengths[1] = min(n, 300)
    return s, lengths


@pytest.mark.parametrize("B", [1, 5, 13, 37])
@pytest.mark.parametrize("nt", THREADS)
def test_plain_rows_thread_split(B, nt):
    s, lengths = _batch(B, 3000, 1)
    want = oracle.topk(s, lengths, 512, nthreads=1)
    got = oracle.topk(s, lengths, 512, nthreads=nt)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("B", [1, 5, 13, 37])
@pytest.mark.parametrize("nt", THREADS)
def test_block_rows_thread_split(B, nt):
    s, lengths = _batch(B, 4000, 2)
    want = oracle.topk_blocks(s, lengths, 8, 100, nthreads=1)
    got = oracle.topk_blocks(s, lengths, 8, 100, nthreads=nt)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("B", [1, 5, 13, 37])
@pytest.mark.parametrize("nt", THREADS)
def test_candidate_rows_thread_split(B, nt):
    s, lengths = _batch(B, 4000, 3)
    blocks = oracle.topk_blocks(np.roll(s, 1, axis=0), np.roll(lengths, 1), 8, 120, nthreads=1)
    want = oracle.topk(s, lengths, 64, cand=blocks, bs=8, nthreads=1)
    got = oracle.topk(s, lengths, 64, cand=blocks, bs=8, nthreads=nt)
    assert np.array_equal(got, want)


def test_each_row_equals_the_single_row_call():
    """The batch call (any thread count) agrees with the one-row entry point."""
    s, lengths = _batch(11, 2500, 4)
    got = oracle.topk(s, lengths, 300, nthreads=4)
    for r in range(s.shape[0]):
        assert np.array_equal(got[r], oracle.topk_row(s[r], int(lengths[r]), 300))


def test_strided_rows_thread_split():
    """Rows read through a row stride larger than the row (a column slice)."""
    s, lengths = _batch(9, 3000, 5)
    view = s[:, :2000]
    lengths = np.minimum(lengths, 2000).astype(np.int32)
    want = oracle.topk(np.ascontiguousarray(view), lengths, 256, nthreads=1)
    for nt in (1, 4, 9, 20):
        assert np.array_equal(oracle.topk(view, lengths, 256, nthreads=nt), want)
