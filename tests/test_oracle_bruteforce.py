"""Pins of the CPU oracle against brute-force rank counting.

Exhaustive over every row of length 6 drawn from the seven-value alphabet
{NaN, -inf, -1, -0.0, +0.0, 1, +inf} (117,649 rows), for every k in [1, 7] and
every valid length in [0, 6]; the oracle's output must equal, slot by slot,
the brute-force ordering (so both the selected set and the selection order are
checked). Then random tie-heavy rows up to n = 64 with and without candidate
blocks.
"""
import itertools

import numpy as np
import pytest

import oracle
from tests import bruteforce as bf

ALPHABET = np.array([np.nan, -np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], dtype=np.float32)


@pytest.fixture(scope="module")
def alphabet_rows():
    n = 6
    idx = np.array(list(itertools.product(range(len(ALPHABET)), repeat=n)), dtype=np.int64)
    return ALPHABET[idx]            # [7**6, 6] float32


@pytest.mark.parametrize("length", range(0, 7))
def test_exhaustive_alphabet(alphabet_rows, length):
    rows = alphabet_rows
    R, n = rows.shape
    valid = np.zeros((R, n), dtype=bool)
    valid[:, :length] = True
    for k in range(1, 8):
        got = oracle.topk(rows, np.full(R, length, np.int32), k)
        want = bf.ordered(rows.astype(np.float64), valid, k)
        assert np.array_equal(got.astype(np.int64), want), (length, k)


def test_random_tie_heavy_rows():
    rng = np.random.default_rng(12345)
    vals = np.array([-1.5, 0.0, 2.25], dtype=np.float32)
    for n in (1, 2, 7, 31, 64):
        rows = vals[rng.integers(0, 3, size=(400, n))]
        lens = rng.integers(0, n + 1, size=400).astype(np.int32)
        valid = np.arange(n)[None, :] < lens[:, None]
        for k in (1, 3, n, n + 5):
            got = oracle.topk(rows, lens, k)
            want = bf.ordered(rows.astype(np.float64), valid, k)
            assert np.array_equal(got.astype(np.int64), want), (n, k)


def test_random_rows_with_special_values():
    rng = np.random.default_rng(7)
    specials = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, 1e-45, -1e-45, 1e-38],
                        dtype=np.float32)
    for n in (5, 17, 48):
        rows = rng.standard_normal((300, n)).astype(np.float32)
        mask = rng.random((300, n)) < 0.3
        rows[mask] = specials[rng.integers(0, len(specials), size=mask.sum())]
        lens = rng.integers(0, n + 1, size=300).astype(np.int32)
        valid = np.arange(n)[None, :] < lens[:, None]
        for k in (1, 4, 16, 60):
            got = oracle.topk(rows, lens, k)
            want = bf.ordered(rows.astype(np.float64), valid, k)
            assert np.array_equal(got.astype(np.int64), want), (n, k)


def test_candidate_restriction_bruteforce():
    rng = np.random.default_rng(99)
    vals = np.array([-2.0, -0.0, 0.0, 0.5, 0.5, 3.0, np.nan, -np.inf], dtype=np.float32)
    for n, bs in ((16, 2), (24, 8), (40, 3), (9, 4)):
        nb = -(-n // bs)
        rows = vals[rng.integers(0, len(vals), size=(200, n))]
        lens = rng.integers(0, n + 1, size=200).astype(np.int32)
        n_cand = max(1, nb // 2)
        cand = np.empty((200, n_cand), np.int32)
        for r in range(200):
            ids = rng.permutation(nb + 2)[:n_cand] - 1   # includes -1 (empty) and an id past the end
            cand[r] = ids
        member = np.zeros((200, n), dtype=bool)
        for r in range(200):
            for b in cand[r]:
                if b >= 0:
                    member[r, b * bs:min(b * bs + bs, n)] = True
        valid = member & (np.arange(n)[None, :] < lens[:, None])
        for k in (1, 5, 12):
            got = oracle.topk(rows, lens, k, cand=cand, bs=bs)
            want = bf.ordered(rows.astype(np.float64), valid, k)
            assert np.array_equal(got.astype(np.int64), want), (n, bs, k)


def test_blocks_bruteforce():
    rng = np.random.default_rng(5)
    vals = np.array([np.nan, -np.inf, -1.0, -0.0, 0.0, 2.0, np.inf], dtype=np.float32)
    for n, bs in ((12, 3), (16, 8), (10, 4), (7, 1)):
        rows = vals[rng.integers(0, len(vals), size=(150, n))]
        lens = rng.integers(0, n + 1, size=150).astype(np.int32)
        bscore, bvalid = bf.block_scores(rows.astype(np.float64), lens, bs)
        for kb in (1, 2, 5):
            got = oracle.topk_blocks(rows, lens, bs, kb)
            want = bf.ordered(bscore, bvalid, kb)
            assert np.array_equal(got.astype(np.int64), want), (n, bs, kb)
