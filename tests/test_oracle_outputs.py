"""Pins for the output-variant oracle (oracle/outputs.py), on the CPU.

Selection order is checked against two things that do not share its code:
the C oracle, whose top-k rows come out already in selection order (it sorts
with its own comparator), and a brute-force pairwise rank. Ascending order,
values and the row gather are checked against their definitions written as
loops. Planted mistakes (a wrong tie rule, a reversed order, a shifted slot, a
shifted row) must each be caught by the checkers.
"""
import numpy as np
import pytest

import oracle
from oracle import outputs

ALPHABET = np.array([np.nan, -np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], np.float32)


def precedes(a_s, a_i, b_s, b_i):
    """a comes before b in selection order (pairwise definition)."""
    an, bn = np.isnan(a_s), np.isnan(b_s)
    if an != bn:
        return bn                      # a non-NaN before any NaN
    if not an and a_s != b_s:          # -0.0 == +0.0 here
        return a_s > b_s
    return a_i < b_i


def check_rank(scores, idx_in, out, n_max):
    """out[r] lists idx_in[r]'s valid entries in selection order, then -1."""
    for r in range(idx_in.shape[0]):
        ids = [int(i) for i in idx_in[r] if 0 <= i < n_max]
        got = [int(i) for i in out[r]]
        m = len(ids)
        if sorted(got[:m]) != sorted(ids) or any(g != -1 for g in got[m:]):
            return False
        s = scores[r]
        for p, i in enumerate(got[:m]):
            before = sum(precedes(s[j], j, s[i], i) for j in ids if j != i)
            if before != p:
                return False
    return True


def check_index(idx_in, out, n_max):
    for r in range(idx_in.shape[0]):
        ids = sorted(int(i) for i in idx_in[r] if 0 <= i < n_max)
        got = [int(i) for i in out[r]]
        if got[:len(ids)] != ids or any(g != -1 for g in got[len(ids):]):
            return False
    return True


def check_values(scores, idx, vals, n_max):
    for r in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            i = int(idx[r, j])
            want = scores[r, i] if 0 <= i < n_max else -np.inf
            if not (np.isnan(want) and np.isnan(vals[r, j])) and vals[r, j] != want:
                return False
            if want == 0 and np.signbit(want) != np.signbit(vals[r, j]):
                return False
    return True


def check_gather(kv, idx, out, n_kv, per_row):
    for r in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            i = int(idx[r, j])
            src = kv[r] if per_row else kv
            want = src[i] if 0 <= i < n_kv else np.zeros(kv.shape[-1], kv.dtype)
            if want.tobytes() != out[r, j].tobytes():
                return False
    return True


def tie_rows(B, n, seed):
    rng = np.random.default_rng(seed)
    return ALPHABET[rng.integers(0, len(ALPHABET), (B, n))].astype(np.float32)


def random_slots(B, k, n, seed, pad=True):
    """Rows of k slots: distinct ids in [0, n) (some out of range), -1 padding."""
    rng = np.random.default_rng(seed)
    out = np.full((B, k), -1, np.int32)
    for r in range(B):
        m = rng.integers(0, k + 1) if pad else k
        ids = rng.permutation(n + 3)[:m] - 1            # includes -1 and n, n+1
        out[r, :m] = ids
    return out


@pytest.mark.parametrize("seed", range(4))
def test_rank_order_reproduces_the_c_oracle(seed):
    """The C oracle emits a row's top-k in selection order; the numpy ordering
    of the same set (shuffled) must give the identical sequence."""
    B, n, k = 40, 37, 16
    s = tie_rows(B, n, seed)
    lens = np.random.default_rng(seed + 100).integers(0, n + 1, B).astype(np.int32)
    top = oracle.topk(s, lens, k)
    rng = np.random.default_rng(seed + 200)
    shuffled = np.stack([rng.permutation(row) for row in top])
    got = outputs.order(s, shuffled, outputs.ORDER_RANK, n)
    np.testing.assert_array_equal(got, top)


@pytest.mark.parametrize("seed", range(6))
def test_rank_order_brute_force(seed):
    B, n, k = 30, 12, 9
    s = tie_rows(B, n, seed)
    idx = random_slots(B, k, n, seed)
    got = outputs.order(s, idx, outputs.ORDER_RANK, n)
    assert check_rank(s, idx, got, n)


def test_rank_order_on_distinct_scores_is_argsort():
    rng = np.random.default_rng(5)
    s = rng.permutation(1000).astype(np.float32)[None, :] - 500.0
    idx = rng.permutation(1000)[:300].astype(np.int32)[None, :]
    got = outputs.order(s, idx, outputs.ORDER_RANK, 1000)[0]
    want = idx[0][np.argsort(-s[0, idx[0]])]
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("seed", range(4))
def test_index_order(seed):
    idx = random_slots(25, 33, 50, seed)
    got = outputs.order(np.zeros((25, 50), np.float32), idx, outputs.ORDER_INDEX, 50)
    assert check_index(idx, got, 50)


def test_asis_returns_the_slots_unchanged():
    idx = random_slots(5, 9, 20, 1)
    np.testing.assert_array_equal(outputs.order(None, idx, outputs.ORDER_ASIS, 20), idx)


@pytest.mark.parametrize("seed", range(3))
def test_values(seed):
    s = tie_rows(20, 15, seed)
    idx = random_slots(20, 11, 15, seed + 7)
    assert check_values(s, idx, outputs.values(s, idx, 15), 15)
    # in selection order the values never increase (NaN last)
    ranked = outputs.order(s, idx, outputs.ORDER_RANK, 15)
    v = outputs.values(s, ranked, 15)
    for r in range(v.shape[0]):
        m = int(np.sum(ranked[r] >= 0))
        vr = v[r, :m]
        fin = vr[~np.isnan(vr)]
        assert np.all(fin[:-1] >= fin[1:])
        assert not np.any(np.isnan(vr[:len(fin)]))


@pytest.mark.parametrize("per_row", [False, True])
def test_gather_rows(per_row):
    rng = np.random.default_rng(3)
    n_kv, D, B, k = 40, 24, 6, 10
    kv = rng.integers(0, 1 << 16, (B, n_kv, D) if per_row else (n_kv, D)).astype(np.uint16)
    idx = random_slots(B, k, n_kv, 9)
    out = outputs.gather_rows(kv, idx, n_kv, per_row)
    assert out.shape == (B, k, D) and out.dtype == kv.dtype
    assert check_gather(kv, idx, out, n_kv, per_row)


def test_checkers_catch_planted_mistakes():
    s = tie_rows(30, 12, 11)
    idx = random_slots(30, 9, 12, 12)
    good = outputs.order(s, idx, outputs.ORDER_RANK, 12)
    assert check_rank(s, idx, good, 12)
    # ties to the higher index
    bad = good.copy()
    for r in range(bad.shape[0]):
        m = int(np.sum(bad[r] >= 0))
        ids = bad[r, :m]
        sc = s[r, ids].astype(np.float64)
        key = np.where(np.isnan(sc), np.inf, -sc) + 0.0
        bad[r, :m] = ids[np.lexsort((-ids, key))]
    assert not np.array_equal(bad, good) and not check_rank(s, idx, bad, 12)
    # reversed order
    rev = good.copy()
    for r in range(rev.shape[0]):
        m = int(np.sum(rev[r] >= 0))
        rev[r, :m] = rev[r, :m][::-1]
    assert not check_rank(s, idx, rev, 12)
    # ascending order that leaves out the last valid id
    asc = outputs.order(s, idx, outputs.ORDER_INDEX, 12)
    short = asc.copy()
    for r in range(short.shape[0]):
        m = int(np.sum(short[r] >= 0))
        if m:
            short[r, m - 1] = -1
    assert check_index(idx, asc, 12) and not check_index(idx, short, 12)
    # values one slot off
    v = outputs.values(s, idx, 12)
    assert not check_values(s, idx, np.roll(v, 1, axis=1), 12)
    # gather of the next row
    kv = np.arange(13 * 4, dtype=np.int32).reshape(13, 4)
    g = outputs.gather_rows(kv, np.clip(idx + 1, -1, 12), 12)
    assert not check_gather(kv, idx, g, 12, False)
