"""Pins of the CPU oracle against closed forms, library routines and invariants.

* Closed forms: all-equal, strictly increasing / decreasing, all -inf, k >= |V|,
  a permutation of 0..n-1.
* Library reductions: on NaN-free rows the selection is the first m of
  ``np.lexsort((index, -score))``; on distinct-valued rows it is the set that
  ``torch.topk`` returns.
* Invariants on every scaled-down workload: count, uniqueness, membership,
  score dominance, lowest-index ties at the threshold, -inf only when needed.
* Two-stage identity: with the same row for both stages and kb >= k, the top-k
  restricted to the top-kb blocks equals the unrestricted top-k.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def as_set(out_row):
    return np.sort(out_row[out_row >= 0])


# ------------------------------------------------------------------ closed forms

@pytest.mark.parametrize("n,k", [(1, 1), (10, 3), (1000, 512), (4096, 512), (600, 2048)])
def test_closed_forms(n, k):
    m = min(n, k)
    cases = {
        "equal": (np.full(n, 0.75, np.float32), np.arange(m)),
        "increasing": (np.arange(n, dtype=np.float32), np.arange(n - m, n)),
        "decreasing": (np.arange(n, 0, -1).astype(np.float32), np.arange(m)),
        "all_neg_inf": (np.full(n, -np.inf, np.float32), np.arange(m)),
        "all_pos_inf": (np.full(n, np.inf, np.float32), np.arange(m)),
        "signed_zeros": (np.where(np.arange(n) % 2 == 0, -0.0, 0.0).astype(np.float32),
                         np.arange(m)),
    }
    for name, (row, want) in cases.items():
        got = oracle.topk_row(row, n, k)
        assert np.array_equal(as_set(got), want), name
        assert np.all(got[m:] == -1), name


def test_permutation_closed_form():
    rng = np.random.default_rng(3)
    for n, k in ((100, 7), (5000, 512), (4096, 4096)):
        perm = rng.permutation(n).astype(np.float32)
        got = oracle.topk_row(perm, n, k)
        want = np.sort(np.nonzero(perm >= n - min(k, n))[0])
        assert np.array_equal(as_set(got), want)


def test_short_rows_return_all_valid():
    row = workloads.normal_row(77, 0, 1000)
    for L in (0, 1, 5, 511, 512):
        got = oracle.topk_row(row, L, 512)
        assert np.array_equal(as_set(got), np.arange(L))
        assert np.all(got[min(L, 512):] == -1)


def test_length_clamped():
    row = workloads.normal_row(77, 1, 64)
    row[-1] = 100.0     # the last valid position is the best, so a short clamp shows
    a = oracle.topk_row(row, 10**6, 16)
    b = oracle.topk_row(row, 64, 16)
    assert np.array_equal(a, b)
    assert a[0] == 63
    c = oracle.topk_row(row, -5, 16)
    assert np.all(c == -1)


# ---------------------------------------------------------- library reductions

def lexsort_topk(row, length, k):
    s = row[:length].astype(np.float64)
    order = np.lexsort((np.arange(length), -s))
    return order[:min(k, length)]


def test_lexsort_reduction_tie_heavy():
    rng = np.random.default_rng(11)
    for trial in range(40):
        n = int(rng.integers(1, 5000))
        row = workloads.round_to_bf16(rng.standard_normal(n).astype(np.float32) * 0.05)
        row[rng.random(n) < 0.05] = -np.inf
        row[rng.random(n) < 0.02] = np.inf
        row[rng.random(n) < 0.05] = -0.0
        length = int(rng.integers(0, n + 1))
        k = int(rng.integers(1, 700))
        got = oracle.topk_row(row, length, k)
        want = lexsort_topk(row, length, k)
        m = len(want)
        assert np.array_equal(got[:m], want)
        assert np.all(got[m:] == -1)


def test_torch_topk_on_distinct_rows():
    rng = np.random.default_rng(13)
    for n, k in ((4096, 512), (262144, 512), (32768, 2048), (777, 100)):
        row = rng.permutation(n).astype(np.float32) * np.float32(0.5) - np.float32(n / 4)
        got = oracle.topk_row(row, n, k)
        want = torch.topk(torch.from_numpy(row), k).indices.numpy()
        assert np.array_equal(as_set(got), np.sort(want))


# ------------------------------------------------------------------ invariants

def before(a_s, a_i, b_s, b_i):
    """Scalar selection order (used on the threshold element only)."""
    if np.isnan(a_s) != np.isnan(b_s):
        return np.isnan(b_s)
    if not np.isnan(a_s) and a_s != b_s:
        return a_s > b_s
    return a_i < b_i


def check_invariants(row, length, k, out, valid_mask=None):
    length = max(0, min(int(length), row.shape[0]))
    if valid_mask is None:
        valid = np.zeros(row.shape[0], dtype=bool)
        valid[:length] = True
    else:
        valid = valid_mask.copy()
        valid[length:] = False
    V = np.nonzero(valid)[0]
    m = min(k, len(V))
    # (i) count and padding
    assert np.all(out[:m] >= 0) and np.all(out[m:] == -1)
    sel = out[:m]
    # (ii) unique, inside V
    assert len(np.unique(sel)) == m
    assert np.all(valid[sel])
    if m == 0:
        return
    unsel = np.setdiff1d(V, sel)
    s = row.astype(np.float64)
    # key: NaN lowest, then real order (-0 == +0)
    def key(x):
        return np.where(np.isnan(x), -np.inf, x), np.isnan(x)
    sk, snan = key(s[sel])
    uk, unan = key(s[unsel])
    if len(unsel):
        # (iii) every selected score >= every unselected one
        worst_sel_nan = snan.any()
        if worst_sel_nan:
            assert unan.all()
        else:
            assert sk.min() >= uk[~unan].max(initial=-np.inf)
        # (iv) ties at the threshold go to the lowest indices
        t_pos = sel[0]
        for p in sel:
            if before(s[t_pos], t_pos, s[p], p):
                t_pos = p
        tie_unsel = unsel[(s[unsel] == s[t_pos]) | (np.isnan(s[unsel]) & np.isnan(s[t_pos]))]
        assert np.all(tie_unsel > t_pos)
    # (v) -inf only if fewer than k entries above -inf; NaN only if fewer than k non-NaN
    n_above_ninf = np.sum(~np.isnan(s[V]) & (s[V] > -np.inf))
    if np.any(s[sel] == -np.inf):
        assert n_above_ninf < k
    n_non_nan = np.sum(~np.isnan(s[V]))
    if np.any(np.isnan(s[sel])):
        assert n_non_nan < k


@pytest.mark.parametrize("w", workloads.small_variants(), ids=lambda w: w.name)
def test_invariants_on_scaled_workloads(w):
    if w.kb:
        blocks = oracle.topk_blocks(w.scores, w.lengths, w.bs, w.kb)
        out = oracle.topk(w.scores, w.lengths, w.k, cand=blocks, bs=w.bs)
        for r in range(w.B):
            member = np.zeros(w.n_max, dtype=bool)
            for b in blocks[r]:
                if b >= 0:
                    member[b * w.bs:(b + 1) * w.bs] = True
            check_invariants(w.scores[r], w.lengths[r], w.k, out[r], member)
    else:
        out = oracle.topk(w.scores, w.lengths, w.k)
        for r in range(w.B):
            check_invariants(w.scores[r], w.lengths[r], w.k, out[r])


def test_invariants_cfg3_full_size():
    for v in "abc":
        w = workloads.cfg3(v)
        out = oracle.topk(w.scores, w.lengths, w.k)
        check_invariants(w.scores[0], w.lengths[0], w.k, out[0])


def test_cfg3c_exact_counts():
    w = workloads.cfg3("c")
    assert int(np.sum(np.isinf(w.scores[0]))) == 235930
    out = oracle.topk(w.scores, w.lengths, 512)[0]
    assert not np.any(np.isinf(w.scores[0][out]))


def test_cfg3b_has_ties_at_threshold():
    """The bf16 variant really exercises the tie rule: ties straddle the cut."""
    w = workloads.cfg3("b")
    out = oracle.topk(w.scores, w.lengths, 512)[0]
    s = w.scores[0]
    t = s[out].min()
    n_gt = int(np.sum(s > t))
    n_eq = int(np.sum(s == t))
    assert n_gt < 512 < n_gt + n_eq
    taken = np.sort(out[s[out] == t])
    ties = np.nonzero(s == t)[0]
    assert np.array_equal(taken, ties[:512 - n_gt])


# --------------------------------------------------------- two-stage identity

@pytest.mark.parametrize("n,bs,kb,k", [(262144, 8, 2048, 512), (5000, 8, 64, 64),
                                        (1000, 3, 50, 20), (4096, 1, 600, 512)])
def test_two_stage_equals_single_stage_same_row(n, bs, kb, k):
    """Every block ranked above a selected position's block holds a selected
    position of its own, so a top-k position's block ranks <= k among blocks:
    with kb >= k, restricting to the top-kb blocks changes nothing."""
    rng = np.random.default_rng(n + bs)
    rows = np.stack([rng.standard_normal(n).astype(np.float32),
                     workloads.round_to_bf16(rng.standard_normal(n).astype(np.float32))])
    lens = np.array([n, n - 3], np.int32)
    blocks = oracle.topk_blocks(rows, lens, bs, kb)
    two = oracle.topk(rows, lens, k, cand=blocks, bs=bs)
    one = oracle.topk(rows, lens, k)
    for r in range(2):
        assert np.array_equal(np.sort(two[r]), np.sort(one[r]))


def test_block_stage_matches_reshaped_max():
    rng = np.random.default_rng(21)
    n, bs, kb = 262144, 8, 2048
    row = rng.standard_normal(n).astype(np.float32)
    bscore = row.reshape(-1, bs).max(axis=1)
    got = oracle.topk_blocks(row[None, :], [n], bs, kb)[0]
    want = oracle.topk_row(bscore, bscore.shape[0], kb)
    assert np.array_equal(got, want)
    # and a partial last block: its max covers only the valid part
    L = n - 5
    bscore2 = bscore.copy()
    bscore2[-1] = row[(n // bs - 1) * bs:L].max()
    got2 = oracle.topk_blocks(row[None, :], [L], bs, kb)[0]
    want2 = oracle.topk_row(bscore2, bscore2.shape[0], kb)
    assert np.array_equal(got2, want2)
