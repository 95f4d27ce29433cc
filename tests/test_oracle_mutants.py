"""The oracle's pins catch plausible mistakes.

Each mutant is a copy of the oracle's C source with one planted mistake (a
flipped tie rule, NaN ranked high, -0.0 ranked below +0.0, a dropped length
clamp inside a partial block, ...), compiled on the CPU into a temporary
library. Every mutant must fail at least one of the checks below, which are the
same kinds of check the real pins use (brute force over the alphabet, closed
forms, library reduction, block brute force, candidate brute force).
"""
import ctypes
import itertools
import os
import subprocess
import tempfile

import numpy as np
import pytest

from tests import bruteforce as bf

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "ltopk_oracle.c")

MUTANTS = {
    "tie_higher_index_first": ("return a->i < b->i;", "return a->i > b->i;"),
    "nan_highest": ("return b_nan; /*", "return a_nan; /*"),
    "ascending": ("return a->s > b->s;", "return a->s < b->s;"),
    "neg_zero_below_pos_zero": (
        "if (!a_nan && a->s != b->s)\n        return a->s > b->s;",
        "if (!a_nan && (a->s != b->s || signbit(a->s) != signbit(b->s)))\n"
        "        return a->s > b->s || (a->s == b->s && !signbit(a->s));"),
    "m_off_by_one": ("int64_t m = n < k ? n : k;", "int64_t m = n < k ? n : k - 1;"),
    "len_clamp_off_by_one": ("if (len > n_max)\n        return n_max;",
                             "if (len > n_max)\n        return n_max - 1;"),
    "partial_block_ignores_len": ("int64_t hi = lo + bs < len ? lo + bs : len;",
                                  "int64_t hi = lo + bs;"),
    "block_scored_by_first": ("if (lto_before(&cur, &best))", "if (0 && lto_before(&cur, &best))"),
    "candidate_past_len": ("if (pos < len)\n                    member[pos] = 1;",
                           "if (pos < len + bs)\n                    member[pos < len ? pos : 0] = 1;"),
    "empty_slot_read_as_block_0": ("if (b < 0)\n                continue;",
                                   "if (b < 0)\n                b = 0;"),
}


def build_mutant(name, tmpdir):
    with open(SRC) as f:
        src = f.read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = os.path.join(tmpdir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmpdir, name + ".so")
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
                    "-pthread", "-o", so, path, "-lm"], check=True)
    lib = ctypes.CDLL(so)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f32p = ctypes.POINTER(ctypes.c_float)
    lib.lt_oracle_topk_batch.argtypes = [f32p, ctypes.c_int64, i32p, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_int32, i32p, ctypes.c_int32, ctypes.c_int32, i32p,
                                         ctypes.c_int]
    lib.lt_oracle_blocks_batch.argtypes = [f32p, ctypes.c_int64, i32p, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, i32p,
                                           ctypes.c_int]
    return lib


def run_topk(lib, rows, lens, k, cand=None, bs=1):
    rows = np.ascontiguousarray(rows, np.float32)
    B, n = rows.shape
    lens = np.ascontiguousarray(lens, np.int32)
    out = np.empty((B, k), np.int32)
    f = lambda a, t: a.ctypes.data_as(ctypes.POINTER(t))
    if cand is not None:
        cand = np.ascontiguousarray(cand, np.int32)
        cp, nc = f(cand, ctypes.c_int32), cand.shape[1]
    else:
        cp, nc = None, 0
    lib.lt_oracle_topk_batch(f(rows, ctypes.c_float), n, f(lens, ctypes.c_int32), B, n, k, cp, nc,
                             bs, f(out, ctypes.c_int32), 1)
    return out


def run_blocks(lib, rows, lens, bs, kb):
    rows = np.ascontiguousarray(rows, np.float32)
    B, n = rows.shape
    lens = np.ascontiguousarray(lens, np.int32)
    out = np.empty((B, kb), np.int32)
    f = lambda a, t: a.ctypes.data_as(ctypes.POINTER(t))
    lib.lt_oracle_blocks_batch(f(rows, ctypes.c_float), n, f(lens, ctypes.c_int32), B, n, bs, kb,
                               f(out, ctypes.c_int32), 1)
    return out


ALPHABET = np.array([np.nan, -np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], dtype=np.float32)


def pins_pass(lib):
    """Return True iff the library passes every check."""
    # brute force over the alphabet, n = 4, all lengths and k
    n = 4
    rows = ALPHABET[np.array(list(itertools.product(range(7), repeat=n)))]
    R = rows.shape[0]
    for L in range(n + 1):
        valid = np.zeros((R, n), bool)
        valid[:, :L] = True
        for k in (1, 2, 3, 5):
            if not np.array_equal(run_topk(lib, rows, np.full(R, L), k).astype(np.int64),
                                  bf.ordered(rows.astype(np.float64), valid, k)):
                return False
    # lengths beyond the row are clamped: compare with the in-range call
    rng = np.random.default_rng(1)
    r = rng.standard_normal((4, 32)).astype(np.float32)
    r[:, -1] = 10.0     # the last position is the best one, so dropping it shows
    if not np.array_equal(run_topk(lib, r, [10**6] * 4, 8), run_topk(lib, r, [32] * 4, 8)):
        return False
    if not np.all(run_topk(lib, r, [10**6] * 4, 8)[:, 0] == 31):
        return False
    # closed form: all equal -> first m
    if not np.array_equal(np.sort(run_topk(lib, np.zeros((1, 50), np.float32), [50], 7)[0]),
                          np.arange(7)):
        return False
    # blocks: brute force
    vals = np.array([np.nan, -np.inf, -1.0, -0.0, 0.0, 2.0, np.inf], np.float32)
    rows = vals[rng.integers(0, 7, size=(200, 13))]
    lens = rng.integers(0, 14, size=200).astype(np.int32)
    bsc, bval = bf.block_scores(rows.astype(np.float64), lens, 4)
    if not np.array_equal(run_blocks(lib, rows, lens, 4, 3).astype(np.int64),
                          bf.ordered(bsc, bval, 3)):
        return False
    # candidates: brute force
    rows = vals[rng.integers(0, 7, size=(200, 14))]
    lens = rng.integers(0, 15, size=200).astype(np.int32)
    cand = np.stack([rng.permutation(6)[:3] - 1 for _ in range(200)]).astype(np.int32)
    member = np.zeros((200, 14), bool)
    for i in range(200):
        for b in cand[i]:
            if b >= 0:
                member[i, b * 3:b * 3 + 3] = True
    valid = member & (np.arange(14)[None, :] < lens[:, None])
    if not np.array_equal(run_topk(lib, rows, lens, 4, cand=cand, bs=3).astype(np.int64),
                          bf.ordered(rows.astype(np.float64), valid, 4)):
        return False
    return True


def test_unmodified_oracle_passes():
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "orig.so")
        subprocess.run(["gcc", "-O2", "-fno-fast-math", "-std=c11", "-D_GNU_SOURCE", "-fPIC",
                        "-shared", "-pthread", "-o", path, SRC, "-lm"], check=True)
        MUTANTS_SAVED = dict(MUTANTS)
        MUTANTS["__identity__"] = ("int32_t i;\n} lto_item;", "int32_t i;\n} lto_item;")
        try:
            lib = build_mutant("__identity__", d)
        finally:
            MUTANTS.clear()
            MUTANTS.update(MUTANTS_SAVED)
        assert pins_pass(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as d:
        lib = build_mutant(name, d)
        assert not pins_pass(lib), "planted mistake %r was not caught" % name
