"""Seeded randomized GPU parity: random batch sizes, row lengths, k, score
distributions (normal, bf16-rounded, few distinct values, -inf and NaN heavy,
constant, clustered windows, ramps both ways), kernel paths and threshold
modes, for plain rows, the block stage and candidate lists. Every row of
every case is compared with the CPU oracle as an index set. The cases are a
fixed function of the seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

import oracle
import topk_index_selection_amd as ltk
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NTH = 16
PATHS = [ltk.PATH_AUTO, ltk.PATH_SPLIT, ltk.PATH_STREAM, ltk.PATH_ROW]
MODES = [ltk.SAMPLE_AUTO, ltk.SAMPLE_NEVER, ltk.SAMPLE_ALWAYS]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ltk.load_library()
    yield
    ltk.lt_debug_force_path(ltk.PATH_AUTO)
    ltk.lt_debug_force_sample(ltk.SAMPLE_AUTO)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def same_sets(got, want, what):
    for r in range(want.shape[0]):
        m = int(np.sum(want[r] >= 0))
        assert np.all(got[r][m:] == -1), (what, r, "padding")
        if not np.array_equal(np.sort(got[r][:m]), np.sort(want[r][:m])):
            miss = np.setdiff1d(want[r][:m], got[r][:m])
            raise AssertionError("%s row %d: %d of %d differ" % (what, r, len(miss), m))


def random_row(rng, n, kind):
    i = np.arange(n)
    x = rng.standard_normal(n).astype(np.float32)
    if kind == "bf16":
        x = workloads.round_to_bf16(x * np.float32(rng.choice([0.01, 1.0, 300.0])))
    elif kind == "few":
        x = rng.integers(0, 7, n).astype(np.float32)
    elif kind == "neginf":
        x[rng.random(n) < rng.uniform(0.5, 0.99)] = -np.inf
    elif kind == "nan":
        x[rng.random(n) < rng.uniform(0.1, 0.9)] = np.nan
        x[rng.random(n) < 0.01] = np.inf
    elif kind == "const":
        x[:] = np.float32(rng.choice([0.0, -0.0, 3.5, -2.0]))
    elif kind == "window":
        w = int(rng.integers(1, max(2, n // 8)))
        lo = int(rng.integers(0, max(1, n - w)))
        x[lo:lo + w] += np.float32(rng.uniform(2, 8))
    elif kind == "rise":
        x = (i / max(n, 1)).astype(np.float32) + np.float32(2 ** -12) * x
    elif kind == "fall":
        x = (1.0 - i / max(n, 1)).astype(np.float32) + np.float32(2 ** -12) * x
    return x.astype(np.float32)


KINDS = ["normal", "bf16", "few", "neginf", "nan", "const", "window", "rise", "fall"]


def make_case(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.choice([1, 1, 2, 3, 7, 33]))
    n_max = int(rng.choice([1, 5, 600, 4096, 4097, 9000, 33000, 70000, 131073, 262144]))
    n_max = min(n_max, 262144 if B <= 3 else 70000)
    k = int(rng.choice([1, 7, 64, 512, 513, 1024, 2048, 4096]))
    lens = rng.integers(0, n_max + 1, B).astype(np.int32)
    lens[0] = n_max
    stride = n_max + (-n_max) % 4 + int(rng.choice([0, 0, 4]))
    s = np.full((B, max(stride, 4)), np.inf, np.float32)
    for r in range(B):
        s[r, :n_max] = random_row(rng, n_max, KINDS[int(rng.integers(len(KINDS)))])
    path = PATHS[int(rng.integers(len(PATHS)))]
    mode = MODES[int(rng.integers(len(MODES)))]
    return s, n_max, lens, k, path, mode, rng


@pytest.mark.parametrize("seed", range(120))
def test_random_plain_rows(seed):
    s, n_max, lens, k, path, mode, _ = make_case(seed)
    what = "seed %d B=%d n_max=%d k=%d path=%d mode=%d" % (seed, s.shape[0], n_max, k, path, mode)
    ltk.lt_debug_force_path(path)
    ltk.lt_debug_force_sample(mode)
    sd = to_dev(s)[:, :n_max]
    out = ltk.lt_topk_run(sd, to_dev(lens), k)
    torch.cuda.synchronize()
    same_sets(out.cpu().numpy(), oracle.topk(s[:, :n_max], lens, k, nthreads=NTH), what)


@pytest.mark.parametrize("seed", range(60))
def test_random_two_stage(seed):
    s, n_max, lens, k, path, mode, rng = make_case(100 + seed)
    bs = int(rng.choice([8, 8, 1, 3]))
    kb = int(rng.choice([7, 300, 2048]))
    k = min(k, 2048)
    what = "seed %d B=%d n_max=%d bs=%d kb=%d k=%d path=%d" % (seed, s.shape[0], n_max, bs, kb, k, path)
    ltk.lt_debug_force_path(path)
    ltk.lt_debug_force_sample(mode)
    sd = to_dev(s)[:, :n_max]
    blocks, out = ltk.lt_topk_two_stage(sd, to_dev(lens), bs, kb, k)
    torch.cuda.synchronize()
    wb = oracle.topk_blocks(s[:, :n_max], lens, bs, kb, nthreads=NTH)
    same_sets(blocks.cpu().numpy(), wb, what + " blocks")
    same_sets(out.cpu().numpy(), oracle.topk(s[:, :n_max], lens, k, cand=wb, bs=bs, nthreads=NTH),
              what + " top-k")
