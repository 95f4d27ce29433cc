"""GPU parity of lt_topk_two_stage: both stages of a shared-candidate layer in
one call (one launch when the block stage takes the split kernel with one
block per thread, kb <= 2048, k <= 512 and blocks of eight; else the two
calls). Each case checks the blocks and the restricted top-k against the CPU
oracle as index sets, through the C ABI.
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


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ltk.load_library()
    yield
    ltk.lt_debug_force_path(ltk.PATH_AUTO)
    ltk.lt_debug_force_fallback(False)


@pytest.fixture(params=["auto", "split", "stream", "row"])
def path(request):
    prev = ltk.lt_debug_force_path({"auto": 0, "split": 1, "stream": 2, "row": 3}[request.param])
    yield request.param
    ltk.lt_debug_force_path(prev)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def same_sets(got, want, what):
    for r in range(want.shape[0]):
        m = int(np.sum(want[r] >= 0))
        assert np.all(got[r][m:] == -1), (what, r, "padding")
        if not np.array_equal(np.sort(got[r][:m]), np.sort(want[r][:m])):
            miss = np.setdiff1d(want[r][:m], got[r][:m])
            raise AssertionError("%s row %d: %d of %d differ" % (what, r, len(miss), m))


def check(scores, lengths, bs, kb, k, what):
    lengths = np.asarray(lengths, np.int32)
    n = scores.shape[1]
    pad = np.full((scores.shape[0], n + (-n) % 4), np.inf, np.float32)
    pad[:, :n] = scores
    s = to_dev(pad)[:, :n]
    blocks, out = ltk.lt_topk_two_stage(s, to_dev(lengths), bs, kb, k)
    torch.cuda.synchronize()
    wb = oracle.topk_blocks(scores, lengths, bs, kb, nthreads=NTH)
    same_sets(blocks.cpu().numpy(), wb, what + " blocks")
    wt = oracle.topk(scores, lengths, k, cand=wb, bs=bs, nthreads=NTH)
    same_sets(out.cpu().numpy(), wt, what + " top-k")


@pytest.mark.parametrize("B", [1, 2, 32])
def test_cfg4(B, path):
    w = workloads.cfg4(B)
    check(w.scores, w.lengths, w.bs, w.kb, w.k, "cfg4 B=%d %s" % (B, path))


@pytest.mark.parametrize("n", [5, 1000, 8191, 9000, 100003, 262144])
@pytest.mark.parametrize("kb,k", [(2048, 512), (300, 7), (7, 1), (2048, 2048), (1024, 512)])
def test_lengths_and_sizes(n, kb, k):
    rng = np.random.default_rng(n + kb + k)
    B = 3
    s = rng.standard_normal((B, n)).astype(np.float32)
    lens = np.array([n, max(1, n - 13), n // 3], np.int32)
    check(s, lens, 8, kb, k, "n=%d kb=%d k=%d" % (n, kb, k))


def test_special_rows():
    """NaN, +-inf, +-0 and heavy ties (a constant row overflows the candidate
    row's survivor list and takes its exact re-read)."""
    n = 262144
    rng = np.random.default_rng(4)
    rows = []
    for r in range(5):
        x = rng.standard_normal(n).astype(np.float32)
        if r == 0:
            x[rng.random(n) < 0.3] = np.nan
        elif r == 1:
            x[rng.random(n) < 0.9] = -np.inf
            x[:100] = np.inf
        elif r == 2:
            x[:] = np.float32(2.0)
        elif r == 3:
            x = workloads.round_to_bf16(x * np.float32(0.01))
        elif r == 4:
            x[rng.random(n) < 0.5] = np.float32(-0.0)
            x[rng.random(n) < 0.5] = np.float32(0.0)
        rows.append(x)
    s = np.stack(rows)
    for r in range(len(rows)):
        check(s[r:r + 1], [n], 8, 2048, 512, "special row %d" % r)
    check(s, [n, n - 5, 70000, n, 4096], 8, 2048, 512, "special batch")


@pytest.mark.parametrize("pattern", ["recent", "ramp", "sinks"])
def test_clustered_rows(pattern):
    w = workloads.clustered(pattern)
    check(w.scores, w.lengths, 8, 2048, 512, pattern)


def test_exact_fallback_then_candidates():
    prev = ltk.lt_debug_force_fallback(True)
    try:
        w = workloads.cfg4(1)
        check(w.scores, w.lengths, w.bs, w.kb, w.k, "forced fallback")
    finally:
        ltk.lt_debug_force_fallback(bool(prev))


def test_graph_replays():
    """20 replays of one captured call, two input sets copied in alternately,
    both outputs checked on every replay."""
    a = workloads.cfg4(1)
    variants = [a.scores, workloads.clustered("recent").scores]
    want = []
    for v in variants:
        wb = oracle.topk_blocks(v, a.lengths, a.bs, a.kb, nthreads=NTH)
        want.append((np.sort(wb, axis=1),
                     np.sort(oracle.topk(v, a.lengths, a.k, cand=wb, bs=a.bs, nthreads=NTH), axis=1)))
    src = [to_dev(v) for v in variants]
    s = src[0].clone()
    l = to_dev(a.lengths)
    blocks = torch.empty((1, a.kb), dtype=torch.int32, device=DEV)
    out = torch.empty((1, a.k), dtype=torch.int32, device=DEV)
    ws = torch.zeros(ltk.lt_topk_workspace_bytes(1, a.n_max, a.k), dtype=torch.uint8, device=DEV)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        ltk.lt_topk_two_stage(s, l, a.bs, a.kb, a.k, out_blocks=blocks, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        ltk.lt_topk_two_stage(s, l, a.bs, a.kb, a.k, out_blocks=blocks, out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(20):
        j = rep % 2
        s.copy_(src[j])
        out.fill_(-7)
        blocks.fill_(-7)
        g.replay()
        gb = np.sort(blocks.cpu().numpy(), axis=1)
        go = np.sort(out.cpu().numpy(), axis=1)
        if not (np.array_equal(gb, want[j][0]) and np.array_equal(go, want[j][1])):
            raise AssertionError("replay %d (input %d) differs from the oracle" % (rep, j))
