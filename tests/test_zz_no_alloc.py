"""lt_topk_run_noalloc (the entry point that allocates nothing) against
lt_topk_run, through the C ABI.

For callers that cannot allocate device memory: the split rows' exchange runs
in the library's built-in buffer instead of a caller workspace. Each case makes
two calls in a row, the second with a smaller input, and compares the index
sets of both with lt_topk_run's on the same inputs (and with the CPU oracle).
The buffer keeps the last call's contents, so the second call also checks
that a call leaves it reusable.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import topk_index_selection_amd as ltk
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NTH = 16


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def sets(out):
    return np.sort(out, axis=1)


def raw_noalloc(s, l, k, out, cand=None):
    lib = ltk.load_library()
    B, n = s.shape
    c = None
    if cand is not None:
        c = ctypes.byref(ltk._Cand(cand[0].data_ptr(), int(cand[0].shape[1]), int(cand[1])))
    return lib.lt_topk_run_noalloc(s.data_ptr(), s.stride(0), l.data_ptr(), B, n, k, c,
                                   out.data_ptr(), torch.cuda.current_stream().cuda_stream)


def compare(scores, lengths, k, what, cand_np=None, bs=8):
    s, l = to_dev(scores), to_dev(lengths)
    B = s.shape[0]
    cand = (to_dev(cand_np), bs) if cand_np is not None else None
    ref = ltk.lt_topk_run(s, l, k, cand=cand)
    out = torch.full((B, k), 0x5EADBEEF, dtype=torch.int32, device=DEV)
    rc = raw_noalloc(s, l, k, out, cand)
    torch.cuda.synchronize()
    assert rc == ltk.LT_OK, (what, rc)
    got = out.cpu().numpy()
    assert np.array_equal(sets(got), sets(ref.cpu().numpy())), what
    if cand_np is not None:
        want = oracle.topk(scores, lengths, k, cand=cand_np, bs=bs, nthreads=NTH)
    else:
        want = oracle.topk(scores, lengths, k, nthreads=NTH)
    assert np.array_equal(sets(got), sets(want)), what


def test_bs1_then_smaller_row():
    a = workloads.cfg3("b")
    compare(a.scores, a.lengths, 512, "bs1 262144")
    b = workloads.cfg3("a", n=40000)
    compare(b.scores, b.lengths, 512, "bs1 40000")


def test_decode_then_smaller_batch():
    d = workloads.cfg2()
    compare(d.scores, d.lengths, 512, "decode 64x32768")
    e = workloads.cfg2(B=5, n_max=20000)
    compare(e.scores, e.lengths, 512, "decode 5x20000")


def test_long_candidate_list_then_shorter():
    rng = np.random.default_rng(21)
    n = 262144
    s = rng.standard_normal((3, n)).astype(np.float32)
    lens = np.array([n, n - 5, n // 3], np.int32)
    cand = np.stack([rng.permutation(n // 8)[:4096] for _ in range(3)]).astype(np.int32)
    compare(s, lens, 512, "candidates 4096 blocks", cand_np=cand)
    compare(s[:1], lens[:1], 512, "candidates 2048 blocks", cand_np=cand[:1, :2048].copy())


def test_streamed_batch_then_split_row():
    """A batch that streams (no split rows: no buffer needed, no row limit) and
    then a split row."""
    w = workloads.cfg5(rows=np.arange(0, 8192, 32))
    compare(w.scores, w.lengths, 512, "prefill 256 rows")
    a = workloads.cfg3("c")
    compare(a.scores, a.lengths, 512, "bs1 90% -inf")


def test_too_many_split_rows_is_enospc():
    """More split rows than the built-in buffer holds: LT_ENOSPC, nothing written."""
    rng = np.random.default_rng(5)
    B, n = ltk.LT_NOALLOC_SPLIT_ROWS + 1, 32768
    s = to_dev(rng.standard_normal((B, n)).astype(np.float32))
    l = to_dev(np.full(B, n, np.int32))
    prev = ltk.lt_debug_force_path(ltk.PATH_SPLIT)
    try:
        assert ltk.lt_debug_launch_shape(B, n)[0] == "split"
        out = torch.full((B, 512), 0x5EADBEEF, dtype=torch.int32, device=DEV)
        rc = raw_noalloc(s, l, 512, out)
        torch.cuda.synchronize()
        assert rc == ltk.LT_ENOSPC
        assert bool((out == 0x5EADBEEF).all())
        # at the limit it runs
        w = workloads.cfg2()
        assert w.B == ltk.LT_NOALLOC_SPLIT_ROWS
        compare(w.scores, w.lengths, 512, "decode at the limit")
    finally:
        ltk.lt_debug_force_path(prev)
    # rows that one workgroup each takes whole need no buffer at all
    out = torch.full((B, 512), 0x5EADBEEF, dtype=torch.int32, device=DEV)
    assert ltk.lt_debug_launch_shape(B, n)[0] == "row"
    assert raw_noalloc(s, l, 512, out) == ltk.LT_OK
    torch.cuda.synchronize()
    want = oracle.topk(s.cpu().numpy(), np.full(B, n, np.int32), 512, nthreads=NTH)
    assert np.array_equal(sets(out.cpu().numpy()), sets(want))


def test_graph_capture_replays():
    """Captured in a graph (the caller that cannot allocate): every replay exact,
    inputs alternated between replays."""
    a, b = workloads.cfg3("a"), workloads.cfg3("b")
    want = [sets(oracle.topk(a.scores, a.lengths, 512, nthreads=NTH)),
            sets(oracle.topk(b.scores, b.lengths, 512, nthreads=NTH))]
    src = [to_dev(a.scores), to_dev(b.scores)]
    s = src[0].clone()
    l = to_dev(a.lengths)
    out = torch.empty((1, 512), dtype=torch.int32, device=DEV)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        ltk.lt_topk_run_noalloc(s, l, 512, out=out)
    torch.cuda.synchronize()
    for rep in range(20):
        s.copy_(src[rep % 2])
        out.fill_(-7)
        g.replay()
        assert np.array_equal(sets(out.cpu().numpy()), want[rep % 2]), rep
    # and an eager call afterwards
    s.copy_(src[0])
    assert np.array_equal(sets(ltk.lt_topk_run_noalloc(s, l, 512).cpu().numpy()), want[0])
