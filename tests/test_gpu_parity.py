"""GPU parity: the HIP path against the CPU oracle, bit-exact as index sets.

Every case runs through the C ABI (libltopk.so via the ctypes binding) on
cuda:0 and compares each row's selected indices, sorted ascending, with the
oracle's; slots past min(k, |V|) must be -1. The five workloads run at full
size (the causal prefill batch on every row of the full launch),
plus an edge suite over every kernel path: one workgroup per row, a row split
over many workgroups, one streaming workgroup per row, and one workgroup per
whole row of up to 32,768 scores.
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


@pytest.fixture(params=["auto", "split", "stream", "row"])
def path(request):
    # "row": one workgroup per whole row wherever n_max <= 32768 (else auto)
    prev = ltk.lt_debug_force_path({"auto": 0, "split": 1, "stream": 2, "row": 3}[request.param])
    yield request.param
    ltk.lt_debug_force_path(prev)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_topk(scores, lengths, k, cand=None, bs=8):
    s = to_dev(scores)
    l = to_dev(np.asarray(lengths, np.int32))
    c = (to_dev(np.asarray(cand, np.int32)), bs) if cand is not None else None
    out = ltk.lt_topk_run(s, l, k, cand=c)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_blocks(scores, lengths, bs, kb):
    out = ltk.lt_topk_blocks(to_dev(scores), to_dev(np.asarray(lengths, np.int32)), bs, kb)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_same_sets(got, want, what=""):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    for r in range(got.shape[0]):
        m = int(np.sum(want[r] >= 0))
        g = got[r]
        assert np.all(g[m:] == -1), (what, r, "padding")
        gs, ws = np.sort(g[:m]), np.sort(want[r][:m])
        if not np.array_equal(gs, ws):
            missing = np.setdiff1d(ws, gs)[:8]
            extra = np.setdiff1d(gs, ws)[:8]
            raise AssertionError("%s row %d: %d/%d differ; missing %s extra %s"
                                 % (what, r, len(np.setdiff1d(ws, gs)), m, missing, extra))


def check(scores, lengths, k, what=""):
    lengths = np.asarray(lengths, np.int32)
    got = gpu_topk(scores, lengths, k)
    want = oracle.topk(scores, lengths, k, nthreads=NTH)
    assert_same_sets(got, want, what)


# ------------------------------------------------------------ the five workloads

def test_cfg1_single_row(path):
    w = workloads.cfg1()
    check(w.scores, w.lengths, w.k, "cfg1")


def test_cfg1_matches_golden():
    w = workloads.cfg1()
    got = np.sort(gpu_topk(w.scores, w.lengths, w.k), axis=1)
    want = []
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "cfg1_topk512.txt")) as f:
        for line in f:
            if not line.startswith("#") and line.strip():
                want.append([int(v) for v in line.split()])
    assert np.array_equal(got, np.array(want, np.int32))


def test_cfg2_decode(path):
    w = workloads.cfg2()
    check(w.scores, w.lengths, w.k, "cfg2")


@pytest.mark.parametrize("variant", ["a", "b", "c"])
def test_cfg3_bs1(variant, path):
    w = workloads.cfg3(variant)
    check(w.scores, w.lengths, w.k, "cfg3" + variant)


@pytest.mark.parametrize("B", [1, 32])
def test_cfg4_two_stage(B, path):
    w = workloads.cfg4(B)
    s, l = to_dev(w.scores), to_dev(w.lengths)
    blocks = ltk.lt_topk_blocks(s, l, w.bs, w.kb)
    out = ltk.lt_topk_run(s, l, w.k, cand=(blocks, w.bs))
    torch.cuda.synchronize()
    want_blocks = oracle.topk_blocks(w.scores, w.lengths, w.bs, w.kb, nthreads=NTH)
    assert_same_sets(blocks.cpu().numpy(), want_blocks, "cfg4 blocks")
    want = oracle.topk(w.scores, w.lengths, w.k, cand=want_blocks, bs=w.bs, nthreads=NTH)
    assert_same_sets(out.cpu().numpy(), want, "cfg4 top-k")


def test_cfg5_prefill_every_row():
    """The full causal prefill batch (8192 rows of ~262,144 scores) in one
    call, as the benchmark times it: every row's index set equal to the
    oracle's."""
    w = workloads.cfg5()
    assert ltk.lt_debug_launch_shape(w.B, w.n_max)[0] == "stream"
    got = gpu_topk(w.scores, w.lengths, w.k)
    want = oracle.topk(w.scores, w.lengths, w.k, nthreads=NTH)
    same = np.all(np.sort(got, axis=1) == np.sort(want, axis=1), axis=1)
    if not np.all(same):
        bad = np.nonzero(~same)[0]
        assert_same_sets(got[bad[:1]], want[bad[:1]], "cfg5 row %d (%d rows differ)"
                         % (bad[0], len(bad)))


def test_prefill_rising_ramp_rows():
    """Near-monotone causal rows rising toward the present (every 8th row of
    the 8192-row ramp batch, one streaming launch): exact."""
    w = workloads.cfg5_ramp(rows=np.arange(0, 8192, 8))
    assert ltk.lt_debug_launch_shape(w.B, w.n_max)[0] == "stream"
    check(w.scores, w.lengths, w.k, "rising ramp")


def test_falling_and_tied_rows_streamed():
    """Rows whose best scores come first (falling) or that tie at the threshold:
    read from the end backwards, every such element enters the buffer; the
    selection must stay exact."""
    rng = np.random.default_rng(31)
    B, n = 1100, 20000
    s = np.empty((B, n), np.float32)
    i = np.arange(n, dtype=np.float32)
    for r in range(B):
        kind = r % 4
        if kind == 0:
            s[r] = (n - i) / n + np.float32(2 ** -12) * rng.standard_normal(n).astype(np.float32)
        elif kind == 1:
            s[r] = np.float32(1.0)                                   # one value throughout
        elif kind == 2:
            s[r] = rng.integers(0, 3, n).astype(np.float32)          # three values
        else:
            s[r] = -i                                                # strictly falling
    lens = np.full(B, n, np.int32)
    lens[::7] = n - 13
    prev = ltk.lt_debug_force_path(ltk.PATH_STREAM)
    try:
        for k in (1, 512, 2048):
            check(s, lens, k, "falling/tied k=%d" % k)
    finally:
        ltk.lt_debug_force_path(prev)


def test_cfg5_rows_all_paths(path):
    """512 causal rows (the prefill recipe), every row checked."""
    rows = np.arange(0, 8192, 16)
    w = workloads.cfg5(rows=rows)
    check(w.scores, w.lengths, w.k, "cfg5 rows")


# ------------------------------------------------------------ edge suite

SHAPES = [(1, 3000), (3, 50000), (40, 9000)]   # one workgroup / split / many rows


@pytest.mark.parametrize("B,n", SHAPES)
@pytest.mark.parametrize("k", [1, 7, 512, 2048, 4096])
def test_lengths_and_k(B, n, k, path):
    rng = np.random.default_rng(B * n + k)
    s = rng.standard_normal((B, n)).astype(np.float32)
    cand_lens = [0, 1, k - 1, k, k + 1, 4 * 37 + 1, 4 * 37 + 2, 4 * 37 + 3, n - 1, n]
    lens = np.array([cand_lens[i % len(cand_lens)] for i in range(B)], np.int32)
    lens = np.clip(lens, 0, n)
    s[np.arange(n)[None, :] >= lens[:, None]] = np.inf   # poison beyond the length
    check(s, lens, k, "lengths")


@pytest.mark.parametrize("B,n", SHAPES)
def test_special_rows(B, n, path):
    rng = np.random.default_rng(n)
    k = 512
    kinds = []
    for r in range(B):
        kind = r % 10
        if kind == 0:
            row = np.full(n, 0.25, np.float32)                       # all equal
        elif kind == 1:
            row = np.full(n, -np.inf, np.float32)                    # all -inf
        elif kind == 2:
            row = np.full(n, -np.inf, np.float32)                    # fewer than k finite
            row[rng.choice(n, min(n, 100), replace=False)] = rng.standard_normal(min(n, 100))
        elif kind == 3:
            row = rng.standard_normal(n).astype(np.float32)          # NaNs sprinkled
            row[rng.random(n) < 0.2] = np.nan
        elif kind == 4:
            row = np.where(rng.random(n) < 0.5, -0.0, 0.0).astype(np.float32)  # +-0 only
        elif kind == 5:
            row = (rng.integers(-3, 4, n) * np.float32(1e-45)).astype(np.float32)  # denormals
        elif kind == 6:
            row = np.arange(n, dtype=np.float32)                     # ascending
        elif kind == 7:
            row = np.arange(n, 0, -1).astype(np.float32)             # descending
        elif kind == 8:
            row = np.full(n, np.nan, np.float32)                     # all NaN
            row[::7] = -np.inf
        else:
            row = workloads.round_to_bf16(rng.standard_normal(n).astype(np.float32))
        kinds.append(row)
    s = np.stack(kinds)
    check(s, np.full(B, n, np.int32), k, "special")


@pytest.mark.parametrize("poison", [np.inf, np.nan, 1e30])
def test_poison_beyond_length(poison, path):
    rng = np.random.default_rng(1)
    B, n = 6, 40000
    s = rng.standard_normal((B, n)).astype(np.float32)
    lens = np.array([0, 5, 511, 4097, 39999, 20000], np.int32)
    s[np.arange(n)[None, :] >= lens[:, None]] = poison
    check(s, lens, 512, "poison")


def test_lengths_clamped():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((3, 9000)).astype(np.float32)
    lens = np.array([-5, 10**9, 9000], np.int32)
    check(s, lens, 512, "clamp")


def test_row_stride_larger_than_n_max():
    rng = np.random.default_rng(3)
    for B, n, stride in ((4, 5000, 5124), (2, 30001, 30004), (300, 7000, 7004)):
        big = np.full((B, stride), np.inf, np.float32)
        big[:, :n] = rng.standard_normal((B, n)).astype(np.float32)
        lens = np.full(B, n, np.int32)
        gs = to_dev(big)[:, :n]
        out = ltk.lt_topk_run(gs, to_dev(lens), 512)
        torch.cuda.synchronize()
        want = oracle.topk(np.ascontiguousarray(big[:, :n]), lens, 512, nthreads=NTH)
        assert_same_sets(out.cpu().numpy(), want, "stride")


def test_heavy_ties_bf16_many_rows(path):
    rng = np.random.default_rng(4)
    s = workloads.round_to_bf16((rng.standard_normal((64, 20000)) * 0.01).astype(np.float32))
    check(s, np.full(64, 20000, np.int32), 512, "bf16 ties")


# ------------------------------------------------------------ blocks / candidates

@pytest.mark.parametrize("bs", [1, 3, 8, 16])
@pytest.mark.parametrize("B,n,kb", [(1, 262144, 2048), (5, 10000, 300), (2, 70000, 4096)])
def test_block_stage(bs, B, n, kb, path):
    rng = np.random.default_rng(bs * 1000 + B)
    s = rng.standard_normal((B, n)).astype(np.float32)
    if B > 1:
        s[1] = workloads.round_to_bf16(s[1] * 0.01)
    lens = np.array([n - (r * 13) % 29 for r in range(B)], np.int32)
    got = gpu_blocks(s, lens, bs, kb)
    want = oracle.topk_blocks(s, lens, bs, kb, nthreads=NTH)
    assert_same_sets(got, want, "blocks bs=%d" % bs)


@pytest.mark.parametrize("bs", [8, 5])
def test_independent_row_candidates(bs, path):
    """Stage 1 on one layer's scores, stage 2 on another's (the shared-candidate data flow)."""
    rng = np.random.default_rng(7 + bs)
    B, n, kb, k = 4, 262144 if bs == 8 else 50000, 2048, 512
    s1 = rng.standard_normal((B, n)).astype(np.float32)
    s2 = rng.standard_normal((B, n)).astype(np.float32)
    lens = np.array([n, n - 1, n - 7, n // 2], np.int32)
    blocks = oracle.topk_blocks(s1, lens, bs, kb, nthreads=NTH)
    got = gpu_topk(s2, lens, k, cand=blocks, bs=bs)
    want = oracle.topk(s2, lens, k, cand=blocks, bs=bs, nthreads=NTH)
    assert_same_sets(got, want, "independent rows")


def test_candidates_with_empty_and_out_of_range_ids(path):
    rng = np.random.default_rng(9)
    B, n, bs, k = 3, 20000, 8, 100
    s = rng.standard_normal((B, n)).astype(np.float32)
    lens = np.array([n, 1003, 0], np.int32)
    nb = -(-n // bs)
    cand = np.stack([rng.permutation(nb + 50)[:600] - 25 for _ in range(B)]).astype(np.int32)
    got = gpu_topk(s, lens, k, cand=cand, bs=bs)
    want = oracle.topk(s, lens, k, cand=cand, bs=bs, nthreads=NTH)
    assert_same_sets(got, want, "cand ids")


# ------------------------------------------------------------ properties

def test_determinism_repeated_calls():
    w = workloads.cfg3("b")
    s, l = to_dev(w.scores), to_dev(w.lengths)
    first = np.sort(ltk.lt_topk_run(s, l, 512).cpu().numpy(), axis=1)
    for _ in range(50):
        again = np.sort(ltk.lt_topk_run(s, l, 512).cpu().numpy(), axis=1)
        assert np.array_equal(first, again)


def test_workspace_reused_across_shapes():
    """One workspace, many calls of different shapes back to back: every result exact."""
    cases = [workloads.cfg2(), workloads.cfg3("b"), workloads.cfg1(), workloads.cfg3("c"),
             workloads.cfg2(B=5, n_max=20000)]
    need = max(ltk.lt_topk_workspace_bytes(w.B, w.n_max, w.k) for w in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for _ in range(2):
        for w in cases:
            out = ltk.lt_topk_run(to_dev(w.scores), to_dev(w.lengths), w.k, ws=ws)
            torch.cuda.synchronize()
            assert_same_sets(out.cpu().numpy(), oracle.topk(w.scores, w.lengths, w.k, nthreads=NTH),
                             w.name)


@pytest.fixture
def fallback():
    prev = ltk.lt_debug_force_fallback(True)
    yield
    ltk.lt_debug_force_fallback(bool(prev))


@pytest.mark.parametrize("name", ["cfg2", "cfg3a", "cfg3b", "cfg3c"])
def test_split_exact_fallback(name, fallback):
    """The last workgroup's exact re-read path, forced on for every split row."""
    w = workloads.make(name)
    prev = ltk.lt_debug_force_path(ltk.PATH_SPLIT)
    try:
        check(w.scores, w.lengths, w.k, name + " fallback")
    finally:
        ltk.lt_debug_force_path(prev)


def test_two_stage_exact_fallback(fallback):
    w = workloads.cfg4(2)
    s, l = to_dev(w.scores), to_dev(w.lengths)
    blocks = ltk.lt_topk_blocks(s, l, w.bs, w.kb)
    out = ltk.lt_topk_run(s, l, w.k, cand=(blocks, w.bs))
    torch.cuda.synchronize()
    want_blocks = oracle.topk_blocks(w.scores, w.lengths, w.bs, w.kb, nthreads=NTH)
    assert_same_sets(blocks.cpu().numpy(), want_blocks, "blocks fallback")
    want = oracle.topk(w.scores, w.lengths, w.k, cand=want_blocks, bs=w.bs, nthreads=NTH)
    assert_same_sets(out.cpu().numpy(), want, "cand fallback")


@pytest.mark.parametrize("order", ["index", "rank"])
def test_long_candidate_lists(order, path):
    """Candidate lists longer than one workgroup holds (4096 blocks of 8 =
    32768 slots) are split over workgroups. In rank order every winner sits
    in the first workgroup's part of the list, which the split path cannot
    prove exact, so its recovery must re-read that part."""
    rng = np.random.default_rng(4096 + len(order))
    B, n, kb, k = 2, 262144, 4096, 512
    s = rng.standard_normal((B, n)).astype(np.float32)
    lens = np.array([n, n - 5], np.int32)
    blocks = oracle.topk_blocks(s, lens, 8, kb, nthreads=NTH)  # rank order
    if order == "index":
        blocks = np.sort(blocks, axis=1)
    got = gpu_topk(s, lens, k, cand=blocks, bs=8)
    want = oracle.topk(s, lens, k, cand=blocks, bs=8, nthreads=NTH)
    assert_same_sets(got, want, "long candidate list, %s order" % order)


def test_long_candidate_list_exact_fallback(fallback):
    """The split candidate path's exact re-read, forced on."""
    rng = np.random.default_rng(4097)
    B, n, kb, k = 2, 262144, 4096, 512
    s = rng.standard_normal((B, n)).astype(np.float32)
    lens = np.array([n - 3, n], np.int32)
    blocks = np.sort(oracle.topk_blocks(s, lens, 8, kb, nthreads=NTH), axis=1)
    got = gpu_topk(s, lens, k, cand=blocks, bs=8)
    want = oracle.topk(s, lens, k, cand=blocks, bs=8, nthreads=NTH)
    assert_same_sets(got, want, "long candidate list, forced fallback")


@pytest.mark.parametrize("pattern", ["recent", "ramp", "sinks"])
def test_clustered_rows_recovery(pattern, path):
    """Scores that cluster as attention scores do: a hot window of recent
    positions, a rising ramp, or 600 tied sink positions at the start. The
    workgroups holding the winners leave some out; the exact set must still
    come back, for plain rows and for the block stage."""
    n = 262144
    rng = np.random.default_rng({"recent": 1, "ramp": 2, "sinks": 3}[pattern])
    base = rng.standard_normal(n).astype(np.float32)
    i = np.arange(n)
    if pattern == "recent":
        s = base + np.float32(4.0) * (i >= n - 16384)
    elif pattern == "ramp":
        s = base + np.float32(2.0) * (i / n) ** 4
    else:
        s = np.where(i < 600, np.float32(10.0), base)
    s = np.stack([s.astype(np.float32), s[::-1].astype(np.float32)])
    lens = np.array([n, n - 9], np.int32)
    check(s[:1], lens[:1], 512, "clustered %s %s" % (pattern, path))
    check(s, lens, 512, "clustered %s B=2 %s" % (pattern, path))
    got = gpu_blocks(s, lens, 8, 2048)
    want = oracle.topk_blocks(s, lens, 8, 2048, nthreads=NTH)
    assert_same_sets(got, want, "clustered blocks %s %s" % (pattern, path))


def test_clustered_rows_recovery_coarse_chunks():
    """Twelve clustered rows: enough rows that the split launches take the
    coarse chunks (8 scores or 4 blocks per thread), whose recovery re-reads
    each flagged chunk in several pieces."""
    n, B = 262144, 12
    rng = np.random.default_rng(12)
    i = np.arange(n)
    rows = []
    for r in range(B):
        base = rng.standard_normal(n).astype(np.float32)
        if r % 3 == 0:
            rows.append(base + np.float32(4.0) * (i >= n - 16384 - 1000 * r))
        elif r % 3 == 1:
            rows.append(base + np.float32(2.0 + 0.1 * r) * (i / n) ** 4)
        else:
            rows.append(np.where((i >= 700 * r) & (i < 700 * r + 600), np.float32(10.0), base))
    s = np.stack(rows).astype(np.float32)
    lens = np.array([n - 17 * r for r in range(B)], np.int32)
    prev = ltk.lt_debug_force_path(ltk.PATH_SPLIT)
    try:
        kern, grid, block = ltk.lt_debug_launch_shape(B, n)
        assert grid[0] == 32, grid  # coarse chunks: 8192 scores per workgroup
        check(s, lens, 512, "clustered coarse")
        got = gpu_blocks(s, lens, 8, 2048)
    finally:
        ltk.lt_debug_force_path(prev)
    want = oracle.topk_blocks(s, lens, 8, 2048, nthreads=NTH)
    assert_same_sets(got, want, "clustered coarse blocks")


@pytest.mark.parametrize("case", ["many_ties", "one_wave", "ties_and_wave", "below_floor_ties"])
@pytest.mark.parametrize("form", ["plain", "blocks"])
def test_recovery_staging_fallbacks(case, form):
    """Rows whose recovery stages flagged chunks in LDS but whose survivors do
    not fit the per-wave lists: more than 2048 of them (3000 tied keys in one
    chunk), or more than 128 in one wave's share (hot positions only at
    offsets 0..63 of every 1024, which the interleaved lists hand to one
    wave). The selection falls back to re-reading the chunks and must stay
    exact; also ties straddling the fast selection's floor."""
    n = 262144
    rng = np.random.default_rng(77)
    i = np.arange(n)
    base = rng.standard_normal(n).astype(np.float32)
    if case == "many_ties":
        row = np.where((i >= 40960) & (i < 40960 + 3000), np.float32(50.0), base)
    elif case == "one_wave":
        hot = (i >= 20 * 4096) & (i < 24 * 4096) & ((i % 1024) < 64)
        row = np.where(hot, np.float32(10.0) + np.float32(0.01) * base, base)
    elif case == "ties_and_wave":
        hot = (i >= 8 * 4096) & (i < 12 * 4096) & ((i % 1024) < 64)
        row = np.where(hot, np.float32(7.0), base)
    else:
        # a tied block just above the other chunks' best scores
        row = np.where((i >= 4096 * 30) & (i < 4096 * 30 + 700), np.float32(4.25), base)
    s = row.astype(np.float32)[None, :]
    lens = np.array([n], np.int32)
    prev = ltk.lt_debug_force_path(ltk.PATH_SPLIT)
    try:
        if form == "plain":
            for k in (512, 2048):
                check(s, lens, k, "%s k=%d" % (case, k))
        else:
            for bs in (1, 8):
                got = gpu_blocks(s, lens, bs, 512)
                assert_same_sets(got, oracle.topk_blocks(s, lens, bs, 512, nthreads=NTH),
                                 "%s blocks bs=%d" % (case, bs))
    finally:
        ltk.lt_debug_force_path(prev)


@pytest.mark.parametrize("n", [50000, 262144])
def test_clustered_winners_trip_the_check(n):
    """All of a row's best scores inside one workgroup's chunk: the gathered
    candidates cannot prove exactness, so the exact path must take over."""
    rng = np.random.default_rng(n)
    B = 3
    s = rng.standard_normal((B, n)).astype(np.float32)
    s[0, 5000:5000 + 2000] += 10.0                      # one chunk holds everything
    s[1] = np.sort(s[1])                                 # ascending: winners at the end
    s[2, ::4096] = 50.0                                  # one winner per chunk, rest i.i.d.
    check(s, np.full(B, n, np.int32), 512, "clustered")


# ------------------------------------------------------------ graph capture

def _graph_case(case):
    """(first, second) input sets of one shape, and the call to capture."""
    if case == "bs1":
        a, b = workloads.cfg3("a"), workloads.cfg3("b")
        return (a.scores, a.lengths), (b.scores, b.lengths), a.k, None
    if case == "decode":
        a = workloads.cfg2()
        return (a.scores, a.lengths), (-a.scores, a.lengths), a.k, None
    if case == "stream":
        a = workloads.cfg5(rows=np.arange(0, 8192, 128))
        return (a.scores, a.lengths), (-a.scores, a.lengths), a.k, ltk.PATH_STREAM
    raise ValueError(case)


@pytest.mark.parametrize("case", ["bs1", "decode", "stream"])
def test_graph_replays_match_oracle(case):
    """The call captured once in a graph and replayed with new scores copied in
    between (eager work between replays): every replay exact. The workspace is
    never cleared between calls, so this also checks that calls leave it reusable."""
    first, second, k, force = _graph_case(case)
    prev = ltk.lt_debug_force_path(force) if force is not None else None
    try:
        s = to_dev(first[0])
        l = to_dev(np.asarray(first[1], np.int32))
        B, n = first[0].shape
        out = torch.empty((B, k), dtype=torch.int32, device=DEV)
        ws = torch.zeros(max(ltk.lt_topk_workspace_bytes(B, n, k), 1 << 20), dtype=torch.uint8,
                         device=DEV)
        want = {0: oracle.topk(first[0], first[1], k, nthreads=NTH),
                1: oracle.topk(second[0], second[1], k, nthreads=NTH)}
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            ltk.lt_topk_run(s, l, k, out=out, ws=ws)  # eager call on the capture stream
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        assert_same_sets(out.cpu().numpy(), want[0], case + " eager")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            ltk.lt_topk_run(s, l, k, out=out, ws=ws)
        torch.cuda.synchronize()
        for rep in range(4):
            src = first if rep % 2 == 0 else second
            s.copy_(to_dev(src[0]))
            out.fill_(12345)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_same_sets(out.cpu().numpy(), want[rep % 2], "%s replay %d" % (case, rep))
    finally:
        if prev is not None:
            ltk.lt_debug_force_path(prev)


def test_graph_two_stage_replays():
    """Block stage and restricted stage captured together, replayed with new scores."""
    a = workloads.cfg4(1)
    variants = [a.scores, -a.scores]
    s = to_dev(a.scores)
    l = to_dev(a.lengths)
    blocks = torch.empty((a.B, a.kb), dtype=torch.int32, device=DEV)
    out = torch.empty((a.B, a.k), dtype=torch.int32, device=DEV)
    ws = torch.zeros(max(ltk.lt_topk_workspace_bytes(a.B, a.n_max, a.kb), 1 << 20),
                     dtype=torch.uint8, device=DEV)
    want = []
    for v in variants:
        wb = oracle.topk_blocks(v, a.lengths, a.bs, a.kb, nthreads=NTH)
        want.append((wb, oracle.topk(v, a.lengths, a.k, cand=wb, bs=a.bs, nthreads=NTH)))
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        ltk.lt_topk_blocks(s, l, a.bs, a.kb, out=blocks, ws=ws)
        ltk.lt_topk_run(s, l, a.k, cand=(blocks, a.bs), out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        ltk.lt_topk_blocks(s, l, a.bs, a.kb, out=blocks, ws=ws)
        ltk.lt_topk_run(s, l, a.k, cand=(blocks, a.bs), out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        s.copy_(to_dev(variants[rep % 2]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same_sets(blocks.cpu().numpy(), want[rep % 2][0], "blocks replay %d" % rep)
        assert_same_sets(out.cpu().numpy(), want[rep % 2][1], "top-k replay %d" % rep)


# ------------------------------------------------------------ context-parallel merge (one GPU)

@pytest.mark.parametrize("variant", ["a", "b", "c"])
def test_cp_shard_merge_emulation(variant):
    """A long row sharded as under context parallelism: local top-k on each of
    8 shards (one batch row per shard), shard offsets added, then the top-k of
    the 8 * k candidates (candidate form with block size 1). The result must be
    the single-row top-k: a global winner has no more predecessors within its
    shard than in the whole row, so it survives its shard's selection."""
    w = workloads.cfg3(variant)
    n, k, P = w.n_max, w.k, 8
    row = to_dev(w.scores[0])
    shards = row.view(P, n // P)
    lens = torch.full((P,), n // P, dtype=torch.int32, device=DEV)
    local = ltk.lt_topk_run(shards, lens, k)
    offs = (torch.arange(P, device=DEV, dtype=torch.int32) * (n // P)).view(P, 1)
    cand = torch.where(local >= 0, local + offs, local).reshape(1, P * k).contiguous()
    merged = ltk.lt_topk_run(row.view(1, n), to_dev(w.lengths), k, cand=(cand, 1))
    torch.cuda.synchronize()
    assert_same_sets(merged.cpu().numpy(), oracle.topk(w.scores, w.lengths, k, nthreads=NTH),
                     "cp merge " + variant)


# ------------------------------------------------------------ block and candidate edge cases

def _special_rows(n, seed):
    """Rows that stress the order: special values, ties, degenerate rows."""
    rng = np.random.default_rng(seed)
    rows = [rng.standard_normal(n).astype(np.float32)]
    rows.append(np.full(n, 0.5, np.float32))                               # all equal
    r = rng.standard_normal(n).astype(np.float32)
    r[rng.choice(n, n // 3, replace=False)] = np.nan                       # NaNs
    rows.append(r)
    r = rng.choice(np.array([0.0, -0.0, 1e-45, -1e-45, 1.0], np.float32), n)
    rows.append(r.astype(np.float32))                                      # zeros, denormals
    r = np.full(n, -np.inf, np.float32)
    r[rng.choice(n, 40, replace=False)] = rng.standard_normal(40).astype(np.float32)
    rows.append(r)                                                         # mostly -inf
    rows.append(workloads.round_to_bf16(rng.standard_normal(n).astype(np.float32) * 0.01))
    r = rng.standard_normal(n).astype(np.float32)
    r[rng.choice(n, 50, replace=False)] = np.inf
    rows.append(r)                                                         # +inf inside
    return np.stack(rows)


@pytest.mark.parametrize("kb", [1, 7, 300, 2048, 4096])
def test_block_stage_special_rows(kb, path):
    n = 20004
    s = _special_rows(n, 11)
    B = s.shape[0]
    lens = np.array([n, n - 1, n - 5, 8 * 900 + 3, n, 17, 1][:B], np.int32)
    got = gpu_blocks(s, lens, 8, kb)
    want = oracle.topk_blocks(s, lens, 8, kb, nthreads=NTH)
    assert_same_sets(got, want, "blocks special kb=%d %s" % (kb, path))


@pytest.mark.parametrize("k", [1, 7, 512, 2048])
def test_candidates_special_rows(k, path):
    n = 40004
    s = _special_rows(n, 12)
    B = s.shape[0]
    rng = np.random.default_rng(13)
    lens = np.array([n, n - 3, 8 * 4000 + 5, n, 29, n, 0][:B], np.int32)
    nb = -(-n // 8)
    cand = np.stack([rng.permutation(nb + 40)[:900] - 20 for _ in range(B)]).astype(np.int32)
    got = gpu_topk(s, lens, k, cand=cand, bs=8)
    want = oracle.topk(s, lens, k, cand=cand, bs=8, nthreads=NTH)
    assert_same_sets(got, want, "cand special k=%d %s" % (k, path))


def test_two_stage_batch_streaming():
    """Many rows: both stages take the streaming kernel on their own."""
    w = workloads.cfg5(rows=np.arange(0, 8192, 8))
    s, l = to_dev(w.scores), to_dev(w.lengths)
    s1 = torch.roll(s, 1, dims=0)
    l1 = torch.roll(l, 1, dims=0)
    blocks = ltk.lt_topk_blocks(s1, l1, 8, 2048)
    out = ltk.lt_topk_run(s, l, 512, cand=(blocks, 8))
    torch.cuda.synchronize()
    rows = np.arange(0, w.B, 37)
    s1h = np.roll(w.scores, 1, axis=0)[rows]
    l1h = np.roll(w.lengths, 1)[rows]
    want_b = oracle.topk_blocks(s1h, l1h, 8, 2048, nthreads=NTH)
    assert_same_sets(blocks.cpu().numpy()[rows], want_b, "batch blocks")
    want = oracle.topk(w.scores[rows], w.lengths[rows], 512, cand=want_b, bs=8, nthreads=NTH)
    assert_same_sets(out.cpu().numpy()[rows], want, "batch top-k")


def _structured_rows(n, seed):
    """Rows that move the streaming kernel's running threshold in unusual ways:
    trends (the histogram's top bin keeps filling), far outliers (its bins grow
    coarse), few distinct values (bins too full to resolve), a narrow range at a
    large magnitude, and a second cluster far above the first."""
    rng = np.random.default_rng(seed)
    z = lambda: rng.standard_normal(n).astype(np.float32)
    t = np.arange(n, dtype=np.float32) / n
    rows = [
        z() + 8.0 * t,                                   # rising trend
        z() - 8.0 * t,                                   # falling trend
        np.where(np.arange(n) == 5, np.float32(1e30), z()),        # early outlier
        np.where(np.arange(n) == n - 7, np.float32(-1e30), z() * 1e-3),  # late outlier, tiny range
        rng.integers(0, 10, n).astype(np.float32),      # ten distinct values
        np.float32(1000.0) + z() * np.float32(1e-4),    # narrow range, large magnitude
        np.where(rng.random(n) < 0.01, z() + 100.0, z()).astype(np.float32),  # far cluster
        ((np.arange(n) % 4099) / 4099.0).astype(np.float32) + z() * 0.01,    # sawtooth
        np.where(rng.random(n) < 0.5, z() * 1e-38, -z() * 1e-38).astype(np.float32),  # denormal-ish
        workloads.round_to_bf16(z() * 3.0 + t * 4.0),   # bf16 ties on a trend
    ]
    return np.stack([r.astype(np.float32) for r in rows])


@pytest.mark.parametrize("k", [512, 2048])
def test_structured_rows(k, path):
    n = 100000
    s = _structured_rows(n, 21)
    B = s.shape[0]
    lens = np.array([n, n - 1, n, n - 13, n, n, 77777, n, n, n - 2][:B], np.int32)
    check(s, lens, k, "structured k=%d %s" % (k, path))


@pytest.mark.parametrize("kb", [300, 2048])
def test_block_stage_structured_rows(kb, path):
    n = 100000
    s = _structured_rows(n, 22)
    B = s.shape[0]
    lens = np.full(B, n, np.int32)
    lens[3] = n - 5
    got = gpu_blocks(s, lens, 8, kb)
    want = oracle.topk_blocks(s, lens, 8, kb, nthreads=NTH)
    assert_same_sets(got, want, "blocks structured kb=%d %s" % (kb, path))


def test_candidates_structured_rows(path):
    n = 100000
    s = _structured_rows(n, 23)
    B = s.shape[0]
    lens = np.full(B, n, np.int32)
    rng = np.random.default_rng(24)
    nb = n // 8
    cand = np.stack([rng.permutation(nb)[:2048] for _ in range(B)]).astype(np.int32)
    got = gpu_topk(s, lens, 512, cand=cand, bs=8)
    want = oracle.topk(s, lens, 512, cand=cand, bs=8, nthreads=NTH)
    assert_same_sets(got, want, "cand structured %s" % path)
