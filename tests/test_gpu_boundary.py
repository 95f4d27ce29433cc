"""GPU checks of the C ABI's workspace contract and error paths.

* A workspace shorter than the call needs (or none while bytes are needed)
  returns LT_ENOSPC before anything is launched: the output keeps its bytes.
* Every call returns its counters to zero: the ticket word that opens each
  row's record reads back as 0 after split plain rows, split block stages and
  split candidate lists, so the workspace needs no clearing between calls.
* Block stages with one position per block and rows just past one workgroup's
  1024 blocks take a workspace (the size query says so) and are exact.
* Many graph replays of split-row calls, alternating two input sets, are
  exact on every replay (the workgroups' exchange through the workspace).

Every call goes through the C ABI (ctypes); results are compared with the CPU
oracle as sorted index sets.
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
SENTINEL = 0x5EADBEEF


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ltk.load_library()
    yield
    ltk.lt_debug_force_path(ltk.PATH_AUTO)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def same_sets(got, want, what):
    for r in range(want.shape[0]):
        m = int(np.sum(want[r] >= 0))
        assert np.all(got[r][m:] == -1), (what, r)
        assert np.array_equal(np.sort(got[r][:m]), np.sort(want[r][:m])), (what, r)


def row_record_words():
    """Words per row record: the size query for one split row."""
    return ltk.lt_topk_workspace_bytes(1, 262144, 512) // 4


# ------------------------------------------------------------ LT_ENOSPC

def _raw_run(s, l, k, out, ws_ptr, ws_bytes, cand=None):
    lib = ltk.load_library()
    B, n = s.shape
    c = None
    if cand is not None:
        c = ctypes.byref(ltk._Cand(cand[0].data_ptr(), int(cand[0].shape[1]), int(cand[1])))
    return lib.lt_topk_run(s.data_ptr(), s.stride(0), l.data_ptr(), B, n, k, c, out.data_ptr(),
                           ws_ptr, ws_bytes, torch.cuda.current_stream().cuda_stream)


def _enospc_cases():
    a = workloads.cfg3("a")
    d = workloads.cfg2()
    return {"bs1": (a.scores, a.lengths), "decode": (d.scores, d.lengths)}


@pytest.fixture
def split_path():
    """Rows split over workgroups (the launches that use a workspace)."""
    prev = ltk.lt_debug_force_path(ltk.PATH_SPLIT)
    yield
    ltk.lt_debug_force_path(prev)


@pytest.mark.parametrize("case", ["bs1", "decode"])
@pytest.mark.parametrize("short", ["null", "one_row_less", "16_bytes_less"])
def test_short_workspace_is_enospc_and_output_untouched(case, short, split_path):
    scores, lengths = _enospc_cases()[case]
    s, l = to_dev(scores), to_dev(lengths)
    B, n = s.shape
    need = ltk.lt_topk_workspace_bytes(B, n, 512)
    assert need > 0
    out = torch.full((B, 512), SENTINEL, dtype=torch.int32, device=DEV)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    size = {"null": 0, "one_row_less": need - 4 * row_record_words(), "16_bytes_less": need - 16}[short]
    ptr = None if short == "null" else ws.data_ptr()
    rc = _raw_run(s, l, 512, out, ptr, size)
    torch.cuda.synchronize()
    assert rc == ltk.LT_ENOSPC
    assert bool((out == SENTINEL).all()), "output written although nothing may be launched"
    assert bool((ws == 0).all()), "workspace written although nothing may be launched"
    # the same call with the full workspace then succeeds
    assert _raw_run(s, l, 512, out, ws.data_ptr(), need) == ltk.LT_OK
    torch.cuda.synchronize()
    same_sets(out.cpu().numpy(), oracle.topk(scores, lengths, 512, nthreads=NTH), case)


def test_short_workspace_enospc_through_the_binding():
    a = workloads.cfg3("a")
    s, l = to_dev(a.scores), to_dev(a.lengths)
    small = torch.zeros(256, dtype=torch.uint8, device=DEV)
    out = torch.full((1, 512), SENTINEL, dtype=torch.int32, device=DEV)
    with pytest.raises(ltk.LtError) as e:
        ltk.lt_topk_run(s, l, 512, out=out, ws=small)
    assert e.value.status == ltk.LT_ENOSPC
    with pytest.raises(ltk.LtError) as e:
        ltk.lt_topk_blocks(s, l, 8, 2048, out=torch.empty((1, 2048), dtype=torch.int32,
                                                          device=DEV), ws=small)
    assert e.value.status == ltk.LT_ENOSPC
    torch.cuda.synchronize()
    assert bool((out == SENTINEL).all())


# ------------------------------------------------------------ counters return to zero

def _split_calls():
    """(name, rows, call(ws)) for calls that split rows over workgroups."""
    a = workloads.cfg3("b")
    d = workloads.cfg2()
    s_a, l_a = to_dev(a.scores), to_dev(a.lengths)
    s_d, l_d = to_dev(d.scores), to_dev(d.lengths)
    rng = np.random.default_rng(11)
    B4, n4 = 3, 262144
    s4 = rng.standard_normal((B4, n4)).astype(np.float32)
    l4 = np.full(B4, n4, np.int32)
    cand = np.stack([rng.permutation(n4 // 8)[:4096] for _ in range(B4)]).astype(np.int32)
    s4d, l4d, c4d = to_dev(s4), to_dev(l4), to_dev(cand)
    return [
        ("plain_bs1", 1, lambda ws: ltk.lt_topk_run(s_a, l_a, 512, ws=ws),
         lambda: oracle.topk(a.scores, a.lengths, 512, nthreads=NTH)),
        ("plain_decode", 64, lambda ws: ltk.lt_topk_run(s_d, l_d, 512, ws=ws),
         lambda: oracle.topk(d.scores, d.lengths, 512, nthreads=NTH)),
        ("blocks", 1, lambda ws: ltk.lt_topk_blocks(s_a, l_a, 8, 2048, ws=ws),
         lambda: oracle.topk_blocks(a.scores, a.lengths, 8, 2048, nthreads=NTH)),
        ("blocks_bs1", 1, lambda ws: ltk.lt_topk_blocks(s_a, l_a, 1, 512, ws=ws),
         lambda: oracle.topk_blocks(a.scores, a.lengths, 1, 512, nthreads=NTH)),
        ("cand_long_list", B4, lambda ws: ltk.lt_topk_run(s4d, l4d, 512, cand=(c4d, 8), ws=ws),
         lambda: oracle.topk(s4, l4, 512, cand=cand, bs=8, nthreads=NTH)),
    ]


def test_ticket_words_read_back_zero():
    prev = ltk.lt_debug_force_path(ltk.PATH_SPLIT)
    try:
        words = row_record_words()
        need = ltk.lt_topk_workspace_bytes(64, 262144, 2048)
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        for name, rows, call, want in _split_calls():
            ws.zero_()
            for rep in range(3):
                out = call(ws)
                torch.cuda.synchronize()
                same_sets(out.cpu().numpy(), want(), "%s call %d" % (name, rep))
                w = ws.view(torch.int32).cpu().numpy()
                tickets = w[np.arange(rows) * words]
                assert np.all(tickets == 0), (name, rep, np.nonzero(tickets)[0][:8])
                # the region past the records actually used was never touched
                assert np.all(w[rows * words:] == 0), name
    finally:
        ltk.lt_debug_force_path(prev)


# ------------------------------------------------------------ one position per block

@pytest.mark.parametrize("n", [1025, 1500, 2048])
@pytest.mark.parametrize("force", [ltk.PATH_AUTO, ltk.PATH_SPLIT])
def test_block_stage_bs1_just_past_one_workgroup(n, force):
    prev = ltk.lt_debug_force_path(force)
    try:
        rng = np.random.default_rng(n)
        B = 3
        s = rng.standard_normal((B, n)).astype(np.float32)
        s[1] = workloads.round_to_bf16(s[1] * 0.01)
        lens = np.array([n, n - 1, 1024], np.int32)
        assert ltk.lt_topk_workspace_bytes(B, n, 512) > 0
        # rows padded to a multiple of 4 floats (the row stride must be)
        pad = np.full((B, n + (-n) % 4), np.inf, np.float32)
        pad[:, :n] = s
        sd = to_dev(pad)[:, :n]
        for kb in (7, 512, 1024):
            got = ltk.lt_topk_blocks(sd, to_dev(lens), 1, kb)
            torch.cuda.synchronize()
            same_sets(got.cpu().numpy(), oracle.topk_blocks(s, lens, 1, kb, nthreads=NTH),
                      "bs1 n=%d kb=%d" % (n, kb))
    finally:
        ltk.lt_debug_force_path(prev)


# ------------------------------------------------------------ many replays of the exchange

def _replay_inputs(case):
    if case == "bs1":
        a, b = workloads.cfg3("a"), workloads.cfg3("b")
        return a.scores, b.scores, a.lengths
    a = workloads.cfg2()
    rng = np.random.default_rng(3)
    b = rng.standard_normal(a.scores.shape).astype(np.float32)
    b[np.arange(a.n_max)[None, :] >= a.lengths[:, None]] = np.inf
    return a.scores, b, a.lengths


@pytest.mark.parametrize("case", ["bs1", "decode"])
def test_split_exchange_200_graph_replays(case, split_path):
    """200 replays of one captured split-row call, the two input sets copied in
    alternately between replays; each replay checked against the oracle, the
    test stopping at the first mismatch."""
    first, second, lengths = _replay_inputs(case)
    B, n = first.shape
    want = [oracle.topk(first, lengths, 512, nthreads=NTH),
            oracle.topk(second, lengths, 512, nthreads=NTH)]
    want_sorted = [np.sort(w, axis=1) for w in want]
    src = [to_dev(first), to_dev(second)]
    s = src[0].clone()
    l = to_dev(lengths)
    out = torch.empty((B, 512), dtype=torch.int32, device=DEV)
    ws = torch.zeros(ltk.lt_topk_workspace_bytes(B, n, 512), dtype=torch.uint8, device=DEV)
    assert ltk.lt_debug_launch_shape(B, n)[0] == "split"
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        ltk.lt_topk_run(s, l, 512, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        ltk.lt_topk_run(s, l, 512, out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(200):
        j = rep % 2
        s.copy_(src[j])
        out.fill_(SENTINEL)
        g.replay()
        got = np.sort(out.cpu().numpy(), axis=1)   # synchronises
        if not np.array_equal(got, want_sorted[j]):
            raise AssertionError("%s replay %d differs from the oracle" % (case, rep))
