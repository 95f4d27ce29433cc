"""GPU parity of the two threshold modes of plain rows split over 2 to 64
workgroups, and of the mode word that chooses between them.

Mode 0: each workgroup bounds the candidates it publishes by its own scores.
Mode 1: every workgroup takes the same threshold from a sample of the whole
row and region sizes from the sample's per-chunk counts. Both are exact for
any input (a bound that turns out too high sends the last workgroup to its
second pass); the tests force each mode on rows shaped to stress it (spread,
clustered, tied, -inf-heavy, a cluster the sample misses, ragged lengths,
few valid scores), then follow the mode word across calls that share a
workspace. Results are compared with the CPU oracle as index sets.
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
    prev = ltk.lt_debug_force_path(ltk.PATH_SPLIT)
    yield
    ltk.lt_debug_force_path(prev)
    ltk.lt_debug_force_sample(ltk.SAMPLE_AUTO)


@pytest.fixture(params=["never", "always"])
def mode(request):
    prev = ltk.lt_debug_force_sample({"never": ltk.SAMPLE_NEVER,
                                      "always": ltk.SAMPLE_ALWAYS}[request.param])
    yield request.param
    ltk.lt_debug_force_sample(prev)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def same_sets(got, want, what):
    for r in range(want.shape[0]):
        m = int(np.sum(want[r] >= 0))
        assert np.all(got[r][m:] == -1), (what, r, "padding")
        if not np.array_equal(np.sort(got[r][:m]), np.sort(want[r][:m])):
            miss = np.setdiff1d(want[r][:m], got[r][:m])
            raise AssertionError("%s row %d: %d of %d differ" % (what, r, len(miss), m))


def run(scores, lengths, k, ws=None):
    s, l = to_dev(scores), to_dev(np.asarray(lengths, np.int32))
    out = ltk.lt_topk_run(s, l, k, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(scores, lengths, k, what):
    lengths = np.asarray(lengths, np.int32)
    same_sets(run(scores, lengths, k), oracle.topk(scores, lengths, k, nthreads=NTH), what)


def clustered_rows(n, seed):
    """Rows whose winners cluster: a hot window, a ramp, tied sinks, a
    600-wide cluster placed between the sample's runs of chunk 3 (the
    sample misses it), and a row whose best scores are spread."""
    rng = np.random.default_rng(seed)
    i = np.arange(n)
    base = lambda: rng.standard_normal(n).astype(np.float32)
    rows = [base() + np.float32(4.0) * (i >= n - min(16384, n // 4)),
            base() + np.float32(2.0) * (i / n) ** 4,
            np.where(i < 600, np.float32(10.0), base()),
            base()]
    hide = base()
    if n > 4 * 4096:
        # chunk 3's runs start at 3 * 4096 + q * 1024 + ((15 + 3 q) % 64) * 16;
        # positions 3 * 4096 + 300 .. + 900 avoid run 0 (offset 240 .. 255)
        # and lie below run 1 (offset 1024 + 288)
        lo = 3 * 4096 + 300
        hide[lo:lo + 600] = np.float32(6.0) + rng.standard_normal(600).astype(np.float32) * 0.1
    rows.append(hide)
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("n", [262144, 100003, 8200])
def test_modes_on_clustered_and_spread_rows(n, mode):
    s = clustered_rows(n, n)
    for r in range(s.shape[0]):
        for k in (512, 7, 1024):
            check(s[r:r + 1], [n], k, "n=%d row %d k=%d %s" % (n, r, k, mode))


@pytest.mark.parametrize("variant", ["a", "b", "c"])
def test_modes_on_bs1_workloads(variant, mode):
    w = workloads.cfg3(variant)
    check(w.scores, w.lengths, 512, "cfg3%s %s" % (variant, mode))


@pytest.mark.parametrize("pattern", ["recent", "ramp", "sinks"])
def test_modes_on_clustered_workloads(pattern, mode):
    w = workloads.clustered(pattern)
    check(w.scores, w.lengths, 512, "%s %s" % (pattern, mode))


def test_modes_on_special_rows(mode):
    """Ragged lengths (the last chunk partial, a row ending inside a sample
    run), few valid scores, all-NaN, constant and -inf-heavy rows, bf16 ties."""
    n = 262144
    rng = np.random.default_rng(77)
    rows, lens = [], []
    for r in range(10):
        x = rng.standard_normal(n).astype(np.float32)
        if r == 1:
            x[:] = np.nan
        elif r == 2:
            x[:] = np.float32(1.5)
        elif r == 3:
            x[rng.random(n) < 0.97] = -np.inf
        elif r == 4:
            x = workloads.round_to_bf16(x * np.float32(0.01))
        elif r == 5:
            x[rng.random(n) < 0.5] = np.nan
        rows.append(x)
        lens.append([n, n, n, n, n, n, 4096 * 5 + 100, 300, 4096 * 2 + 1, n - 4096 * 3 - 7][r])
    s = np.stack(rows)
    for k in (1, 512, 1024):
        for r in range(len(rows)):
            check(s[r:r + 1], lens[r:r + 1], k, "special row %d k=%d %s" % (r, k, mode))


def test_modes_on_batches(mode):
    """Several rows per launch (one record each), lengths spanning 2 to 64
    workgroups."""
    n = 262144
    rng = np.random.default_rng(5)
    s = clustered_rows(n, 9)
    s = np.concatenate([s, rng.standard_normal((3, n)).astype(np.float32)])
    lens = np.array([n, n - 5, 70000, 4097, 131072, 262000, 9000, 200000], np.int32)
    check(s, lens, 512, "batch %s" % mode)


def _mode_word(ws, row=0):
    """The row record's mode word (word 1 of the record; the size query for
    one split row gives the record's length)."""
    words = ltk.lt_topk_workspace_bytes(1, 262144, 512) // 4
    return int(ws.view(torch.int32)[row * words + 1].item())


def test_mode_word_follows_the_rows():
    """With the default setting, a fresh workspace starts in mode 0; a
    clustered row there needs the second pass and sets mode 1; the next call
    samples (and keeps mode 1 while a workgroup publishes many candidates); a
    spread row in mode 1 sets mode 0 again. Every call is exact."""
    ltk.lt_debug_force_sample(ltk.SAMPLE_AUTO)
    rec = workloads.clustered("recent")
    iid = workloads.cfg3("a")
    want_rec = oracle.topk(rec.scores, rec.lengths, 512, nthreads=NTH)
    want_iid = oracle.topk(iid.scores, iid.lengths, 512, nthreads=NTH)
    ws = torch.zeros(ltk.lt_topk_workspace_bytes(1, 262144, 512), dtype=torch.uint8, device=DEV)
    seq = [(iid, want_iid, 0), (rec, want_rec, 1), (rec, want_rec, 1), (iid, want_iid, 0),
           (iid, want_iid, 0), (rec, want_rec, 1)]
    for step, (w, want, mode_after) in enumerate(seq):
        same_sets(run(w.scores, w.lengths, 512, ws=ws), want, "step %d" % step)
        assert _mode_word(ws) == mode_after, (step, _mode_word(ws))


def test_mode_word_under_graph_replays():
    """50 replays of one captured call, clustered and spread inputs copied in
    alternately: the mode word flips between replays, every result exact."""
    ltk.lt_debug_force_sample(ltk.SAMPLE_AUTO)
    rec = workloads.clustered("sinks")
    iid = workloads.cfg3("b")
    want = [np.sort(oracle.topk(w.scores, w.lengths, 512, nthreads=NTH), axis=1) for w in (rec, iid)]
    src = [to_dev(rec.scores), to_dev(iid.scores)]
    s = src[0].clone()
    l = to_dev(rec.lengths)
    out = torch.empty((1, 512), dtype=torch.int32, device=DEV)
    ws = torch.zeros(ltk.lt_topk_workspace_bytes(1, 262144, 512), dtype=torch.uint8, device=DEV)
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
    for rep in range(50):
        j = (rep // 2) % 2  # two replays per input: one in each mode on the switch
        s.copy_(src[j])
        out.fill_(-7)
        g.replay()
        got = np.sort(out.cpu().numpy(), axis=1)
        if not np.array_equal(got, want[j]):
            raise AssertionError("replay %d (input %d) differs from the oracle" % (rep, j))
