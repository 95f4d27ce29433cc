"""GPU parity of the split kernel's tie break. When every candidate left at
the selection's prefix has one key, the last workgroup of a row of four
scores per thread takes the lowest indices among them from the order of its
gathered slots (regions follow the chunks, each published in position
order) instead of a pass per index digit. These rows tie the selection's
last key across chunks, slot groups and waves: a block of tied scores at the
top (attention sinks) at several places, ties scattered over the whole row,
ties below a few larger scores, bf16-rounded and few-valued rows, a constant
row, in both threshold modes, for k = 512, 1024 and 2048 and a ragged
length. Results are compared with the CPU oracle as index sets.
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
N = 262144


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ltk.load_library()
    prev = ltk.lt_debug_force_path(ltk.PATH_SPLIT)
    yield
    ltk.lt_debug_force_path(prev)
    ltk.lt_debug_force_sample(ltk.SAMPLE_AUTO)


def tied_row(kind, n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n).astype(np.float32)
    if kind.startswith("block"):
        p0 = min(int(kind[5:]), n - 600)
        x[p0:p0 + 600] = np.float32(10.0)
    elif kind == "scatter":
        x[rng.choice(n, 700, replace=False)] = np.float32(10.0)
    elif kind == "below_top":
        pos = rng.choice(n, 1200, replace=False)
        x[pos[:300]] = np.float32(20.0)
        x[pos[300:]] = np.float32(10.0)
    elif kind == "bf16_fine":
        x = workloads.round_to_bf16(x * np.float32(0.01))
    elif kind == "bf16_coarse":
        x = workloads.round_to_bf16(x * np.float32(300.0))
    elif kind == "few":
        x = rng.integers(0, 7, n).astype(np.float32)
    elif kind == "const":
        x[:] = np.float32(-3.0)
    return x


KINDS = ["block0", "block4090", "block131000", "block261544", "scatter", "below_top",
         "bf16_fine", "bf16_coarse", "few", "const"]


def check(x, n, k, what, ws=None):
    pad = np.full((1, N), np.inf, np.float32)
    pad[0, :n] = x[:n]
    s = torch.from_numpy(pad).to(DEV)[:, :n]
    l = torch.tensor([n], dtype=torch.int32, device=DEV)
    out = ltk.lt_topk_run(s, l, k, ws=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0]
    want = oracle.topk(pad[:, :n], np.array([n], np.int32), k, nthreads=NTH)[0]
    m = int(np.sum(want >= 0))
    assert np.all(got[m:] == -1), (what, "padding")
    if not np.array_equal(np.sort(got[:m]), np.sort(want[:m])):
        raise AssertionError("%s: %d of %d differ" % (what, len(np.setdiff1d(want[:m], got[:m])), m))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("k", [512, 1024, 2048])
@pytest.mark.parametrize("n", [N, 100003])
@pytest.mark.parametrize("mode", ["never", "always"])
def test_tied_rows(kind, k, n, mode):
    prev = ltk.lt_debug_force_sample({"never": ltk.SAMPLE_NEVER, "always": ltk.SAMPLE_ALWAYS}[mode])
    try:
        check(tied_row(kind, n, 7), n, k, "%s n=%d k=%d %s" % (kind, n, k, mode))
    finally:
        ltk.lt_debug_force_sample(prev)


@pytest.mark.parametrize("kind", ["block0", "scatter", "below_top", "bf16_fine"])
def test_tied_rows_mode_word(kind):
    """Four calls sharing a workspace, so the mode word moves between the
    threshold modes as the calls go."""
    ws = ltk.workspace(ltk.lt_topk_workspace_bytes(1, N, 512), DEV)
    x = tied_row(kind, N, 11)
    for call in range(4):
        check(x, N, 512, "%s call %d" % (kind, call), ws=ws)


def test_graph_replays_tied_rows():
    """30 replays of one captured call on the split path, three rows copied
    in turn (tied sinks, bf16 ties, spread scores), so the mode word moves
    between the threshold modes across replays; every replay is checked."""
    rows = [tied_row("block0", N, 21), tied_row("bf16_fine", N, 22), tied_row("none", N, 23)]
    want = [np.sort(oracle.topk(r[None, :], np.array([N], np.int32), 512, nthreads=NTH), axis=1)
            for r in rows]
    src = [torch.from_numpy(r[None, :].copy()).to(DEV) for r in rows]
    s = src[0].clone()
    l = torch.tensor([N], dtype=torch.int32, device=DEV)
    out = torch.empty((1, 512), dtype=torch.int32, device=DEV)
    ws = torch.zeros(ltk.lt_topk_workspace_bytes(1, N, 512), dtype=torch.uint8, device=DEV)
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
    for rep in range(30):
        j = rep % 3
        s.copy_(src[j])
        out.fill_(-7)
        g.replay()
        got = np.sort(out.cpu().numpy(), axis=1)
        if not np.array_equal(got, want[j]):
            raise AssertionError("replay %d (row %d) differs from the oracle" % (rep, j))
