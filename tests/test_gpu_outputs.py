"""GPU parity of the output variants (lt_topk_order, lt_gather_rows) against
oracle/outputs.py, exact: indices element by element, values and gathered
bytes bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import outputs
import topk_index_selection_amd as ltk
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NTH = 16
ALPHABET = np.array([np.nan, -np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], np.float32)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def mixed_rows(B, n, seed):
    """Half the rows tie-heavy (special values), half N(0,1) with NaN/-0 sprinkled."""
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((B, n)).astype(np.float32)
    s[rng.random((B, n)) < 0.01] = np.nan
    s[rng.random((B, n)) < 0.01] = -0.0
    t = ALPHABET[rng.integers(0, len(ALPHABET), (B, n))]
    s[::2] = t[::2]
    return s


def random_slots(B, k, n, seed):
    rng = np.random.default_rng(seed)
    out = np.full((B, k), -1, np.int32)
    for r in range(B):
        m = int(rng.integers(0, k + 1))
        out[r, :m] = (rng.permutation(n + 3)[:m] - 1)[:m]
    return out


def bits_equal(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("k", [1, 7, 128, 129, 512, 2048, 4096])
@pytest.mark.parametrize("how", [ltk.LT_ORDER_ASIS, ltk.LT_ORDER_INDEX, ltk.LT_ORDER_RANK])
def test_order_of_selections(k, how):
    """The real use: reorder lt_topk_run's output and read the values."""
    B, n = 12, 9000
    s = mixed_rows(B, n, k)
    lens = np.random.default_rng(k + 1).integers(0, n + 1, B).astype(np.int32)
    lens[0], lens[1] = n, 3
    sd = to_dev(s)
    idx = ltk.lt_topk_run(sd, to_dev(lens), k)
    sel = idx.cpu().numpy()
    idx, vals = ltk.lt_topk_order(idx, how, scores=sd, vals=True)
    torch.cuda.synchronize()
    want = outputs.order(s, sel, how, n)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    assert bits_equal(vals.cpu().numpy(), outputs.values(s, want, n))
    if how == ltk.LT_ORDER_RANK:
        # in selection order a row's top-k is exactly the oracle's output
        np.testing.assert_array_equal(want, oracle.topk(s, lens, k, nthreads=NTH))


@pytest.mark.parametrize("k", [5, 300, 2048])
@pytest.mark.parametrize("how", [ltk.LT_ORDER_INDEX, ltk.LT_ORDER_RANK])
@pytest.mark.parametrize("with_vals", [False, True])
def test_order_of_arbitrary_slots(k, how, with_vals):
    """Slots with -1, out-of-range ids and any order."""
    B, n = 9, 5000
    s = mixed_rows(B, n, 7 * k)
    sl = random_slots(B, k, n, k)
    idx = to_dev(sl)
    r = ltk.lt_topk_order(idx, how, scores=to_dev(s), vals=with_vals)
    torch.cuda.synchronize()
    want = outputs.order(s, sl, how, n)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    if with_vals:
        assert bits_equal(r[1].cpu().numpy(), outputs.values(s, want, n))


def test_index_order_needs_no_scores():
    sl = random_slots(6, 40, 100, 3)
    idx = to_dev(sl)
    ltk.lt_topk_order(idx, ltk.LT_ORDER_INDEX, n_max=100)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), outputs.order(None, sl, outputs.ORDER_INDEX, 100))


def test_asis_values_keep_slots():
    B, n, k = 5, 700, 64
    s = mixed_rows(B, n, 4)
    sl = random_slots(B, k, n, 5)
    idx = to_dev(sl)
    _, v = ltk.lt_topk_order(idx, ltk.LT_ORDER_ASIS, scores=to_dev(s), vals=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), sl)
    assert bits_equal(v.cpu().numpy(), outputs.values(s, sl, n))


def test_order_on_prefill_rows():
    """Sampled rows of the causal prefill batch: select, then selection order with values."""
    w = workloads.cfg5(rows=np.arange(0, 8192, 512))
    sd = to_dev(w.scores)
    idx = ltk.lt_topk_run(sd, to_dev(w.lengths), 512)
    idx, v = ltk.lt_topk_order(idx, ltk.LT_ORDER_RANK, scores=sd, vals=True)
    torch.cuda.synchronize()
    want = oracle.topk(w.scores, w.lengths, 512, nthreads=NTH)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    assert bits_equal(v.cpu().numpy(), outputs.values(w.scores, want, w.n_max))


@pytest.mark.parametrize("row_elems", [8, 24, 576])
@pytest.mark.parametrize("per_row", [False, True])
def test_gather_rows(row_elems, per_row):
    rng = np.random.default_rng(row_elems)
    B, k, n_kv = 6, 512, 3000
    shape = (B, n_kv, row_elems) if per_row else (n_kv, row_elems)
    kv = rng.integers(0, 1 << 16, shape).astype(np.uint16)
    sl = random_slots(B, k, n_kv, row_elems + 1)
    out = ltk.lt_gather_rows(to_dev(kv.view(np.int16)), to_dev(sl), per_row=per_row)
    torch.cuda.synchronize()
    want = outputs.gather_rows(kv, sl, n_kv, per_row)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)


def test_gather_rows_strided_cache():
    """Cache rows wider than what is gathered: kv_stride > row_bytes."""
    rng = np.random.default_rng(11)
    full = rng.integers(0, 1 << 31, (4000, 40)).astype(np.int32)
    sl = random_slots(3, 100, 4000, 12)
    kvd = to_dev(full)[:, :16]                      # 64 of 160 bytes per row
    out = ltk.lt_gather_rows(kvd, to_dev(sl))
    torch.cuda.synchronize()
    want = outputs.gather_rows(np.ascontiguousarray(full[:, :16]), sl, 4000)
    np.testing.assert_array_equal(out.cpu().numpy(), want)


def test_gather_many_rows():
    """More batch rows than one launch's grid height (65535)."""
    B, k, n_kv = 70000, 3, 50
    rng = np.random.default_rng(13)
    kv = rng.integers(0, 1 << 31, (n_kv, 4)).astype(np.int32)
    sl = rng.integers(-2, n_kv + 2, (B, k)).astype(np.int32)
    out = ltk.lt_gather_rows(to_dev(kv), to_dev(sl))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), outputs.gather_rows(kv, sl, n_kv))


def test_select_order_gather_pipeline():
    """Selection, ascending order, cache gather: the consumer's full input."""
    w = workloads.cfg3("a")
    sd = to_dev(w.scores)
    rng = np.random.default_rng(17)
    kv = rng.integers(0, 1 << 16, (w.n_max, 576)).astype(np.uint16)
    idx = ltk.lt_topk_run(sd, to_dev(w.lengths), 512)
    ltk.lt_topk_order(idx, ltk.LT_ORDER_INDEX, n_max=w.n_max)
    out = ltk.lt_gather_rows(to_dev(kv.view(np.int16)), idx)
    torch.cuda.synchronize()
    sel = outputs.order(None, oracle.topk(w.scores, w.lengths, 512, nthreads=NTH),
                        outputs.ORDER_INDEX, w.n_max)
    np.testing.assert_array_equal(idx.cpu().numpy(), sel)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), outputs.gather_rows(kv, sel, w.n_max))
