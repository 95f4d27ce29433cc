"""Stored values: the pages' constants, and oracle regression fixtures.

``page_constants.json`` holds the numbers the pages state (with citations);
the synthetic workloads must use them. The ``*_topk512.txt`` files were written
by ``tests/golden/make_golden.py`` (oracle + seeded inputs only); the oracle
must still reproduce them.
"""
import json
import os

import numpy as np

import oracle
import workloads

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_rows(name):
    rows = []
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([int(v) for v in line.split()])
    return np.array(rows, dtype=np.int64)


def test_workloads_use_page_constants():
    with open(os.path.join(HERE, "page_constants.json")) as f:
        c = json.load(f)
    assert workloads.K_SELECT == c["k_select"]["value"]
    assert workloads.K_BLOCKS == c["k_blocks"]["value"]
    assert workloads.BLOCK_SIZE == c["block_size"]["value"]
    assert workloads.COMPRESS == c["compression"]["value"]
    assert workloads.CTX_TOKENS == c["context_tokens"]["value"]
    assert workloads.N_LONG == c["context_tokens"]["value"] // c["compression"]["value"]
    # the causal prefill rows end at the last token of the 1M context
    lens = workloads.cfg5_lengths()
    assert workloads.CFG5_FIRST_POS + workloads.CFG5_B - 1 == c["context_tokens"]["value"] - 1
    assert lens.max() == (c["context_tokens"]["value"] - 1) // c["compression"]["value"]
    assert abs(c["pytorch_topk_us"]["value"] / c["lightning_topk_us"]["value"] - c["speedup"]["value"]) < 0.05


def test_oracle_reproduces_cfg1_golden():
    w = workloads.cfg1()
    got = np.sort(oracle.topk(w.scores, w.lengths, w.k), axis=1)
    assert np.array_equal(got, load_rows("cfg1_topk512.txt"))


def test_oracle_reproduces_cfg3b_small_golden():
    w = workloads.cfg3("b", n=20000)
    got = np.sort(oracle.topk(w.scores, w.lengths, w.k), axis=1)
    assert np.array_equal(got, load_rows("cfg3b_small_topk512.txt"))
