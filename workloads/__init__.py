"""Seeded synthetic inputs for CSA indexer top-k selection.

This module is shared by the oracle side (tests, CPU baseline) and the GPU side
(tests, benchmark). It holds NO selection arithmetic: it only draws scores,
lengths and candidate-free layouts from fixed seeds.

Every row's scores come from ``numpy.random.Generator(PCG64(SeedSequence((cfg,
row))))``; lengths and permutations come from the separate stream
``SeedSequence((cfg, 65536 + j))``. i.i.d. N(0, 1) fp32 scores stand in for
real indexer scores (those would need trained weights and FP4 indexer inputs,
neither of which exists here).

Workload shapes follow the pages:

* k = 512 positions per index-source layer; 2048 candidate blocks of 8
  positions ("SGLang 与 Miles 为 DeepSeek-V4.1 提供首日支持", xhh.club, Q&A on
  cross-layer sharing);
* CSA keeps one compressed position per 4 tokens, position = token position
  divided by 4 (AICon 2026 Shenzhen speaker page, aicon.infoq.cn, abstract and
  outline 二.1); a 1M-token context therefore gives 2**20 / 4 = 262144
  positions (talk notes on devpress.csdn.net, section 3.2, measure top-k at a
  1M-token context and batch size 1).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import hashlib
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

K_SELECT = 512            # positions per index-source layer
K_BLOCKS = 2048           # shared candidate blocks
BLOCK_SIZE = 8            # positions per candidate block
COMPRESS = 4              # CSA: one compressed position per 4 tokens
CTX_TOKENS = 1 << 20      # "1M-token context"
N_LONG = CTX_TOKENS // COMPRESS   # 262144 compressed positions

LEN_STREAM = 65536        # offset of the non-score random streams


def row_rng(cfg: int, row: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence((cfg, row))))


def aux_rng(cfg: int, j: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence((cfg, LEN_STREAM + j))))


def normal_row(cfg: int, row: int, n: int) -> np.ndarray:
    return row_rng(cfg, row).standard_normal(n, dtype=np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even) and widen back to fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    scores: np.ndarray          # [B, n_max] float32, C-contiguous
    lengths: np.ndarray         # [B] int32
    k: int
    kb: int = 0                 # > 0: two-stage (blocks of bs, then top-k)
    bs: int = 1
    rows: Optional[np.ndarray] = None   # global row ids when only a subset was drawn
    description: str = ""

    @property
    def B(self) -> int:
        return int(self.scores.shape[0])

    @property
    def n_max(self) -> int:
        return int(self.scores.shape[1])

    def sha256(self) -> str:
        h = hashlib.sha256()
        h.update(np.ascontiguousarray(self.scores).view(np.uint8).reshape(-1)[: 1 << 26])
        h.update(self.lengths.tobytes())
        return h.hexdigest()[:16]


def _fill_rows(out: np.ndarray, cfg: int, rows: Sequence[int], lengths: np.ndarray,
               poison: Optional[float], threads: int) -> None:
    n = out.shape[1]

    def one(j):
        r = int(rows[j])
        out[j, :] = normal_row(cfg, r, n)
        if poison is not None:
            out[j, int(lengths[j]):] = poison

    if threads > 1 and len(rows) > 1:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(len(rows))))
    else:
        for j in range(len(rows)):
            one(j)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def cfg1(n: int = 4096, k: int = K_SELECT) -> Workload:
    """Single row, N = 4096, all valid, k = 512."""
    s = normal_row(1, 0, n)[None, :].copy()
    return Workload("cfg1_single_4096", s, np.array([n], np.int32), k,
                    description="B=1, N=4096, N(0,1), k=512, all valid")


def cfg2_lengths(B: int = 64, n_max: int = 32768, lo: int = 256) -> np.ndarray:
    lens = aux_rng(2, 0).integers(lo, n_max, size=B, endpoint=True).astype(np.int32)
    forced = [256, 511, 512, 513, n_max]
    for j, v in enumerate(forced[:B]):
        lens[j] = min(v, n_max)
    return lens


def cfg2(B: int = 64, n_max: int = 32768, k: int = K_SELECT) -> Workload:
    """Decode batch: B rows, uniform length in [256, n_max], +inf beyond length."""
    lens = cfg2_lengths(B, n_max, min(256, n_max))
    s = np.empty((B, n_max), np.float32)
    _fill_rows(s, 2, range(B), lens, np.inf, _threads())
    return Workload("cfg2_decode_64x32768", s, lens, k,
                    description="B=64, Nmax=32768, len~U[256,32768] (rows 0-4 forced to "
                                "256,511,512,513,32768), N(0,1), +inf poison beyond len")


def cfg3(variant: str = "a", n: int = N_LONG, k: int = K_SELECT) -> Workload:
    """1M-token context at batch size 1: one row of 262144 positions."""
    s = normal_row(3, 0, n)
    if variant == "b":
        s = round_to_bf16(s)
    elif variant == "c":
        n_inf = n - int(np.floor(0.1 * n))
        perm = aux_rng(3, 2).permutation(n)
        s = s.copy()
        s[perm[:n_inf]] = -np.inf
    elif variant != "a":
        raise ValueError(variant)
    desc = {"a": "N(0,1)", "b": "N(0,1) rounded to bf16 (heavy ties)",
            "c": "N(0,1) with 90% -inf"}[variant]
    return Workload("cfg3%s_bs1_262144" % variant, s[None, :].copy(),
                    np.array([n], np.int32), k, description="B=1, N=262144, k=512, " + desc)


def clustered(pattern: str, n: int = N_LONG, k: int = K_SELECT) -> Workload:
    """One row of N(0,1) scores shaped the way attention scores cluster:
    'recent' adds 4 to the last 16384 positions (a hot recent window), 'ramp'
    adds 2 (i/n)^4 (scores rising toward the present), 'sinks' sets the first
    600 positions to 10.0 (tied attention sinks at the start)."""
    s = normal_row(6, {"recent": 0, "ramp": 1, "sinks": 2}[pattern], n)
    i = np.arange(n)
    if pattern == "recent":
        s = s + np.float32(4.0) * (i >= n - 16384)
    elif pattern == "ramp":
        s = s + np.float32(2.0) * (i / n) ** 4
    else:
        s = np.where(i < 600, np.float32(10.0), s)
    return Workload("clustered_%s_%d" % (pattern, n), s.astype(np.float32)[None, :].copy(),
                    np.array([n], np.int32), k,
                    description="B=1, N=%d, k=%d, clustered (%s)" % (n, k, pattern))


def cfg4(B: int = 1, n: int = N_LONG, k: int = K_SELECT, kb: int = K_BLOCKS,
         bs: int = BLOCK_SIZE) -> Workload:
    """Two-stage shared candidates: top-2048 blocks of 8, then top-512 inside."""
    s = np.empty((B, n), np.float32)
    lens = np.full(B, n, np.int32)
    _fill_rows(s, 4, range(B), lens, None, _threads())
    return Workload("cfg4_twostage_B%d_262144" % B, s, lens, k, kb=kb, bs=bs,
                    description="B=%d, N=262144, blocks of 8 scored by max, top-2048 blocks "
                                "then top-512 inside them" % B)


CFG5_B = 8192
CFG5_FIRST_POS = 1_040_384


def cfg5_lengths(B: int = CFG5_B, first_pos: int = CFG5_FIRST_POS) -> np.ndarray:
    pos = first_pos + np.arange(B, dtype=np.int64)
    return (pos // COMPRESS).astype(np.int32)


def cfg5(rows: Optional[Sequence[int]] = None, n_max: int = N_LONG, k: int = K_SELECT,
         out: Optional[np.ndarray] = None) -> Workload:
    """Causal prefill: 8192 query rows at token positions 1,040,384 ... 1,048,575.

    Row i has valid length floor(pos_i / 4) over n_max = 262144 positions, +inf
    beyond it. ``rows`` draws only the listed rows (same values as in the full
    batch); ``out`` lets a caller supply the [len(rows), n_max] buffer.
    """
    all_lens = cfg5_lengths()
    rows_arr = np.arange(CFG5_B) if rows is None else np.asarray(rows, dtype=np.int64)
    lens = all_lens[rows_arr].astype(np.int32)
    s = out if out is not None else np.empty((len(rows_arr), n_max), np.float32)
    _fill_rows(s, 5, rows_arr, lens, np.inf, _threads())
    return Workload("cfg5_prefill_8192x262144", s, lens, k,
                    rows=None if rows is None else rows_arr,
                    description="B=8192, Nmax=262144, len=floor(pos/4), pos=1040384+i, "
                                "N(0,1), +inf poison beyond len, k=512")


def cfg5_ramp(rows: Optional[Sequence[int]] = None, n_max: int = N_LONG,
              k: int = K_SELECT) -> Workload:
    """The causal prefill batch with near-monotone rows rising toward the
    present: row r holds i / len_r + 2**-12 * z_i at position i (z_i N(0, 1)
    from the row's own stream, cfg 7), +inf past len_r. The trend grows by
    1/len per position and the noise spans a few hundred positions of it, so
    read in index order nearly every score would enter the row's running
    top-512; attention scores that favour recent positions lean this way."""
    all_lens = cfg5_lengths()
    rows_arr = np.arange(CFG5_B) if rows is None else np.asarray(rows, dtype=np.int64)
    lens = all_lens[rows_arr].astype(np.int32)
    s = np.empty((len(rows_arr), n_max), np.float32)
    i = np.arange(n_max, dtype=np.float32)

    def one(j):
        L = int(lens[j])
        z = normal_row(7, int(rows_arr[j]), n_max)
        s[j, :] = i / np.float32(L) + np.float32(2.0 ** -12) * z
        s[j, L:] = np.inf

    with _cf.ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(one, range(len(rows_arr))))
    return Workload("cfg5_prefill_rising_ramp_8192x262144", s, lens, k,
                    rows=None if rows is None else rows_arr,
                    description="B=8192, Nmax=262144, len=floor(pos/4), i/len + 2^-12 N(0,1), "
                                "+inf poison beyond len, k=512")


CONFIGS: Dict[str, callable] = {
    "cfg1": cfg1,
    "cfg2": cfg2,
    "cfg3a": lambda: cfg3("a"),
    "cfg3b": lambda: cfg3("b"),
    "cfg3c": lambda: cfg3("c"),
    "cfg4b1": lambda: cfg4(1),
    "cfg4b32": lambda: cfg4(32),
    "cfg5": cfg5,
}


def make(name: str) -> Workload:
    return CONFIGS[name]()


def small_variants() -> List[Workload]:
    """Scaled-down versions of the five workloads (same recipes, small sizes)."""
    out = [cfg1(), cfg2(B=12, n_max=3000), cfg3("a", n=20000), cfg3("b", n=20000),
           cfg3("c", n=20000), cfg4(B=2, n=16384, kb=256, k=64)]
    w5 = cfg5(rows=[0, 1, 4095, 8191])
    w5 = Workload("cfg5_rows", w5.scores[:, :65536].copy(),
                  np.minimum(w5.lengths, 65536 - 3 * np.arange(4, dtype=np.int32)), 512,
                  description="cfg5 rows truncated to 65536")
    out.append(w5)
    return out
