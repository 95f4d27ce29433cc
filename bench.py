#!/usr/bin/env python3
"""Benchmark of CSA indexer top-k selection on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline step: one lt_topk_run over the causal prefill batch -- 8192 query
rows at token positions 1,040,384 ... 1,048,575 of a 1M-token context, row i
valid up to floor(pos_i / 4) of 262,144 compressed positions, k = 512 -- with
the scores already resident in HBM. ``value`` is rows/s over the K timed
steps. The same run also reports, as latency (µs per call against an empty
kernel launched the same way):
  * batch size 1 at 262,144 positions (i.i.d., bf16-rounded, 90 % -inf);
  * the decode batch (64 rows up to 32,768 positions);
  * the two-stage shared-candidate selection (top-2048 blocks of 8, then
    top-512 inside) at batch 1 and 32.
Every number is printed only after the same run's results were checked
against the CPU oracle, every row of every configuration (the gathered cache
rows of the prefill batch on 256 rows). ``cpu_baseline`` is the wall time of
the oracle call that checked the prefill batch: all 8192 rows on up to 16
host threads, with the host's CPU count and model.

Output: one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per top-512 at N=262144 BS=1; prefill rows/s; HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "topk_index_selection_amd", "csrc", "ltopk_kernels.hip")
OUTPUT_SRC = os.path.join(ROOT, "topk_index_selection_amd", "csrc", "ltopk_output.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "stream_kernel_prefill_8192x262144_traffic.txt")
TRAFFIC_FILE_BLOCKS = os.path.join(ROOT, "profiles",
                                   "stream_kernel_blocks_prefill_8192x262144_traffic.txt")
TRAFFIC_FILE_CAND = os.path.join(ROOT, "profiles",
                                 "stream_kernel_candidates_prefill_8192x2048x8_traffic.txt")
TRAFFIC_FILE_ORDER = os.path.join(ROOT, "profiles", "order_kernel_prefill_8192x512_traffic.txt")
TRAFFIC_FILE_BS1 = os.path.join(ROOT, "profiles", "split_kernel_bs1_262144_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(path: str = KERNEL_SRC) -> str:
    """Hash of the device part of a kernel source (everything above its
    host-side section), so host-only edits keep the counters current."""
    with open(path, "rb") as f:
        src = f.read()
    cut = src.find(b"// ------------------------------------------------------------------ host side")
    return hashlib.sha256(src if cut < 0 else src[:cut]).hexdigest()[:16]


def read_traffic(path, src=KERNEL_SRC):
    """HBM bytes per launch measured by rocprofv3 counters, if they are still
    current (the file records the hash of the kernel source it was taken on)."""
    try:
        with open(path) as f:
            vals = {}
            for line in f:
                if line.startswith("#") or "=" not in line:
                    continue
                key, v = line.split("=", 1)
                vals[key.strip()] = v.strip()
        if vals.get("kernel_source_sha256_16") != src_hash(src):
            return None
        return int(float(vals["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def throughput(nbytes: int, rows: int, us: float) -> dict:
    """Per-call figures of a latency configuration from its algorithmic bytes."""
    return {"us_per_row": round(us / rows, 3), "rows_per_s": round(rows / us * 1e6, 1),
            "algorithmic_bytes": int(nbytes), "GBps": round(nbytes / us / 1e3, 1),
            "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}


def algorithmic_bytes(lengths: np.ndarray, k: int) -> int:
    """Scores read once (4 B per valid position), indices written, lengths read."""
    return int(4 * np.sum(lengths.astype(np.int64)) + 4 * k * len(lengths) + 4 * len(lengths))


def check_sets(got: np.ndarray, want: np.ndarray, what: str):
    for r in range(want.shape[0]):
        m = int(np.sum(want[r] >= 0))
        if not (np.all(got[r][m:] == -1)
                and np.array_equal(np.sort(got[r][:m]), np.sort(want[r][:m]))):
            raise SystemExit("PARITY FAILURE in %s row %d: no numbers reported" % (what, r))


def host_info(nthreads: int) -> dict:
    """The host the CPU oracle runs on: logical CPUs, the ones this process may
    use, the CPU model, and the threads the oracle is given."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"host_logical_cpus": os.cpu_count(), "usable_cpus": usable, "cpu_model": model,
            "threads_used": nthreads}


def oracle_threads() -> int:
    """Threads for the CPU oracle: the CPUs this process may use, at most 16 (a
    one-GPU share of the GPU host's CPUs)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return max(1, min(16, usable))


def same_sets_all(got: np.ndarray, want: np.ndarray) -> bool:
    """Every row's index set (and its count of -1 slots) equal: rows compared
    sorted, all at once."""
    return got.shape == want.shape and np.array_equal(np.sort(got, axis=1), np.sort(want, axis=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="do not report the oracle's time as the CPU baseline")
    ap.add_argument("--check-rows", type=int, default=None,
                    help="prefill rows checked against the oracle (default: all 8192); "
                         "profiler runs may check fewer, and say so in the output")
    ap.add_argument("--parts", default="prefill,two_stage,outputs,ramp,latency",
                    help="comma-separated parts to run: prefill (always), two_stage, outputs, "
                         "ramp, latency")
    ap.add_argument("--no-extra", action="store_true", help="only the prefill batch")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain copy kernel of 1 GiB (counter calibration)")
    ap.add_argument("--latency-only", default=None, metavar="NAMES",
                    help="comma-separated latency entries (e.g. bs1_262144_iid) run alone, "
                         "for a profile of one configuration; prints them as one JSON line")
    ap.add_argument("--latency-light", action="store_true",
                    help="few repetitions in the latency timings (for counter collection, "
                         "where every launch is serialised)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(rows of a batch are independent, so N GPUs would each run their own share). "
              "Got --gpus %d." % args.gpus, file=sys.stderr)
        sys.exit(2)
    parts = set(args.parts.split(",")) | {"prefill"}
    if args.no_extra:
        parts = {"prefill"}

    import torch
    import topk_index_selection_amd as ltk
    import workloads
    import oracle

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ltk.load_library()
    stream = torch.cuda.current_stream()
    nthreads = oracle_threads()
    if args.latency_light:
        REPS.update(calls=10, replays=2, trials=1, eager=20, cold=2)
    if args.latency_only:
        only = set(args.latency_only.split(","))
        out = {"latency_us": latency_suite(torch, ltk, workloads, oracle, nthreads, only)}
        if args.latency_light:
            out["latency_reps"] = dict(REPS)
        if args.calib_copy:
            out["calib_copy_bytes_each_way"] = calib_copy(torch, dev)
        print(json.dumps(out), flush=True)
        return

    # ------------------------------------------------------------ prefill (headline)
    t0 = time.time()
    w = workloads.cfg5()
    log("prefill input generated in %.1f s (%.2f GB)" % (time.time() - t0, w.scores.nbytes / 1e9))
    B, n_max, k = w.B, w.n_max, w.k
    host_scores = w.scores            # kept: every row is checked against the oracle
    lengths_np = w.lengths.copy()
    if args.check_rows is None or args.check_rows >= B:
        check_rows = np.arange(B)
    else:
        rng = np.random.default_rng(12345)
        check_rows = np.unique(np.concatenate([[0, B // 2, B - 1],
                                               rng.choice(B, max(args.check_rows - 3, 0),
                                                          replace=False)]))
    all_rows = len(check_rows) == B
    host_check = host_scores if all_rows else host_scores[check_rows]
    t0 = time.time()
    inputs = input_digest(host_scores, lengths_np, nthreads)
    inputs["seeds"] = ("numpy PCG64, SeedSequence((5, row)) per row, standard_normal float32; "
                       "+inf past each row's length")
    log("prefill input digest in %.1f s" % (time.time() - t0))
    scores = torch.from_numpy(host_scores).to(dev)
    lengths = torch.from_numpy(lengths_np).to(dev)
    out = torch.empty((B, k), dtype=torch.int32, device=dev)
    ws = ltk.workspace(ltk.lt_topk_workspace_bytes(B, n_max, k), dev)

    def step():
        ltk.lt_topk_run(scores, lengths, k, out=out, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    wall_ms = (t_end - t_start) * 1e3 / args.steps
    launch_ms = e0.elapsed_time(e1) / args.steps
    got = out.cpu().numpy()
    # The oracle over the checked rows (by default the whole batch), timed: the
    # same run is the CPU baseline.
    t0 = time.perf_counter()
    want = oracle.topk(host_check, lengths_np[check_rows], k, nthreads=nthreads)
    oracle_s = time.perf_counter() - t0
    if not same_sets_all(got[check_rows], want):
        check_sets(got[check_rows], want, "prefill")   # names the first differing row
        raise SystemExit("PARITY FAILURE in prefill: no numbers reported")
    log("prefill: %.3f ms/step wall, %.3f ms per launch (events), parity ok on %d of %d rows "
        "(oracle %.1f s on %d threads)"
        % (wall_ms, launch_ms, len(check_rows), B, oracle_s, nthreads))

    alg = algorithmic_bytes(lengths_np, k)
    achieved = alg / (launch_ms * 1e-3) / 1e9
    rows_per_s = B / (wall_ms * 1e-3)
    traffic = read_traffic(TRAFFIC_FILE)

    result = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill: 8192 rows x 262144 fp32 scores N(0,1), "
                        "len=floor(pos/4) for pos 1040384..1048575, k=512",
            "rows": B, "n_max": n_max, "k": k,
            "kernel": "stream_kernel: one wave per row, fp32 threshold test, 1024-slot LDS buffer with a 256-bin key histogram",
        },
        "parity": {"rows_checked": int(len(check_rows)), "rows": B,
                   "rule": "index sets equal to the CPU oracle's, row by row (sorted)"},
        "inputs": inputs,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": alg,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = {
            "value": round(len(check_rows) / oracle_s, 2),
            "unit": "rows/s",
            "cores": nthreads,
            "kind": "oracle",
            "sample": "%d of the %d prefill rows (%s), %.1f s wall on %d host threads: the "
                      "sort-based C oracle, the same call that checked this run's parity"
                      % (len(check_rows), B, "the whole batch" if all_rows else "sampled",
                         oracle_s, nthreads),
            **host_info(nthreads),
        }
        log("cpu baseline: %.1f rows/s on %d threads" % (len(check_rows) / oracle_s, nthreads))

    # ------------------------------------------------------------ two-stage on the prefill batch
    # The shared-candidate data flow with independent rows: the blocks of row
    # i-1's scores (standing in for another layer) restrict row i.
    if "two_stage" in parts:
        s1 = torch.roll(scores, 1, dims=0)
        l1 = torch.roll(lengths, 1, dims=0)
        blocks = torch.empty((B, 2048), dtype=torch.int32, device=dev)
        out2 = torch.empty((B, k), dtype=torch.int32, device=dev)

        def stage1():
            ltk.lt_topk_blocks(s1, l1, 8, 2048, out=blocks, ws=ws)

        def stage2():
            ltk.lt_topk_run(scores, lengths, k, cand=(blocks, 8), out=out2, ws=ws)

        def two_stage():
            stage1()
            stage2()

        for _ in range(2):
            two_stage()
        torch.cuda.synchronize()
        reps = max(3, args.steps // 2)
        ms2 = time_events(torch, stream, two_stage, reps)
        ms_b = time_events(torch, stream, stage1, reps)
        ms_c = time_events(torch, stream, stage2, reps)
        # oracle: blocks of every row, then each row restricted to the previous row's blocks
        wb_own = oracle.topk_blocks(host_check, lengths_np[check_rows], 8, 2048, nthreads=nthreads)
        got_b = blocks.cpu().numpy()
        if all_rows:
            wb = np.roll(wb_own, 1, axis=0)
            ok_b = same_sets_all(got_b, wb)
        else:
            prev = (check_rows - 1) % B
            wb = oracle.topk_blocks(host_scores[prev], lengths_np[prev], 8, 2048,
                                    nthreads=nthreads)
            ok_b = same_sets_all(got_b[check_rows], wb)
        if not ok_b:
            raise SystemExit("PARITY FAILURE in two-stage prefill blocks: no numbers reported")
        wt = oracle.topk(host_check, lengths_np[check_rows], k, cand=wb, bs=8, nthreads=nthreads)
        if not same_sets_all(out2.cpu().numpy()[check_rows], wt):
            raise SystemExit("PARITY FAILURE in two-stage prefill top-k: no numbers reported")
        # block stage: scores read once, block ids written; candidate stage: block
        # ids read, the 16384 candidate scores of each row gathered, indices written
        byt_b = alg - 4 * k * B + 4 * 2048 * B
        byt_c = 4 * 2048 * B + B * (16384 * 4) + 4 * k * B + 4 * B
        byt = byt_b + byt_c
        tb, tc = read_traffic(TRAFFIC_FILE_BLOCKS), read_traffic(TRAFFIC_FILE_CAND)
        result["two_stage_prefill"] = {
            "workload": "blocks of row i-1 (top-2048 of 8) restrict row i's top-512, 8192 "
                        "prefill rows",
            "ms": round(ms2, 4), "rows_per_s": round(B / (ms2 * 1e-3), 1),
            "algorithmic_bytes": int(byt), "GBps": round(byt / (ms2 * 1e-3) / 1e9, 1),
            # measured HBM bytes of both stages (counters) and their ratio to
            # the algorithmic bytes; the candidates' 32-byte gathers cost whole
            # lines
            "traffic": tb + tc if tb is not None and tc is not None else None,
            "traffic_ratio": round((tb + tc) / byt, 4) if tb is not None and tc is not None else None,
            "rows_checked": int(len(check_rows)),
            "block_stage": {"ms": round(ms_b, 4), "algorithmic_bytes": int(byt_b),
                            "GBps": round(byt_b / (ms_b * 1e-3) / 1e9, 1),
                            "frac_of_hbm_peak": round(byt_b / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": read_traffic(TRAFFIC_FILE_BLOCKS)},
            "candidate_stage": {"ms": round(ms_c, 4), "algorithmic_bytes": int(byt_c),
                                "GBps": round(byt_c / (ms_c * 1e-3) / 1e9, 1),
                                "frac_of_hbm_peak": round(byt_c / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "traffic": read_traffic(TRAFFIC_FILE_CAND)}}
        log("two-stage prefill: %.3f ms per call (block stage %.3f, candidate stage %.3f), parity "
            "ok on %d rows" % (ms2, ms_b, ms_c, len(check_rows)))
        del s1, l1, blocks, out2

    # ------------------------------------------------------------ output variants
    # What the consumer receives: the prefill selection in selection order with
    # its scores, and the selected rows of a compressed-KV cache (synthetic
    # bf16-sized rows, [262144, 576] x 2 B = 1152 B per row, one cache shared by
    # the batch's rows) gathered in ascending index order.
    if "outputs" in parts:
        from oracle import outputs as oout

        idx_r = out.clone()
        vals = torch.empty((B, k), dtype=torch.float32, device=dev)
        ms_o = time_events(torch, stream, lambda: ltk.lt_topk_order(
            idx_r, ltk.LT_ORDER_RANK, scores=scores, out_vals=vals), 10, warm=1)
        got_i = idx_r.cpu().numpy()[check_rows]
        if not np.array_equal(got_i, want):   # the oracle writes selection order
            raise SystemExit("PARITY FAILURE: selection order")
        got_v = vals.cpu().numpy()[check_rows]
        if not np.array_equal(got_v.view(np.uint32),
                              oout.values(host_check, want, n_max).view(np.uint32)):
            raise SystemExit("PARITY FAILURE: selection-order values")
        byt_o = 4 * B * k * 4  # indices read + written, scores read, values written
        result["order_rank_values_prefill"] = {
            "workload": "8192 prefill selections of 512 put in selection order with their scores",
            "us": round(ms_o * 1e3, 2), "algorithmic_bytes": byt_o,
            "GBps": round(byt_o / (ms_o * 1e-3) / 1e9, 1), "rows_checked": int(len(check_rows)),
            "traffic": read_traffic(TRAFFIC_FILE_ORDER, OUTPUT_SRC)}
        log("order (selection order + values), prefill: %.1f us per call, parity ok on %d rows"
            % (ms_o * 1e3, len(check_rows)))

        D = 576
        g = torch.Generator(device=dev)
        g.manual_seed(12345)
        kv = torch.randint(-32768, 32768, (n_max, D), dtype=torch.int16, device=dev, generator=g)
        idx_i = out.clone()
        ltk.lt_topk_order(idx_i, ltk.LT_ORDER_INDEX, n_max=n_max)
        gout = torch.empty((B, k, D), dtype=torch.int16, device=dev)
        ms_g = time_events(torch, stream, lambda: ltk.lt_gather_rows(kv, idx_i, out=gout), 5,
                           warm=1)
        sel = oout.order(None, want, oout.ORDER_INDEX, n_max)
        if not np.array_equal(idx_i.cpu().numpy()[check_rows], sel):
            raise SystemExit("PARITY FAILURE: ascending order")
        # the gathered bytes of 256 rows (4.8 GB for all rows would dwarf the run)
        grows = np.sort(np.random.default_rng(7).choice(len(check_rows), min(256, len(check_rows)),
                                                        replace=False))
        rows_t = torch.from_numpy(check_rows[grows]).to(dev)
        got_g = gout.index_select(0, rows_t).cpu().numpy()
        if not np.array_equal(got_g, oout.gather_rows(kv.cpu().numpy(), sel[grows], n_max)):
            raise SystemExit("PARITY FAILURE: cache-row gather")
        byt_g = 2 * B * k * D * 2 + 4 * B * k
        result["gather_kv_prefill"] = {
            "workload": "8192 x 512 selected rows of 1152 B from a [262144, 576] 2-byte cache",
            "ms": round(ms_g, 4), "algorithmic_bytes": byt_g,
            "GBps": round(byt_g / (ms_g * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(byt_g / (ms_g * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "rows_checked": int(len(grows))}
        log("gather of the selected cache rows, prefill: %.3f ms per call (%.0f GB/s), parity ok "
            "on %d rows" % (ms_g, byt_g / (ms_g * 1e-3) / 1e9, len(grows)))
        del idx_r, vals, kv, idx_i, gout

    del scores, out, host_check, host_scores, w
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ rising-ramp prefill batch
    # The same causal batch with near-monotone rows rising toward the present
    # (i/len + 2^-12 N(0,1)): read in index order nearly every score would
    # enter a row's running top-512.
    if "ramp" in parts:
        wr = workloads.cfg5_ramp()
        sr = torch.from_numpy(wr.scores).to(dev)
        lr = torch.from_numpy(wr.lengths).to(dev)
        outr = torch.empty((B, k), dtype=torch.int32, device=dev)
        ms_r = time_events(torch, stream, lambda: ltk.lt_topk_run(sr, lr, k, out=outr, ws=ws),
                           max(3, args.steps // 2), warm=2)
        rcheck = check_rows if not all_rows else np.arange(B)
        want_r = oracle.topk(wr.scores if all_rows else wr.scores[rcheck], wr.lengths[rcheck], k,
                             nthreads=nthreads)
        if not same_sets_all(outr.cpu().numpy()[rcheck], want_r):
            raise SystemExit("PARITY FAILURE in the rising-ramp prefill batch: no numbers reported")
        alg_r = algorithmic_bytes(wr.lengths, k)
        result["prefill_rising_ramp"] = {
            "workload": "causal prefill batch, 8192 rows of i/len + 2^-12 N(0,1) (rising toward "
                        "the present), k=512",
            "ms": round(ms_r, 4), "rows_per_s": round(B / (ms_r * 1e-3), 1),
            "algorithmic_bytes": alg_r, "GBps": round(alg_r / (ms_r * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg_r / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "rows_checked": int(len(rcheck))}
        log("rising-ramp prefill: %.3f ms per call, parity ok on %d rows" % (ms_r, len(rcheck)))
        del wr, sr, lr, outr, want_r
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ latency-bound configs
    if "latency" in parts:
        result["latency_us"] = latency_suite(torch, ltk, workloads, oracle, nthreads)

    if args.calib_copy:
        result["calib_copy_bytes_each_way"] = calib_copy(torch, dev)
    if args.latency_light:
        result["latency_reps"] = dict(REPS)

    print(json.dumps(result), flush=True)


def calib_copy(torch, dev) -> int:
    """A plain copy kernel over 1 GiB of fp32 (torch.neg), three times: the
    known byte counts that scale the HBM traffic counters."""
    n = 1 << 28
    a = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b
    return 4 * n


# Repetitions of the latency timings (bench.py --latency-light lowers them).
REPS = {"calls": 100, "replays": 20, "trials": 5, "eager": 200, "cold": 20}


def time_events(torch, stream, fn, reps, warm=0):
    """ms per call: `reps` back-to-back calls between two events on `stream`."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_graph(torch, fn, calls=None, replays=None, trials=None):
    """µs per call: `calls` calls captured in one graph, replayed; median of trials."""
    calls = REPS["calls"] if calls is None else calls
    replays = REPS["replays"] if replays is None else replays
    trials = REPS["trials"] if trials is None else trials
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    res = []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3 / (calls * replays))
    return statistics.median(res)


def time_eager(torch, fn, calls=None, trials=None):
    calls = REPS["eager"] if calls is None else calls
    trials = REPS["trials"] if trials is None else trials
    for _ in range(20):
        fn()
    torch.cuda.synchronize()
    res = []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3 / calls)
    return statistics.median(res)


def time_cold(torch, fn, reps=None):
    """µs of single calls with cold caches: before each, a 512 MiB write on the
    same stream evicts L2 and the 256 MB MALL; only the call sits between the
    events. Median over reps."""
    reps = REPS["cold"] if reps is None else reps
    scrub = torch.empty(128 << 20, dtype=torch.float32, device="cuda:0")
    res = []
    for i in range(reps):
        scrub.fill_(float(i))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3)
    del scrub
    return statistics.median(res)


def input_digest(scores, lengths, nthreads):
    """SHA-256 of the lengths, and of the scores as the SHA-256 over the
    concatenated per-row SHA-256 digests (rows hashed in parallel)."""
    from concurrent.futures import ThreadPoolExecutor
    rows = np.ascontiguousarray(scores)
    with ThreadPoolExecutor(max_workers=nthreads) as ex:
        parts = list(ex.map(lambda r: hashlib.sha256(memoryview(rows[r]).cast("B")).digest(),
                            range(rows.shape[0])))
    return {"scores_rowwise_sha256": hashlib.sha256(b"".join(parts)).hexdigest(),
            "lengths_sha256": hashlib.sha256(np.ascontiguousarray(lengths).tobytes()).hexdigest()}


def latency_suite(torch, ltk, workloads, oracle, nthreads, only=None):
    dev = torch.device("cuda:0")

    def wanted(name):
        return only is None or name in only
    res = {"timing": "graph: median of 5 trials of 20 replays of a captured graph of 100 calls; "
                     "eager: 200 back-to-back calls from Python (includes host call overhead); "
                     "floor: empty kernel with the same grid, timed the same way; inputs warm "
                     "in cache as when the indexer has just written them; cold: single calls, "
                     "each after a 512 MiB write that evicts L2 and MALL, median of 20"}

    def one(name, w, cold=False):
        if not wanted(name):
            return
        s = torch.from_numpy(w.scores).to(dev)
        l = torch.from_numpy(w.lengths).to(dev)
        o = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
        wsb = ltk.workspace(ltk.lt_topk_workspace_bytes(w.B, w.n_max, w.k), dev)

        def fn():
            ltk.lt_topk_run(s, l, w.k, out=o, ws=wsb)

        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        want = oracle.topk(w.scores, w.lengths, w.k, nthreads=nthreads)
        oracle_ms = (time.perf_counter() - t0) * 1e3
        check_sets(o.cpu().numpy(), want, name)
        g = time_graph(torch, fn)
        e = time_eager(torch, fn)
        kern, grid, block = ltk.lt_debug_launch_shape(w.B, w.n_max)
        fl = time_graph(torch, lambda: ltk.lt_debug_empty_launch(grid[0], grid[1], block))
        check_sets(o.cpu().numpy(), oracle.topk(w.scores, w.lengths, w.k, nthreads=nthreads), name)
        res[name] = {"graph_us": round(g, 2), "eager_us": round(e, 2), "floor_us": round(fl, 2),
                     "kernel": kern, "grid": list(grid), "block": block,
                     **throughput(algorithmic_bytes(w.lengths, w.k), w.B, g),
                     "oracle_ms": round(oracle_ms, 2), "oracle_threads": min(nthreads, w.B),
                     "inputs": input_digest(w.scores, w.lengths, nthreads)}
        if name == "bs1_262144_iid":
            # HBM bytes per launch from the counters (scores plus the exchange)
            res[name]["traffic"] = read_traffic(TRAFFIC_FILE_BS1)
        if cold:
            c = time_cold(torch, fn)
            check_sets(o.cpu().numpy(), oracle.topk(w.scores, w.lengths, w.k, nthreads=nthreads),
                       name)
            res[name]["cold_us"] = round(c, 2)
            log("%s: %.2f us/call cold (512 MiB scrub before each call)" % (name, c))
        log("%s: %.2f us/call (graph), %.2f us eager, floor %.2f us" % (name, g, e, fl))

    one("single_row_4096", workloads.cfg1())
    for v in "abc":
        one("bs1_262144_" + {"a": "iid", "b": "bf16_ties", "c": "90pct_neg_inf"}[v],
            workloads.cfg3(v), cold=True)
    # rows whose winners cluster, as attention scores do (recent window,
    # rising ramp, tied sinks): the split kernel's recovery path
    for pat in ("recent", "ramp", "sinks"):
        one("bs1_262144_clustered_" + pat, workloads.clustered(pat))
    w2 = workloads.cfg2()
    one("decode_64x32768", w2)

    for B in (1, 32):
        if not wanted("two_stage_B%d_262144" % B):
            continue
        w = workloads.cfg4(B)
        s = torch.from_numpy(w.scores).to(dev)
        l = torch.from_numpy(w.lengths).to(dev)
        blocks = torch.empty((B, w.kb), dtype=torch.int32, device=dev)
        o = torch.empty((B, w.k), dtype=torch.int32, device=dev)
        wsb = ltk.workspace(ltk.lt_topk_workspace_bytes(B, w.n_max, w.kb), dev)

        def fn():
            # both stages in one call (one launch where the shapes allow)
            ltk.lt_topk_two_stage(s, l, w.bs, w.kb, w.k, out_blocks=blocks, out=o, ws=wsb)

        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        wb = oracle.topk_blocks(w.scores, w.lengths, w.bs, w.kb, nthreads=nthreads)
        wt = oracle.topk(w.scores, w.lengths, w.k, cand=wb, bs=w.bs, nthreads=nthreads)
        oracle_ms = (time.perf_counter() - t0) * 1e3
        check_sets(blocks.cpu().numpy(), wb, "two-stage blocks")
        check_sets(o.cpu().numpy(), wt, "two-stage top-k")
        g = time_graph(torch, fn)
        e = time_eager(torch, fn)
        name = "two_stage_B%d_262144" % B
        # scores read once by the block stage, its block ids written and read
        # back, the candidates' scores gathered, indices written, lengths read
        nb = (w.lengths.astype(np.int64) + w.bs - 1) // w.bs
        ab = int(np.sum(4 * w.lengths.astype(np.int64) + 2 * 4 * w.kb
                        + 4 * np.minimum(nb, w.kb) * w.bs + 4 * w.k + 2 * 4))
        res[name] = {"graph_us": round(g, 2), "eager_us": round(e, 2), **throughput(ab, B, g),
                     "oracle_ms": round(oracle_ms, 2), "oracle_threads": min(nthreads, B)}
        log("%s: %.2f us/call (graph), %.2f us eager" % (name, g, e))
        del s, l, blocks, o

    # the entries below run together, when any of them is asked for
    if only is not None and not only & {"layer_loop_60x_bs1_262144", "cp8_shard_merge_262144",
                                        "order_rank_values_bs1_512", "gather_kv_bs1_512x1152B"}:
        return res

    # One token's selections across the layers of a model: 60 top-512 calls
    # over 60 different rows of ~260K valid scores (prefill rows 0..59), one
    # graph (the talk notes' 100 us x 60 layers framing).
    L = 60
    wl = workloads.cfg5(rows=np.arange(L))
    lens = wl.lengths
    sl = torch.from_numpy(wl.scores).to(dev)
    ll = torch.from_numpy(lens).to(dev)
    lo = torch.empty((L, 512), dtype=torch.int32, device=dev)
    wsl = ltk.workspace(ltk.lt_topk_workspace_bytes(1, 262144, 512), dev)
    views = [(sl[i:i + 1], ll[i:i + 1], lo[i:i + 1]) for i in range(L)]

    def layers():
        for sv, lv, ov in views:
            ltk.lt_topk_run(sv, lv, 512, out=ov, ws=wsl)

    layers()
    torch.cuda.synchronize()
    check_sets(lo.cpu().numpy(), oracle.topk(wl.scores, lens, 512, nthreads=nthreads), "layer loop")
    g = time_graph(torch, layers, calls=1)
    res["layer_loop_60x_bs1_262144"] = {"graph_us_per_token": round(g, 2),
                                        "us_per_layer": round(g / L, 2)}
    log("layer loop: %.1f us per token for %d layers (%.2f us per layer)" % (g, L, g / L))
    del sl, ll, lo

    # Context-parallel shard merge on one GPU: 8 shards of 32768 positions
    # (local top-512 each, global offsets), then the top-512 of the 4096
    # candidates (candidate form, block size 1).
    w = workloads.cfg3("a")
    n, P = w.n_max, 8
    row = torch.from_numpy(w.scores[0]).to(dev)
    shards = row.view(P, n // P)
    slen = torch.full((P,), n // P, dtype=torch.int32, device=dev)
    rlen = torch.from_numpy(w.lengths).to(dev)
    loc = torch.empty((P, 512), dtype=torch.int32, device=dev)
    cand = torch.empty((1, P * 512), dtype=torch.int32, device=dev)
    mo = torch.empty((1, 512), dtype=torch.int32, device=dev)
    offs = (torch.arange(P, device=dev, dtype=torch.int32) * (n // P)).view(P, 1)
    wsc = ltk.workspace(ltk.lt_topk_workspace_bytes(P, n, 512), dev)

    def cp():
        ltk.lt_topk_run(shards, slen, 512, out=loc, ws=wsc)
        torch.add(loc, offs, out=cand.view(P, 512))
        ltk.lt_topk_run(row.view(1, n), rlen, 512, cand=(cand, 1), out=mo, ws=wsc)

    cp()
    torch.cuda.synchronize()
    check_sets(mo.cpu().numpy(), oracle.topk(w.scores, w.lengths, 512, nthreads=nthreads), "cp merge")
    g = time_graph(torch, cp)
    res["cp8_shard_merge_262144"] = {"graph_us": round(g, 2)}
    log("cp shard merge (8 shards): %.2f us/call (graph)" % g)

    # Output variants at BS=1 (262144 i.i.d. scores): the selection put in
    # selection order with its scores, and the gather of its 512 cache rows
    # (1152 B each, from a [262144, 576] 2-byte cache).
    from oracle import outputs as oout
    w = workloads.cfg3("a")
    s = torch.from_numpy(w.scores).to(dev)
    l = torch.from_numpy(w.lengths).to(dev)
    o = ltk.lt_topk_run(s, l, 512)
    v = torch.empty((1, 512), dtype=torch.float32, device=dev)

    def f_order():
        ltk.lt_topk_order(o, ltk.LT_ORDER_RANK, scores=s, out_vals=v)

    f_order()
    torch.cuda.synchronize()
    want = oracle.topk(w.scores, w.lengths, 512, nthreads=nthreads)
    if not np.array_equal(o.cpu().numpy(), want) or not np.array_equal(
            v.cpu().numpy().view(np.uint32), oout.values(w.scores, want, w.n_max).view(np.uint32)):
        raise SystemExit("PARITY FAILURE: selection order at BS=1")
    g_o = time_graph(torch, f_order)
    fl_o = time_graph(torch, lambda: ltk.lt_debug_empty_launch(1, 1, 256))
    res["order_rank_values_bs1_512"] = {"graph_us": round(g_o, 2), "floor_us": round(fl_o, 2)}
    log("order (selection order + values), BS=1: %.2f us/call (graph), floor %.2f us"
        % (g_o, fl_o))
    D = 576
    gen = torch.Generator(device=dev)
    gen.manual_seed(54321)
    kv = torch.randint(-32768, 32768, (w.n_max, D), dtype=torch.int16, device=dev, generator=gen)
    gout = torch.empty((1, 512, D), dtype=torch.int16, device=dev)

    def f_gather():
        ltk.lt_gather_rows(kv, o, out=gout)

    f_gather()
    torch.cuda.synchronize()
    if not np.array_equal(gout.cpu().numpy(), oout.gather_rows(kv.cpu().numpy(), want, w.n_max)):
        raise SystemExit("PARITY FAILURE: cache-row gather at BS=1")
    g_g = time_graph(torch, f_gather)
    fl_g = time_graph(torch, lambda: ltk.lt_debug_empty_launch(-(-512 * D * 2 // 16 // 1024), 1,
                                                                256))
    res["gather_kv_bs1_512x1152B"] = {"graph_us": round(g_g, 2), "floor_us": round(fl_g, 2)}
    log("gather of 512 cache rows, BS=1: %.2f us/call (graph), floor %.2f us" % (g_g, fl_g))
    return res


if __name__ == "__main__":
    main()
