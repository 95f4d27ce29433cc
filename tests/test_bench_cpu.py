"""CPU checks of the measurement path in bench.py: the byte counts its
roofline divides by, the per-configuration throughput arithmetic, the
refusal of more than one GPU, and the rule that measured HBM traffic is
reported only for the kernel source it was taken on."""
import os
import subprocess
import sys

import numpy as np

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_algorithmic_bytes():
    # 8192 rows at positions 1,040,384 + i, 4:1 compression: the valid
    # lengths run from 260,096 to 262,143 and sum to 2,139,090,944 scores
    lens = workloads.cfg5_lengths()
    assert lens.min() == 260096 and lens.max() == 262143
    assert int(lens.astype(np.int64).sum()) == 2139090944
    # 4 B per valid score + 4 B per output index + 4 B per length
    assert bench.algorithmic_bytes(lens, 512) == 4 * 2139090944 + 4 * 512 * 8192 + 4 * 8192
    assert bench.algorithmic_bytes(lens, 512) == 8573173760


def test_throughput_fields():
    t = bench.throughput(nbytes=8_000_000, rows=4, us=2.0)
    assert t["us_per_row"] == 0.5
    assert t["rows_per_s"] == 2_000_000.0
    assert t["GBps"] == 4000.0                       # 8 MB in 2 us
    assert t["frac_of_hbm_peak"] == 0.5              # of 8000 GB/s


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_the_profiled_source(tmp_path):
    good = tmp_path / "traffic.txt"
    good.write_text("# comment\nkernel_source_sha256_16 = %s\nhbm_bytes_per_launch = 123456\n"
                    % bench.src_hash())
    assert bench.read_traffic(str(good)) == 123456
    # a file taken on another source (here: the output kernels' file) is stale
    assert bench.read_traffic(str(good), bench.OUTPUT_SRC) is None
    other = tmp_path / "other.txt"
    other.write_text("kernel_source_sha256_16 = %s\nhbm_bytes_per_launch = 7\n"
                     % bench.src_hash(bench.OUTPUT_SRC))
    assert bench.read_traffic(str(other), bench.OUTPUT_SRC) == 7
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel_source_sha256_16 = 0000000000000000\nhbm_bytes_per_launch = 1\n")
    assert bench.read_traffic(str(stale)) is None
    assert bench.read_traffic(str(tmp_path / "missing.txt")) is None


def test_parity_gate_compares_whole_sets():
    want = np.array([[5, 3, 9, -1], [0, 1, 2, 3]], np.int32)
    assert bench.same_sets_all(np.array([[9, 5, 3, -1], [3, 2, 1, 0]], np.int32), want)
    assert bench.same_sets_all(np.array([[-1, 9, 5, 3], [3, 2, 1, 0]], np.int32), want)
    assert not bench.same_sets_all(np.array([[9, 5, 4, -1], [3, 2, 1, 0]], np.int32), want)
    assert not bench.same_sets_all(np.array([[9, 5, 3, 3], [3, 2, 1, 0]], np.int32), want)
    assert not bench.same_sets_all(want[:1], want)


def test_cpu_baseline_host_fields():
    n = bench.oracle_threads()
    assert 1 <= n <= 16
    info = bench.host_info(n)
    assert info["threads_used"] == n
    assert info["host_logical_cpus"] == os.cpu_count()
    assert 1 <= info["usable_cpus"] <= os.cpu_count()
