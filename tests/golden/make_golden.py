"""Write the oracle's expected outputs for small seeded workloads.

Calls only ``oracle`` (the CPU oracle) and ``workloads`` (seeded inputs). Run
from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle      # noqa: E402
import workloads   # noqa: E402


def write(name, arr, header):
    path = os.path.join(HERE, name)
    with open(path, "w") as f:
        f.write("# " + header + "\n")
        for row in np.atleast_2d(arr):
            f.write(" ".join(str(int(v)) for v in row) + "\n")
    print("wrote", path)


def main():
    w = workloads.cfg1()
    out = oracle.topk(w.scores, w.lengths, w.k)
    write("cfg1_topk512.txt", np.sort(out, axis=1),
          "oracle top-512 of the single-row workload (N=4096, N(0,1), seed (1,0)), "
          "indices sorted ascending")
    w = workloads.cfg3("b", n=20000)
    out = oracle.topk(w.scores, w.lengths, w.k)
    write("cfg3b_small_topk512.txt", np.sort(out, axis=1),
          "oracle top-512 of the bf16-rounded row (N=20000, seed (3,0)), indices sorted ascending")


if __name__ == "__main__":
    main()
