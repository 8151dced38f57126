"""Writes tests/golden/c1_block_samples.txt from the CPU oracle only.

The pages print no values for this block, so this fixture is a frozen record
of the oracle's own output on the fp32 workload (single ResidualBlock,
64 -> 64, [1,4,16,16,64], seed 0): it catches an unintended change to the
oracle's arithmetic.  Regenerate only together with a change to oracle.c whose
commit message names the passage that justifies it.

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from causal_convolution_amd import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_block_samples.txt")

# (t, h, w, c) positions: corners, edges, the first frame and interior points
SAMPLES = [(0, 0, 0, 0), (0, 0, 15, 63), (0, 15, 0, 5), (1, 7, 8, 31), (2, 0, 9, 12),
           (3, 15, 15, 63), (3, 8, 0, 40), (2, 11, 4, 7), (1, 15, 15, 0), (3, 3, 3, 3)]


def compute():
    wl = workloads.WORKLOADS["c1"]
    p = workloads.make_params(wl, seed=0)
    x = workloads.make_x_host(wl, seed=0)
    blk = oracle.Block(p["gamma1"], p["beta1"], p["wa"], p["ba"], p["gamma2"], p["beta2"],
                       p["wb"], p["bb"], p["ws"], p["bs"])
    return oracle.resblock_full(blk, x)


def main():
    y = compute()
    with open(OUT, "w") as f:
        f.write("# oracle ResidualBlock output, workload c1 (fp32 64->64 [1,4,16,16,64] seed 0)\n")
        f.write("# written by tests/golden/make_golden.py; columns: t h w c float32-bits value\n")
        for (t, h, w, c) in SAMPLES:
            v = np.float32(y[0, t, h, w, c])
            f.write(f"{t} {h} {w} {c} {v.view(np.uint32):08x} {float(v):.9g}\n")


if __name__ == "__main__":
    main()
