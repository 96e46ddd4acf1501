"""Writes the regression fixtures in this folder.  Calls only the CPU oracle.

quant_small.txt: a 4x256 FP32 input (seeded, with a few large values and a
zero group), its 1x128 codes and FP32 scale bit patterns; and a 256x128 input
quantized as one 128x128 block pair.  Method: 1x128 activation tiles and
128x128 weight blocks ("Should Fixing Deepseek Take 60 Steps?", Figure 7(a)),
max-abs scales computed online (why-be.why-be.co.kr page, online max-abs
passage), E4M3 codes (jp-study.kr page, E4M3-on-all-tensors passage).

Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import oracle  # noqa: E402


def inputs():
    rng = np.random.default_rng(2024)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    x[0, 3] = 300.0
    x[1, 130] = -1000.0
    x[2, :128] = 0.0
    x[3] *= np.float32(1e-30)
    w = (rng.standard_normal((256, 128)) * 0.02).astype(np.float32)
    return x, w


def main():
    x, w = inputs()
    q, s = oracle.quant_1x128(x)
    qw, sw, _ = oracle.quant_128x128(w)
    with open(os.path.join(HERE, "quant_small.txt"), "w") as f:
        f.write("# written by tests/golden/make_golden.py from the CPU oracle; do not edit\n")
        f.write("# 1x128: rows of codes (hex), then scales s[g][r] as FP32 bit patterns\n")
        for r in range(q.shape[0]):
            f.write("q1 " + q[r].tobytes().hex() + "\n")
        f.write("s1 " + " ".join(f"{v:08x}" for v in s.view(np.uint32).ravel()) + "\n")
        f.write("# 128x128: codes of each row of the 256x128 input, then the 2 block scales\n")
        for r in range(qw.shape[0]):
            f.write("q2 " + qw[r].tobytes().hex() + "\n")
        f.write("s2 " + " ".join(f"{v:08x}" for v in sw.view(np.uint32).ravel()) + "\n")


if __name__ == "__main__":
    main()
