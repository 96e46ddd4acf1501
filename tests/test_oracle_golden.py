"""Regression fixture for the oracle's quantizers (tests/golden/quant_small.txt,
written by tests/golden/make_golden.py from the oracle itself).  It guards
against unintended changes; the oracle's correctness pins are the other
test_oracle_* files."""
import os
import sys

import numpy as np

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, HERE)
import make_golden  # noqa: E402


def _read():
    rows = {"q1": [], "s1": [], "q2": [], "s2": []}
    with open(os.path.join(HERE, "quant_small.txt")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            tag, rest = line.split(" ", 1)
            rows[tag].append(rest.strip())
    q1 = np.array([np.frombuffer(bytes.fromhex(h), np.uint8) for h in rows["q1"]])
    s1 = np.array([int(v, 16) for v in rows["s1"][0].split()], np.uint32)
    q2 = np.array([np.frombuffer(bytes.fromhex(h), np.uint8) for h in rows["q2"]])
    s2 = np.array([int(v, 16) for v in rows["s2"][0].split()], np.uint32)
    return q1, s1, q2, s2


def test_quant_fixture(oracle):
    x, w = make_golden.inputs()
    q1, s1, q2, s2 = _read()
    q, s = oracle.quant_1x128(x)
    assert np.array_equal(q, q1) and np.array_equal(s.view(np.uint32).ravel(), s1)
    qw, sw, _ = oracle.quant_128x128(w)
    assert np.array_equal(qw, q2) and np.array_equal(sw.view(np.uint32).ravel(), s2)
    # hand-checkable entries: row 0 group 0 has amax 300 -> s = 300/448
    assert s[0, 0] == np.float32(300.0) / np.float32(448.0) and q[0, 3] == 0x7E
    assert s[0, 2] == 0.0 and np.all(q[2, :128] == 0)          # all-zero group
    assert q[1, 130] == 0xFE                                   # -1000 is the amax
