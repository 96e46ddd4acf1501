"""Throughput of the GEMM's compute slot on the full chip, register-only
(tests/probes/mfma_rates.hip): the 16x16x128 and 32x32x64 FP8 matrix
instructions, accumulating in place or with the FP32 promotion of a fresh
partial sum per 128-wide K block (jp-study.kr page, Figure 7(b)), with two or
one computing waves per SIMD.  The table it prints backs the choice of
16x16x128 for the FP32-scale GEMM; only completion and sane rates are
asserted (timings are not a pass/fail criterion)."""
import os
import re
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "mfma_rates")


def test_mfma_rates_probe():
    assert os.path.exists(EXE), "probe not built (python tests/probes/build_probes.py)"
    res = subprocess.run([EXE, "2000"], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    rates = [float(m.group(1)) for m in re.finditer(r"(\d+\.\d+) of 5\.0 PFLOP/s", res.stdout)]
    assert len(rates) == 20 and all(0.05 < r < 1.2 for r in rates), rates
