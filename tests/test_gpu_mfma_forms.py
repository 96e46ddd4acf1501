"""The FP32-scale GEMM multiplies each 128-wide K block with the plain
16x16x128 FP8 matrix instruction and applies the block scales in the FP32
promotion (jp-study.kr page, Figure 7(b)).  tests/probes/mfma_forms.hip
checks that the plain instruction equals the scaled form with unit E8M0
scales, bit for bit, on 262,144 outputs of random E4M3 operands."""
import os
import re
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "mfma_forms")


def test_plain_mfma_equals_unit_scaled():
    assert os.path.exists(EXE), "probe not built (python tests/probes/build_probes.py)"
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    m = re.search(r"outputs (\d+), bitwise equal (\d+), nonzero (\d+)", res.stdout)
    assert res.returncode == 0 and m, res.stdout + res.stderr
    total, same, nonzero = map(int, m.groups())
    assert total == 262144 and same == total and nonzero > total // 2
