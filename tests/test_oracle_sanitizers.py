"""The oracle's own pins, rerun against a build of fp8_oracle.c with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; the oracle
never runs on the GPU).  Any out-of-bounds access, use of freed memory,
signed overflow, invalid shift or misaligned access in the oracle ends the
child run with an error.

The child is a separate Python process with the sanitizer runtimes preloaded
(Python itself is not built with them) and FP8Q_ORACLE_LIB pointing at the
instrumented library; leak checking is off, since the interpreter keeps its
own allocations until exit."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_e4m3.py", "test_oracle_quant.py", "test_oracle_gemm.py",
        "test_oracle_pow2.py", "test_oracle_golden.py"]


def _runtime(name: str) -> str | None:
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    path = subprocess.run([gcc, f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from oracle import oracle
    lib = oracle.build_oracle(str(tmp_path / "liboracle_san.so"),
                              ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=all"])
    env = dict(os.environ)
    env.update({"FP8Q_ORACLE_LIB": lib,
                "LD_PRELOAD": f"{os.path.realpath(asan)}:{os.path.realpath(ubsan)}",
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=23",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=24"})
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           *[os.path.join(ROOT, "tests", p) for p in PINS]]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    tail = (res.stdout[-3000:] + "\n" + res.stderr[-3000:])
    assert res.returncode == 0, f"sanitized oracle run failed (rc {res.returncode}):\n{tail}"
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
    print(res.stdout.strip().splitlines()[-1])
