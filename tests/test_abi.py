"""The C ABI without a GPU: the library loads, exports every function that
include/fp8q.h declares, and rejects bad arguments on the host before any HIP
call (every call below fails validation or is a zero-sized no-op, so nothing
is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP = 0, 1, 2, 3, 4
A = 0x100000          # a 16-byte-aligned stand-in address (never dereferenced)
MIS = 0x100001        # misaligned stand-in


@pytest.fixture(scope="module")
def lib():
    from fp8_fine_grained_quant_amd import ops
    return ops._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fp8_quant_1x128", "fp8_quant_128x128", "fp8_blockscaled_gemm", "fp8_grouped_gemm",
              "fp8_dispatch_rows", "fp8q_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from fp8_fine_grained_quant_amd import ops
    raw = ctypes.CDLL(ops.library_path())
    for n in declared_functions():
        assert hasattr(raw, n), f"{n} declared in fp8q.h but not exported"


def test_exports_are_only_the_abi():
    from fp8_fine_grained_quant_amd import ops
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", ops.library_path()], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions()), exported ^ set(declared_functions())


def test_status_strings(lib):
    assert lib.fp8q_status_string(0) == b"FP8Q_OK"
    for st in (EINVAL, EALIGN, EUNSUPPORTED, EHIP):
        assert lib.fp8q_status_string(st).startswith(b"FP8Q_E")
    assert b"unknown" in lib.fp8q_status_string(99)


def q1(lib, x=A, dt=1, rows=4, cols=256, xs_r=256, xs_c=1, q=A, ldq=256, s=A, lds=4):
    return lib.fp8_quant_1x128(x, dt, rows, cols, xs_r, xs_c, q, ldq, s, lds, None)


def test_quant_1x128_validation(lib):
    assert q1(lib, rows=-1) == EINVAL
    assert q1(lib, dt=7) == EINVAL
    assert q1(lib, rows=0) == OK and q1(lib, cols=0) == OK          # no-ops
    assert q1(lib, x=None) == EINVAL and q1(lib, q=None) == EINVAL and q1(lib, s=None) == EINVAL
    assert q1(lib, ldq=255) == EINVAL
    assert q1(lib, lds=3) == EINVAL
    assert q1(lib, x=MIS) == EALIGN                                 # bf16 needs 2-byte alignment
    assert q1(lib, dt=0, x=A + 2) == EALIGN                         # f32 needs 4
    assert q1(lib, s=A + 2) == EALIGN
    assert q1(lib, xs_r=3, xs_c=2) == EINVAL                        # neither stride is 1
    assert q1(lib, xs_r=100, xs_c=1) == EINVAL                      # pitch < cols
    # transposed view: physical [cols, rows] with pitch xs_c
    assert q1(lib, xs_r=1, xs_c=2) == EINVAL                        # pitch < rows
    # size limits, checked before any device access (the pointers are never used)
    big = (1 << 24) * 128 + 1                                       # 2^24 + 1 groups per row
    assert q1(lib, cols=big, xs_r=big, ldq=big) == EUNSUPPORTED
    assert q1(lib, rows=1 << 23, cols=1 << 32, xs_r=1, xs_c=1 << 23, ldq=1 << 32,
              lds=1 << 23) == EUNSUPPORTED                         # 2^31 tiles, transposed


def q2(lib, w=A, dt=1, rows=256, cols=256, ldw=256, q=A, ldq=256, s=A, qt=None, ldqt=0):
    return lib.fp8_quant_128x128(w, dt, rows, cols, ldw, q, ldq, s, qt, ldqt, None)


def test_quant_128x128_validation(lib):
    assert q2(lib, cols=-5) == EINVAL
    assert q2(lib, dt=2) == EINVAL
    assert q2(lib, rows=0) == OK
    assert q2(lib, w=None) == EINVAL
    assert q2(lib, ldw=128) == EINVAL and q2(lib, ldq=128) == EINVAL
    assert q2(lib, qt=A, ldqt=100) == EINVAL
    assert q2(lib, w=MIS) == EALIGN and q2(lib, dt=0, w=A + 2) == EALIGN
    assert q2(lib, s=A + 1) == EALIGN
    assert q2(lib, rows=1 << 23, cols=1 << 32, ldw=1 << 32, ldq=1 << 32) == EUNSUPPORTED  # 2^31 blocks


def gemm(lib, a=A, lda=512, sa=A, ldsa=256, b=A, ldb=512, sb=A, mode=0, sbs0=4, sbs1=1, c=A,
         cdt=1, ldc=256, M=256, N=256, K=512):
    return lib.fp8_blockscaled_gemm(a, lda, sa, ldsa, b, ldb, sb, mode, sbs0, sbs1, c, cdt, ldc, M,
                                    N, K, None)


def test_gemm_validation(lib):
    assert gemm(lib, M=0) == OK and gemm(lib, N=0) == OK
    assert gemm(lib, M=-1) == EINVAL
    assert gemm(lib, mode=2) == EINVAL
    assert gemm(lib, cdt=3) == EINVAL
    assert gemm(lib, a=None) == EINVAL and gemm(lib, sb=None) == EINVAL and gemm(lib, c=None) == EINVAL
    assert gemm(lib, lda=256) == EINVAL and gemm(lib, ldb=256) == EINVAL
    assert gemm(lib, ldc=255) == EINVAL and gemm(lib, ldsa=255) == EINVAL
    assert gemm(lib, K=100, lda=112, ldb=112) == EUNSUPPORTED
    assert gemm(lib, K=0) == EUNSUPPORTED
    assert gemm(lib, a=MIS) == EALIGN and gemm(lib, c=A + 8) == EALIGN and gemm(lib, sa=A + 1) == EALIGN
    assert gemm(lib, lda=520) == EALIGN and gemm(lib, ldc=258) == EALIGN
    assert gemm(lib, sbs0=-1) == EINVAL
    assert gemm(lib, mode=1, sbs0=100) == EINVAL                    # ROW128 pitch < N


def ggemm(lib, a=A, lda=512, sa=A, ldsa=256, b=A, ldb=512, sb=A, off=A, G=4, M=256, c=A, cdt=1,
          ldc=256, N=256, K=512):
    return lib.fp8_grouped_gemm(a, lda, sa, ldsa, b, ldb, sb, off, G, M, c, cdt, ldc, N, K, None)


def test_grouped_gemm_validation(lib):
    assert ggemm(lib, G=0) == EINVAL
    assert ggemm(lib, M=0) == OK
    assert ggemm(lib, off=None) == EINVAL
    assert ggemm(lib, off=A + 2) == EALIGN
    assert ggemm(lib, G=100000) == EUNSUPPORTED
    assert ggemm(lib, K=200, lda=208, ldb=208) == EUNSUPPORTED
    assert ggemm(lib, ldsa=100) == EINVAL


def disp(lib, qs=A, ldqs=7168, ss=A, lds_s=100, T=100, idx=A, R=300, C=7168, qd=A, ldqd=7168, sd=A,
         lds_d=300):
    return lib.fp8_dispatch_rows(qs, ldqs, ss, lds_s, T, idx, R, C, qd, ldqd, sd, lds_d, None)


def test_dispatch_rows_validation(lib):
    assert disp(lib, R=-1) == EINVAL and disp(lib, C=-1) == EINVAL and disp(lib, T=-1) == EINVAL
    assert disp(lib, R=0) == OK and disp(lib, C=0) == OK              # no-ops
    for k in ("qs", "ss", "idx", "qd", "sd"):
        assert disp(lib, **{k: None}) == EINVAL
    assert disp(lib, ldqs=7000) == EINVAL and disp(lib, ldqd=7000) == EINVAL
    assert disp(lib, lds_s=99) == EINVAL and disp(lib, lds_d=299) == EINVAL
    assert disp(lib, ss=A + 2) == EALIGN and disp(lib, sd=A + 1) == EALIGN
    assert disp(lib, idx=A + 2) == EALIGN


def test_pow2_variants_validate_like_their_counterparts(lib):
    assert lib.fp8_quant_1x128_pow2(A, 1, 4, 256, 256, 1, A, 255, A, 4, None) == EINVAL
    assert lib.fp8_quant_1x128_pow2(A, 1, 0, 256, 256, 1, A, 256, A, 4, None) == OK
    assert lib.fp8_quant_128x128_pow2(A, 1, 4, 256, 256, A, 256, A + 2, None, 0, None) == EALIGN
    assert lib.fp8_blockscaled_gemm_pow2(A, 256, A, 256, A, 512, A, 0, 4, 1, A, 1, 256, 256, 256,
                                         512, None) == EINVAL                   # lda < K
    assert lib.fp8_blockscaled_gemm_pow2(A, 512, A, 256, A, 512, A, 0, 4, 1, A, 1, 256, 256, 256,
                                         500, None) == EUNSUPPORTED
    assert lib.fp8_grouped_gemm_pow2(A, 512, A, 256, A, 512, A, None, 4, 256, A, 1, 256, 256, 512,
                                     None) == EINVAL
