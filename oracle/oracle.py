"""CPU oracle for fine-grained FP8 quantization and block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the product package never does.

This is a thin ctypes layer over ``liboracle.so`` (built from
``fp8_oracle.c`` by ``build_oracle()``); all arithmetic lives in the C file,
whose header states the method and the readings it follows: E4M3 on all
tensors (jp-study.kr page, E4M3-on-all-tensors passage); 1x128 activation
tiles and 128x128 weight blocks ("Should Fixing Deepseek Take 60 Steps?",
Figure 7(a)) with max-abs scales computed online (why-be.why-be.co.kr page,
online max-abs passage); per-128-K promotion into FP32 (jp-study.kr page,
Figure 7(b)).

Arrays are numpy.  BF16 tensors are passed as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
SCALE_BLOCK128, SCALE_ROW128 = 0, 1

_lib = None


def build_oracle(out: str | None = None, extra_flags=()) -> str:
    """Compile fp8_oracle.c with gcc into liboracle.so, or into `out` with
    extra compiler flags (the sanitizer build); always rebuilds."""
    out = out or _LIB
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", *extra_flags,
           _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


# FP8Q_ORACLE_LIB names another build of fp8_oracle.c to load instead (the
# sanitizer run of the oracle's own tests uses it).
_ALT_LIB = os.environ.get("FP8Q_ORACLE_LIB")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _ALT_LIB:
        path = _ALT_LIB
    else:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_oracle()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.or_e4m3_decode.restype = ctypes.c_double
    lib.or_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.or_e4m3_encode.restype = ctypes.c_uint8
    lib.or_e4m3_encode.argtypes = [ctypes.c_float]
    lib.or_e4m3_encode_array.argtypes = [P, P, I64]
    lib.or_e4m3_decode_array.argtypes = [P, P, I64]
    lib.or_group_scale.argtypes = [ctypes.c_float, P, P]
    lib.or_group_scale_pow2.argtypes = [ctypes.c_float, P, P]
    lib.or_quant_1x128.argtypes = [P, I, I64, I64, I64, I64, P, I64, P, I64, I]
    lib.or_quant_128x128.argtypes = [P, I, I64, I64, I64, P, I64, P, P, I64, I]
    lib.or_quant_1x128_rule.argtypes = [P, I, I64, I64, I64, I64, P, I64, P, I64, I, I]
    lib.or_quant_128x128_rule.argtypes = [P, I, I64, I64, I64, P, I64, P, P, I64, I, I]
    lib.or_gemm_exact.argtypes = [P, I64, P, I64, P, I64, P, I, I64, I64, I64, I64, I64,
                                  P, P, I]
    lib.or_gemm_exact_elems.argtypes = [P, I64, P, I64, P, I64, P, I, I64, I64, I64,
                                        P, P, I64, P, P, I]
    lib.or_grouped_gemm_exact_elems.argtypes = [P, I64, P, I64, P, I64, P, P, I64, I64,
                                                I64, P, P, I64, P, P, I]
    _lib = lib
    return lib


def host_threads() -> int:
    return len(os.sched_getaffinity(0))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle input must be float32 or uint16 (bf16 bits), got {x.dtype}")


# --- E4M3 -------------------------------------------------------------------

def e4m3_decode(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float64)
    _load().or_e4m3_decode_array(_ptr(b), _ptr(out), b.size)
    return out


def e4m3_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().or_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def group_scale(amax: float):
    """(s, inv) for one group with maximum absolute value amax (FP32)."""
    s = ctypes.c_float()
    inv = ctypes.c_float()
    _load().or_group_scale(ctypes.c_float(amax), ctypes.byref(s), ctypes.byref(inv))
    return np.float32(s.value), np.float32(inv.value)


# scale rules: FP32 amax/448 (the method's), or the power of two an E8M0
# exponent carries (smallest 2^e with amax <= 448 * 2^e, e in [-127, 127])
RULE_FP32, RULE_POW2 = 0, 1


def group_scale_pow2(amax: float):
    """(s, inv) = (2^e, 2^-e) for one group under the power-of-two rule."""
    s = ctypes.c_float()
    inv = ctypes.c_float()
    _load().or_group_scale_pow2(ctypes.c_float(amax), ctypes.byref(s), ctypes.byref(inv))
    return np.float32(s.value), np.float32(inv.value)


# --- quantization -----------------------------------------------------------

def quant_1x128(x: np.ndarray, transposed: bool = False, threads: int | None = None,
                rule: int = RULE_FP32):
    """1x128 groups along the last axis of the 2-D array ``x``.

    With ``transposed=True`` the groups run along the FIRST axis instead
    (128x1 groups on the stored tensor, i.e. 1x128 on its transpose) and the
    returned codes are those of the transpose.  Returns (q, s) with
    q[r, c] codes of the logical matrix and s[g, r] its scales.
    """
    x = np.ascontiguousarray(x)
    dt = _dtype_code(x)
    R0, C0 = x.shape
    if transposed:
        rows, cols, xs_r, xs_c = C0, R0, 1, C0
    else:
        rows, cols, xs_r, xs_c = R0, C0, C0, 1
    g = (cols + 127) // 128
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((g, rows), dtype=np.float32)
    _load().or_quant_1x128_rule(_ptr(x), dt, rows, cols, xs_r, xs_c, _ptr(q), cols, _ptr(s),
                                rows, threads or host_threads(), rule)
    return q, s


def quant_128x128(w: np.ndarray, with_transpose: bool = False, threads: int | None = None,
                  rule: int = RULE_FP32):
    """128x128 blocks.  Returns (q, s, q_t) with s[i, j] the scale of block
    (i, j) and q_t the transposed codes (or None)."""
    w = np.ascontiguousarray(w)
    dt = _dtype_code(w)
    rows, cols = w.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=np.float32)
    q_t = np.empty((cols, rows), dtype=np.uint8) if with_transpose else None
    _load().or_quant_128x128_rule(_ptr(w), dt, rows, cols, cols, _ptr(q), cols, _ptr(s),
                                  _ptr(q_t), rows, threads or host_threads(), rule)
    return q, s, q_t


# --- GEMM -------------------------------------------------------------------

def _gemm_args(qa, sa, qb, sb):
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qb = np.ascontiguousarray(qb, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    return qa, sa, qb, sb


def gemm_exact(qa, sa, qb, sb, mode=SCALE_BLOCK128, sbs=None, threads=None):
    """Exact-per-K-block reference of C = A * B^T for all elements.

    qa[M, K] and qb[N, K] are E4M3 codes; sa[K/128, M].  BLOCK128:
    sb[(n/128)*sbs0 + kb*sbs1] (default: sb is [ceil(N/128), K/128]
    row-major); ROW128: sb[kb, n].  Returns (C*, S) as float64 [M, N].
    """
    qa, sa, qb, sb = _gemm_args(qa, sa, qb, sb)
    M, K = qa.shape
    N = qb.shape[0]
    assert qb.shape[1] == K and K % 128 == 0
    if sbs is None:
        sbs = (K // 128, 1) if mode == SCALE_BLOCK128 else (N, 0)
    c = np.empty((M, N), dtype=np.float64)
    s = np.empty((M, N), dtype=np.float64)
    _load().or_gemm_exact(_ptr(qa), K, _ptr(sa), sa.shape[1], _ptr(qb), K, _ptr(sb), mode,
                          sbs[0], sbs[1], M, N, K, _ptr(c), _ptr(s),
                          threads or host_threads())
    return c, s


def gemm_exact_elems(qa, sa, qb, sb, mi, ni, mode=SCALE_BLOCK128, sbs=None, threads=None,
                     K=None):
    """As gemm_exact, for the listed elements (mi[e], ni[e]) only.

    qa / qb may be any 2-D uint8 arrays whose first K columns hold the codes
    (default K: all columns); sa is [K/128, M]."""
    qa, sa, qb, sb = _gemm_args(qa, sa, qb, sb)
    lda, ldb, ldsa = qa.shape[1], qb.shape[1], sa.shape[1]
    K = qa.shape[1] if K is None else K
    assert K % 128 == 0 and K <= lda and K <= ldb
    N = qb.shape[0]
    if sbs is None:
        sbs = (K // 128, 1) if mode == SCALE_BLOCK128 else (N, 0)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    c = np.empty(mi.shape, dtype=np.float64)
    s = np.empty(mi.shape, dtype=np.float64)
    _load().or_gemm_exact_elems(_ptr(qa), lda, _ptr(sa), ldsa, _ptr(qb), ldb, _ptr(sb), mode,
                                sbs[0], sbs[1], K, _ptr(mi), _ptr(ni), mi.size, _ptr(c),
                                _ptr(s), threads or host_threads())
    return c, s


def grouped_gemm_exact_elems(qa, sa, qw, sw, offsets, mi, ni, threads=None):
    """Grouped GEMM reference on listed elements.

    qa[M_total, K] codes, sa[K/128, M_total]; qw[G, N, K] codes,
    sw[G, ceil(N/128), K/128]; offsets int32[G+1]."""
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    G, N, K = qw.shape
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    c = np.empty(mi.shape, dtype=np.float64)
    s = np.empty(mi.shape, dtype=np.float64)
    _load().or_grouped_gemm_exact_elems(_ptr(qa), K, _ptr(sa), sa.shape[1], _ptr(qw), K,
                                        _ptr(sw), _ptr(offsets), G, N, K, _ptr(mi),
                                        _ptr(ni), mi.size, _ptr(c), _ptr(s),
                                        threads or host_threads())
    return c, s


# --- acceptance -------------------------------------------------------------

def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of BF16 values at |x| (the unit in the last place of a BF16
    number with the same binade as x; 2^-133 for |x| below the normal
    range)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -126)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def gemm_tolerance(c_ref: np.ndarray, s_ref: np.ndarray, bf16_out: bool) -> np.ndarray:
    """Per-element bound: 1e-3 * sum|a*b| (FP32 output), plus one BF16 ulp
    of the exact value for BF16 output."""
    tol = 1e-3 * np.asarray(s_ref, dtype=np.float64)
    if bf16_out:
        tol = tol + bf16_ulp(c_ref)
    return tol
