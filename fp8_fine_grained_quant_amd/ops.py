"""Python binding of libfp8q (include/fp8q.h), same names as the C entry points.

Only argument marshalling happens here: tensor shapes and strides become the
C sizes and leading dimensions, outputs are allocated with torch when not
given, and the call is enqueued on the current HIP stream of the tensors'
device.  All arithmetic runs in the library's HIP kernels.  If the library
has not been built, importing this module raises ImportError -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfp8q.so")

F32, BF16 = 0, 1
SCALE_BLOCK128, SCALE_ROW128 = 0, 1
_STATUS = {0: "FP8Q_OK", 1: "FP8Q_EINVAL", 2: "FP8Q_EALIGN", 3: "FP8Q_EUNSUPPORTED",
           4: "FP8Q_EHIP"}


def library_path() -> str:
    return _LIB_PATH


def _load_library():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build the HIP library first "
            "(python -m fp8_fine_grained_quant_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fp8_quant_1x128.restype = I
    lib.fp8_quant_1x128.argtypes = [P, I, I64, I64, I64, I64, P, I64, P, I64, P]
    lib.fp8_quant_128x128.restype = I
    lib.fp8_quant_128x128.argtypes = [P, I, I64, I64, I64, P, I64, P, P, I64, P]
    lib.fp8_blockscaled_gemm.restype = I
    lib.fp8_blockscaled_gemm.argtypes = [P, I64, P, I64, P, I64, P, I, I64, I64, P, I, I64, I64,
                                         I64, I64, P]
    lib.fp8_grouped_gemm.restype = I
    lib.fp8_grouped_gemm.argtypes = [P, I64, P, I64, P, I64, P, P, I64, I64, P, I, I64, I64,
                                     I64, P]
    for name, base in (("fp8_quant_1x128_pow2", "fp8_quant_1x128"),
                       ("fp8_quant_128x128_pow2", "fp8_quant_128x128"),
                       ("fp8_blockscaled_gemm_pow2", "fp8_blockscaled_gemm"),
                       ("fp8_grouped_gemm_pow2", "fp8_grouped_gemm")):
        getattr(lib, name).restype = I
        getattr(lib, name).argtypes = getattr(lib, base).argtypes
    lib.fp8_dispatch_rows.restype = I
    lib.fp8_dispatch_rows.argtypes = [P, I64, P, I64, I64, P, I64, I64, P, I64, P, I64, P]
    lib.fp8q_status_string.restype = ctypes.c_char_p
    lib.fp8q_status_string.argtypes = [I]
    return lib


_lib = _load_library()


class Fp8qError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fp8q_status_string(status)}")


def fp8q_status_string(status: int) -> str:
    return _lib.fp8q_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise Fp8qError(status, where)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libfp8q operates on device tensors")


# --- quantization -------------------------------------------------------------

def fp8_quant_1x128(x: torch.Tensor, transposed: bool = False, q: torch.Tensor | None = None,
                    s: torch.Tensor | None = None, pow2: bool = False):
    """1x128 tile quantization of a 2-D activation tensor (bf16 or fp32).

    transposed=False: groups of 128 along dim 1; returns q [R, C] uint8 codes
    and s [ceil(C/128), R] FP32 scales.
    transposed=True: groups of 128 along dim 0 (128x1 on the stored tensor,
    for the weight-gradient GEMM); returns the codes of x^T, q [C, R], and
    s [ceil(R/128), C].
    pow2=True calls fp8_quant_1x128_pow2 (power-of-two scales).
    """
    _require_cuda(x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    # a size-1 dimension may carry any stride; it is never stepped over
    if x.stride(1) != 1 and C != 1:
        raise ValueError("x must be contiguous along dim 1")
    ld = x.stride(0) if R != 1 else C
    if not transposed:
        rows, cols, xs_r, xs_c = R, C, ld, 1
    else:
        rows, cols, xs_r, xs_c = C, R, 1, ld
    g = (cols + 127) // 128
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((g, rows), dtype=torch.float32, device=x.device)
    _require_cuda(q, s)
    fn = _lib.fp8_quant_1x128_pow2 if pow2 else _lib.fp8_quant_1x128
    st = fn(_ptr(x), _dtype_code(x), rows, cols, xs_r, xs_c, _ptr(q), q.stride(0), _ptr(s),
            s.stride(0), _stream(x))
    _check(st, "fp8_quant_1x128" + ("_pow2" if pow2 else ""))
    return q, s


def fp8_quant_128x128(w: torch.Tensor, with_transpose: bool = False,
                      q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                      q_t: torch.Tensor | None = None, pow2: bool = False):
    """128x128 block quantization of a 2-D weight (bf16 or fp32).

    Returns q [R, C] codes, s [ceil(R/128), ceil(C/128)] scales and, if
    requested, the transposed codes q_t [C, R].  pow2=True calls
    fp8_quant_128x128_pow2 (power-of-two scales)."""
    _require_cuda(w)
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be 2-D and contiguous along dim 1")
    R, C = w.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty(((R + 127) // 128, (C + 127) // 128), dtype=torch.float32,
                        device=w.device)
    if with_transpose and q_t is None:
        q_t = torch.empty((C, R), dtype=torch.uint8, device=w.device)
    _require_cuda(q, s, q_t)
    if not s.is_contiguous():
        raise ValueError("s must be contiguous")
    fn = _lib.fp8_quant_128x128_pow2 if pow2 else _lib.fp8_quant_128x128
    st = fn(_ptr(w), _dtype_code(w), R, C, w.stride(0), _ptr(q), q.stride(0), _ptr(s), _ptr(q_t),
            q_t.stride(0) if q_t is not None else 0, _stream(w))
    _check(st, "fp8_quant_128x128" + ("_pow2" if pow2 else ""))
    return q, s, q_t


# --- GEMM -------------------------------------------------------------------

def _out_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError("output dtype must be bfloat16 or float32")


def _check_tensor(t: torch.Tensor, name: str, dtype, shape) -> None:
    """t must have this dtype and shape and be unit-stride along its last
    dimension (a size-1 last dimension may carry any stride)."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dim() >= 1 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous along its last dimension")


def _check_out(c: torch.Tensor, M: int, N: int) -> None:
    if c.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("c must be bfloat16 or float32")
    _check_tensor(c, "c", c.dtype, (M, N))
    if c.stride(1) != 1:
        raise ValueError("c must be contiguous along dim 1")


def _alloc_out(M: int, N: int, dtype, device) -> torch.Tensor:
    """Output [M, N] whose row pitch is a multiple of 4 elements (the GEMM
    stores 4 consecutive columns per lane); a view of a padded buffer when N
    is not."""
    ld = (N + 3) // 4 * 4
    buf = torch.empty((M, ld), dtype=dtype, device=device)
    return buf if ld == N else buf[:, :N]


def fp8_blockscaled_gemm(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                         out_dtype=torch.bfloat16, scale_mode: int = SCALE_BLOCK128,
                         c: torch.Tensor | None = None, pow2: bool = False):
    """C = A * B^T with per-128-K promotion.

    a [M, K] and b [N, K] uint8 E4M3 codes (K contiguous); sa [K/128, M]
    (any row pitch); sb: SCALE_BLOCK128 -> 2-D [ceil(N/128), K/128] (any
    strides, e.g. a transposed view); SCALE_ROW128 -> [K/128, N] (row pitch
    >= N).  pow2=True calls fp8_blockscaled_gemm_pow2 (power-of-two scales
    applied by the matrix instruction)."""
    _require_cuda(a, sa, b, sb)
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = a.shape
    N = b.shape[0]
    if a.dtype != torch.uint8 or b.dtype != torch.uint8:
        raise TypeError("a and b must be uint8 E4M3 codes")
    if b.shape[1] != K or a.stride(1) != 1 or b.stride(1) != 1:
        raise ValueError("a, b must be [M,K] / [N,K] with K contiguous")
    nkb = K // 128
    _check_tensor(sa, "sa", torch.float32, (nkb, M))
    if scale_mode == SCALE_BLOCK128:
        if sb.dtype != torch.float32 or tuple(sb.shape) != ((N + 127) // 128, nkb):
            raise ValueError(f"BLOCK128 sb must be float32 [{(N + 127) // 128}, {nkb}] "
                             f"(any strides), got {sb.dtype} {tuple(sb.shape)}")
        sbs0, sbs1 = sb.stride(0), sb.stride(1)
    elif scale_mode == SCALE_ROW128:
        _check_tensor(sb, "ROW128 sb", torch.float32, (nkb, N))
        sbs0, sbs1 = sb.stride(0), 0
    else:
        raise ValueError(f"unknown scale_mode {scale_mode}")
    if c is None:
        c = _alloc_out(M, N, out_dtype, a.device)
    _require_cuda(c)
    _check_out(c, M, N)
    fn = _lib.fp8_blockscaled_gemm_pow2 if pow2 else _lib.fp8_blockscaled_gemm
    st = fn(_ptr(a), a.stride(0), _ptr(sa), sa.stride(0), _ptr(b), b.stride(0), _ptr(sb),
            scale_mode, sbs0, sbs1, _ptr(c), _out_code(c.dtype), c.stride(0), M, N, K, _stream(a))
    _check(st, "fp8_blockscaled_gemm" + ("_pow2" if pow2 else ""))
    return c


def fp8_grouped_gemm(a: torch.Tensor, sa: torch.Tensor, w: torch.Tensor, sw: torch.Tensor,
                     offsets: torch.Tensor, out_dtype=torch.bfloat16,
                     c: torch.Tensor | None = None, pow2: bool = False):
    """Per-group GEMM: rows [offsets[g], offsets[g+1]) of A times W_g^T.

    a [M_total, K] codes, sa [K/128, M_total]; w [G, N, K] codes (contiguous
    per group), sw [G, ceil(N/128), K/128] contiguous; offsets int32 [G+1] on
    the device.  pow2=True calls fp8_grouped_gemm_pow2."""
    _require_cuda(a, sa, w, sw, offsets)
    if a.dim() != 2 or w.dim() != 3:
        raise ValueError("a must be 2-D and w 3-D")
    M, K = a.shape
    G, N, K2 = w.shape
    if a.dtype != torch.uint8 or w.dtype != torch.uint8:
        raise TypeError("a and w must be uint8 E4M3 codes")
    if K2 != K or a.stride(1) != 1 or w.stride(2) != 1 or w.stride(0) != N * w.stride(1):
        raise ValueError("a [M,K], w [G,N,K] with K contiguous and groups dense")
    _check_tensor(sa, "sa", torch.float32, (K // 128, M))
    if (sw.dtype != torch.float32 or not sw.is_contiguous()
            or tuple(sw.shape) != (G, (N + 127) // 128, K // 128)):
        raise ValueError("sw must be a contiguous float32 [G, ceil(N/128), K/128] tensor")
    if offsets.dtype != torch.int32 or offsets.numel() != G + 1 or not offsets.is_contiguous():
        raise ValueError("offsets must be a contiguous int32 [G+1] tensor")
    if c is None:
        c = _alloc_out(M, N, out_dtype, a.device)
    _require_cuda(c)
    _check_out(c, M, N)
    fn = _lib.fp8_grouped_gemm_pow2 if pow2 else _lib.fp8_grouped_gemm
    st = fn(_ptr(a), a.stride(0), _ptr(sa), sa.stride(0), _ptr(w), w.stride(1), _ptr(sw),
            _ptr(offsets), G, M, _ptr(c), _out_code(c.dtype), c.stride(0), N, K, _stream(a))
    _check(st, "fp8_grouped_gemm" + ("_pow2" if pow2 else ""))
    return c


# --- FP8 dispatch --------------------------------------------------------------

def fp8_dispatch_rows(q_src: torch.Tensor, s_src: torch.Tensor, index: torch.Tensor,
                      q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """Gather token rows of 1x128-quantized activations into expert order.

    q_src [T, C] uint8 codes and s_src [ceil(C/128), T] FP32 scales (the
    output of fp8_quant_1x128); index int32 [R] on the device, row r taking
    token index[r] (entries outside [0, T) are skipped).  Returns q [R, C]
    and s [ceil(C/128), R]."""
    _require_cuda(q_src, s_src, index)
    if q_src.dim() != 2 or q_src.stride(1) != 1 or q_src.dtype != torch.uint8:
        raise ValueError("q_src must be a 2-D uint8 tensor, contiguous along dim 1")
    T, C = q_src.shape
    G = (C + 127) // 128
    if s_src.dim() != 2 or s_src.shape[0] != G or s_src.shape[1] != T or s_src.stride(1) != 1:
        raise ValueError("s_src must be [ceil(C/128), T], contiguous along dim 1")
    if index.dtype != torch.int32 or index.dim() != 1 or not index.is_contiguous():
        raise ValueError("index must be a contiguous int32 vector")
    R = index.numel()
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=q_src.device)
    if s is None:
        s = torch.empty((G, R), dtype=torch.float32, device=q_src.device)
    _require_cuda(q, s)
    st = _lib.fp8_dispatch_rows(_ptr(q_src), q_src.stride(0), _ptr(s_src), s_src.stride(0), T,
                                _ptr(index), R, C, _ptr(q), q.stride(0), _ptr(s), s.stride(0),
                                _stream(q_src))
    _check(st, "fp8_dispatch_rows")
    return q, s
