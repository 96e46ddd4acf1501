"""Fine-grained FP8 quantization and block-scaled FP8 GEMM for MI355X (gfx950).

The compute lives in ``libfp8q.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fp8q.h``).  The Python names below are thin bindings with
the same names as the C entry points; they only marshal tensor pointers, sizes
and the current HIP stream.  Importing a binding loads the library and fails
loudly if it has not been built -- there is no fallback implementation.

``synth`` (seeded synthetic inputs) imports without the library.
"""
_BINDINGS = ("fp8_quant_1x128", "fp8_quant_128x128", "fp8_blockscaled_gemm",
             "fp8_grouped_gemm", "fp8_dispatch_rows", "fp8q_status_string", "library_path", "Fp8qError",
             "F32", "BF16", "SCALE_BLOCK128", "SCALE_ROW128")

__all__ = list(_BINDINGS) + ["synth"]


def __getattr__(name):
    if name in _BINDINGS:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
