// fp8q_api.hip -- the C ABI of libfp8q (declared in include/fp8q.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so each error status can be produced without a GPU, then
// dispatches to one kernel launch on the caller's stream.
#include "fp8q.h"
#include "kernels.h"

#define FP8Q_API extern "C" __attribute__((visibility("default")))

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_EHIP; }

}  // namespace

FP8Q_API const char* fp8q_status_string(int status) {
    switch (status) {
        case FP8Q_OK: return "FP8Q_OK";
        case FP8Q_EINVAL: return "FP8Q_EINVAL: invalid argument";
        case FP8Q_EALIGN: return "FP8Q_EALIGN: misaligned pointer or leading dimension";
        case FP8Q_EUNSUPPORTED: return "FP8Q_EUNSUPPORTED: unsupported shape";
        case FP8Q_EHIP: return "FP8Q_EHIP: kernel launch failed";
        default: return "FP8Q: unknown status";
    }
}

namespace {

int quant_1x128_impl(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t xs_r,
                     int64_t xs_c, uint8_t* q, int64_t ldq, float* s, int64_t lds, int rule,
                     hipStream_t stream) {
    if (rows < 0 || cols < 0) return FP8Q_EINVAL;
    if (x_dtype != FP8Q_F32 && x_dtype != FP8Q_BF16) return FP8Q_EINVAL;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_EINVAL;
    if (ldq < cols || lds < rows) return FP8Q_EINVAL;
    if (!aligned(x, x_dtype == FP8Q_BF16 ? 2 : 4) || !aligned(s, 4)) return FP8Q_EALIGN;
    // The kernels use 16-byte loads and 8-byte stores wherever the pointers
    // and pitches allow it, and element accesses elsewhere.
    if (xs_c == 1 && (xs_r >= cols || rows == 1)) {
        // row-contiguous input; a launch covers whole 4-row bands of fewer
        // than 2^31 groups
        if ((cols + 127) / 128 > (int64_t(1) << 24)) return FP8Q_EUNSUPPORTED;
        const int64_t ldx = rows == 1 ? cols : xs_r;
        return launch_status(fp8q::launch_quant_rows(x, x_dtype, rows, cols, ldx, q, ldq, s,
                                                     lds, rule, stream));
    }
    if (xs_r == 1 && (xs_c >= rows || cols == 1)) {
        // Stored transposed: physical tensor [cols, rows] with row pitch xs_c;
        // 128x1 groups along its rows, codes written transposed, in 128x256
        // tiles (fewer than 2^31 of them).
        if ((cols + 127) / 128 * ((rows + 255) / 256) > 0x7FFFFFFF) return FP8Q_EUNSUPPORTED;
        const int64_t ldx = cols == 1 ? rows : xs_c;
        return launch_status(fp8q::launch_quant_tiles(x, x_dtype, fp8q::kTileCols, cols, rows,
                                                      ldx, nullptr, 0, q, ldq, s, lds, rule,
                                                      stream));
    }
    return FP8Q_EINVAL;
}

int quant_128x128_impl(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                       uint8_t* q, int64_t ldq, float* s, uint8_t* q_t, int64_t ldqt, int rule,
                       hipStream_t stream) {
    if (rows < 0 || cols < 0) return FP8Q_EINVAL;
    if (w_dtype != FP8Q_F32 && w_dtype != FP8Q_BF16) return FP8Q_EINVAL;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!w || !q || !s) return FP8Q_EINVAL;
    if (ldw < cols || ldq < cols) return FP8Q_EINVAL;
    if (q_t && ldqt < rows) return FP8Q_EINVAL;
    if (!aligned(w, w_dtype == FP8Q_BF16 ? 2 : 4) || !aligned(s, 4)) return FP8Q_EALIGN;
    // one workgroup per 128x128 block
    if ((rows + 127) / 128 * ((cols + 127) / 128) > 0x7FFFFFFF) return FP8Q_EUNSUPPORTED;
    return launch_status(fp8q::launch_quant_tiles(w, w_dtype, fp8q::kTileBlock, rows, cols, ldw, q,
                                                  ldq, q_t, ldqt, s, 0, rule, stream));
}

}  // namespace

FP8Q_API int fp8_quant_1x128(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t xs_r,
                             int64_t xs_c, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             hipStream_t stream) {
    return quant_1x128_impl(x, x_dtype, rows, cols, xs_r, xs_c, q, ldq, s, lds, fp8q::kRuleFP32,
                            stream);
}

FP8Q_API int fp8_quant_1x128_pow2(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                  int64_t xs_r, int64_t xs_c, uint8_t* q, int64_t ldq, float* s,
                                  int64_t lds, hipStream_t stream) {
    return quant_1x128_impl(x, x_dtype, rows, cols, xs_r, xs_c, q, ldq, s, lds, fp8q::kRulePow2,
                            stream);
}

FP8Q_API int fp8_quant_128x128(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                               uint8_t* q, int64_t ldq, float* s, uint8_t* q_t, int64_t ldqt,
                               hipStream_t stream) {
    return quant_128x128_impl(w, w_dtype, rows, cols, ldw, q, ldq, s, q_t, ldqt, fp8q::kRuleFP32,
                              stream);
}

FP8Q_API int fp8_quant_128x128_pow2(const void* w, int w_dtype, int64_t rows, int64_t cols,
                                    int64_t ldw, uint8_t* q, int64_t ldq, float* s, uint8_t* q_t,
                                    int64_t ldqt, hipStream_t stream) {
    return quant_128x128_impl(w, w_dtype, rows, cols, ldw, q, ldq, s, q_t, ldqt, fp8q::kRulePow2,
                              stream);
}

namespace {

int check_gemm_common(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                      const uint8_t* b, int64_t ldb, const float* sb, void* c, int c_dtype,
                      int64_t ldc, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return FP8Q_EINVAL;
    if (c_dtype != FP8Q_F32 && c_dtype != FP8Q_BF16) return FP8Q_EINVAL;
    if (!a || !sa || !b || !sb || !c) return FP8Q_EINVAL;
    if (lda < K || ldb < K || ldc < N || ldsa < M) return FP8Q_EINVAL;
    if (K == 0 || K % 128 != 0) return FP8Q_EUNSUPPORTED;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16) || !aligned(sa, 4) ||
        !aligned(sb, 4))
        return FP8Q_EALIGN;
    if (lda % 16 != 0 || ldb % 16 != 0 || ldc % 4 != 0) return FP8Q_EALIGN;
    // the kernels address a 256-row tile with 32-bit byte offsets
    if (lda > (int64_t(1) << 24) || ldb > (int64_t(1) << 24)) return FP8Q_EUNSUPPORTED;
    return FP8Q_OK;
}

}  // namespace

namespace {

int gemm_impl(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
              int64_t ldb, const float* sb, int b_scale_mode, int64_t sbs0, int64_t sbs1, void* c,
              int c_dtype, int64_t ldc, int64_t M, int64_t N, int64_t K, bool pow2,
              hipStream_t stream) {
    if (M == 0 || N == 0) {
        if (M < 0 || N < 0) return FP8Q_EINVAL;
        return FP8Q_OK;
    }
    if (b_scale_mode != FP8Q_SCALE_BLOCK128 && b_scale_mode != FP8Q_SCALE_ROW128)
        return FP8Q_EINVAL;
    int st = check_gemm_common(a, lda, sa, ldsa, b, ldb, sb, c, c_dtype, ldc, M, N, K);
    if (st != FP8Q_OK) return st;
    if (sbs0 < 0 || sbs1 < 0) return FP8Q_EINVAL;
    if (b_scale_mode == FP8Q_SCALE_ROW128 && sbs0 < N) return FP8Q_EINVAL;
    if (b_scale_mode == FP8Q_SCALE_BLOCK128 && ((N + 127) / 128) * sbs0 > (int64_t(1) << 29))
        return FP8Q_EUNSUPPORTED;  // 32-bit byte offsets into sb
    // tiles of 256x256 (256x224 for some ROW128 shapes: counted with the
    // narrower width) are numbered with 32-bit indices
    if ((M + 255) / 256 * ((N + 223) / 224) > 0x7FFFFFFF) return FP8Q_EUNSUPPORTED;
    fp8q::GemmParams p{};
    p.a = a; p.lda = lda; p.sa = sa; p.ldsa = ldsa;
    p.b = b; p.ldb = ldb; p.sb = sb; p.sbs0 = sbs0; p.sbs1 = sbs1;
    p.c = c; p.ldc = ldc; p.M = M; p.N = N; p.K = K;
    return launch_status(fp8q::launch_gemm(p, b_scale_mode, c_dtype, pow2, stream));
}

int grouped_gemm_impl(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                      const uint8_t* b, int64_t ldb, const float* sb, const int32_t* offsets,
                      int64_t num_groups, int64_t M_total, void* c, int c_dtype, int64_t ldc,
                      int64_t N, int64_t K, bool pow2, hipStream_t stream) {
    if (num_groups <= 0 || M_total < 0 || N < 0) return FP8Q_EINVAL;
    if (M_total == 0 || N == 0) return FP8Q_OK;
    if (!offsets) return FP8Q_EINVAL;
    int st = check_gemm_common(a, lda, sa, ldsa, b, ldb, sb, c, c_dtype, ldc, M_total, N, K);
    if (st != FP8Q_OK) return st;
    if (!aligned(offsets, 4)) return FP8Q_EALIGN;
    if (num_groups > fp8q::kMaxGroups) return FP8Q_EUNSUPPORTED;
    if (M_total > 0x7FFFFFFF) return FP8Q_EUNSUPPORTED;  // offsets are int32
    if (((M_total + 255) / 256 + num_groups) * ((N + 255) / 256) > 0x7FFFFFFF)
        return FP8Q_EUNSUPPORTED;
    fp8q::GemmParams p{};
    p.a = a; p.lda = lda; p.sa = sa; p.ldsa = ldsa;
    p.b = b; p.ldb = ldb; p.sb = sb; p.sbs0 = K / 128; p.sbs1 = 1;
    p.c = c; p.ldc = ldc; p.M = M_total; p.N = N; p.K = K;
    p.offsets = offsets; p.num_groups = num_groups;
    return launch_status(fp8q::launch_grouped_gemm(p, c_dtype, pow2, stream));
}

}  // namespace

FP8Q_API int fp8_blockscaled_gemm(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                  const uint8_t* b, int64_t ldb, const float* sb,
                                  int b_scale_mode, int64_t sbs0, int64_t sbs1, void* c,
                                  int c_dtype, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                  hipStream_t stream) {
    return gemm_impl(a, lda, sa, ldsa, b, ldb, sb, b_scale_mode, sbs0, sbs1, c, c_dtype, ldc, M, N,
                     K, false, stream);
}

FP8Q_API int fp8_blockscaled_gemm_pow2(const uint8_t* a, int64_t lda, const float* sa,
                                       int64_t ldsa, const uint8_t* b, int64_t ldb,
                                       const float* sb, int b_scale_mode, int64_t sbs0,
                                       int64_t sbs1, void* c, int c_dtype, int64_t ldc, int64_t M,
                                       int64_t N, int64_t K, hipStream_t stream) {
    return gemm_impl(a, lda, sa, ldsa, b, ldb, sb, b_scale_mode, sbs0, sbs1, c, c_dtype, ldc, M, N,
                     K, true, stream);
}

FP8Q_API int fp8_grouped_gemm(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                              const uint8_t* b, int64_t ldb, const float* sb,
                              const int32_t* offsets, int64_t num_groups, int64_t M_total,
                              void* c, int c_dtype, int64_t ldc, int64_t N, int64_t K,
                              hipStream_t stream) {
    return grouped_gemm_impl(a, lda, sa, ldsa, b, ldb, sb, offsets, num_groups, M_total, c,
                             c_dtype, ldc, N, K, false, stream);
}

FP8Q_API int fp8_grouped_gemm_pow2(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                   const uint8_t* b, int64_t ldb, const float* sb,
                                   const int32_t* offsets, int64_t num_groups, int64_t M_total,
                                   void* c, int c_dtype, int64_t ldc, int64_t N, int64_t K,
                                   hipStream_t stream) {
    return grouped_gemm_impl(a, lda, sa, ldsa, b, ldb, sb, offsets, num_groups, M_total, c,
                             c_dtype, ldc, N, K, true, stream);
}

FP8Q_API int fp8_dispatch_rows(const uint8_t* q_src, int64_t ldq_src, const float* s_src,
                               int64_t lds_src, int64_t src_rows, const int32_t* index,
                               int64_t rows, int64_t cols, uint8_t* q_dst, int64_t ldq_dst,
                               float* s_dst, int64_t lds_dst, hipStream_t stream) {
    if (rows < 0 || cols < 0 || src_rows < 0) return FP8Q_EINVAL;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!q_src || !s_src || !index || !q_dst || !s_dst) return FP8Q_EINVAL;
    if (ldq_src < cols || ldq_dst < cols || lds_src < src_rows || lds_dst < rows)
        return FP8Q_EINVAL;
    if (!aligned(s_src, 4) || !aligned(s_dst, 4) || !aligned(index, 4)) return FP8Q_EALIGN;
    if ((rows + 255) / 256 * 8 > 0x7FFFFFFF) return FP8Q_EUNSUPPORTED;  // grid size
    fp8q::DispatchParams p{};
    p.q_src = q_src; p.ldq_src = ldq_src; p.s_src = s_src; p.lds_src = lds_src;
    p.src_rows = src_rows; p.index = index; p.rows = rows; p.cols = cols;
    p.q_dst = q_dst; p.ldq_dst = ldq_dst; p.s_dst = s_dst; p.lds_dst = lds_dst;
    p.vec = aligned(q_src, 16) && aligned(q_dst, 16) && ldq_src % 16 == 0 && ldq_dst % 16 == 0;
    return launch_status(fp8q::launch_dispatch_rows(p, stream));
}
