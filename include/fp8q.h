/*
 * fp8q.h -- C ABI of libfp8q: fine-grained FP8 quantization and the FP8
 * block-scaled GEMM on AMD MI355X (gfx950).
 *
 * The method is DeepSeek-V3's fine-grained FP8 scheme as the source pages
 * describe it (pages cited by title, or by site where untitled):
 *   - every GEMM operand is E4M3, 4 exponent and 3 mantissa bits, including
 *     the gradients of the backward GEMMs (jp-study.kr page, passage on the
 *     hybrid E4M3/E5M2 formats of prior work);
 *   - activations are scaled per 1x128 tile (one token, 128 channels),
 *     weights per 128x128 block (128 input x 128 output channels)
 *     ("Should Fixing Deepseek Take 60 Steps?", Figure 7(a));
 *   - each tile's or block's largest magnitude is measured at quantization
 *     time and mapped onto the largest E4M3 value (why-be.why-be.co.kr page,
 *     passage after Figure 7(a); "Should Fixing Deepseek Take 60 Steps?", the
 *     max-abs scaling passage);
 *   - the GEMM consumes FP8 operands and writes BF16 or FP32 ("Should Fixing
 *     Deepseek Take 60 Steps?", GEMM passage before Figure 7(a)); partial
 *     sums are moved into FP32 at intervals and scaled there ("promotion",
 *     jp-study.kr page, Figure 7(b)); Fprop, Dgrad and Wgrad all run in FP8
 *     (Figure 6 on both pages).
 *
 * Numeric contract (the pages leave these open; this library fixes them):
 *   - E4M3 means OCP E4M3FN: bias 7, largest finite 448, no infinities;
 *   - per group: s = amax / 448 and inv = min(448 / amax, FLT_MAX), both IEEE
 *     single-precision divisions; each code is the round-to-nearest-even,
 *     sign-preserving, saturating (+-448) encoding of the FP32 product x*inv;
 *     the stored scale s is the dequantization factor (x ~= decode(q) * s);
 *   - an all-zero group gets s = +0.0 and codes 0x00 / 0x80 (sign kept);
 *   - GEMM results follow sum_kb (sa*sb) * sum_{k in kb} decode(a)*decode(b)
 *     with FP32 accumulation; the summation order inside a K block is the
 *     matrix core's, so results are not bit-reproducible against another
 *     implementation, only run to run.
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or synchronizes and keeps no state; calls are
 *     reentrant and asynchronous on `stream` (NULL = the default stream).
 *   - Inputs are read only.  Outputs are overwritten inside their logical
 *     extent; padding between rows (leading dimensions) is never written.
 *   - Return value: FP8Q_OK, or an error status.  Arguments are validated on
 *     the host before any HIP call (FP8Q_EINVAL, FP8Q_EALIGN,
 *     FP8Q_EUNSUPPORTED); FP8Q_EHIP reports a failed kernel launch.  Faults
 *     inside a kernel surface at the caller's next synchronization.
 *   - Zero-sized problems (rows or cols == 0; M or N == 0) return FP8Q_OK and
 *     launch nothing.
 *   - Results are bitwise reproducible from run to run (no atomics, no
 *     split-K).
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    FP8Q_OK = 0,
    FP8Q_EINVAL = 1,       /* null pointer, negative size, bad enum, ld < width */
    FP8Q_EALIGN = 2,       /* pointer or leading dimension misaligned          */
    FP8Q_EUNSUPPORTED = 3, /* shape the kernels do not handle (e.g. K % 128)   */
    FP8Q_EHIP = 4          /* kernel launch failed                             */
};

/* Element types of quantizer inputs and GEMM outputs. */
enum { FP8Q_F32 = 0, FP8Q_BF16 = 1 };

/* Granularity of the GEMM's B-operand scales. */
enum {
    FP8Q_SCALE_BLOCK128 = 0, /* one scale per 128(N) x 128(K) block of B   */
    FP8Q_SCALE_ROW128 = 1    /* one scale per row n of B per 128 K         */
};

/*
 * fp8_quant_1x128 -- 1x128 tile quantization of activations
 * ("Should Fixing Deepseek Take 60 Steps?", Figure 7(a)).
 *
 * Quantizes the logical matrix X[rows, cols] whose element (r, c) is
 * x[r*xs_r + c*xs_c] (elements of type x_dtype), in groups of 128
 * consecutive columns of one row: group g of row r covers columns
 * [128g, min(128g+128, cols)).
 *   q : uint8 codes, q[r*ldq + c] for r < rows, c < cols; ldq >= cols.
 *   s : FP32 scales, s[g*lds + r] for g < ceil(cols/128); lds >= rows.
 * Exactly one of xs_r, xs_c must be 1:
 *   xs_c == 1 -- row-contiguous input (activation X[tokens, channels]);
 *                requires xs_r >= cols.
 *   xs_r == 1 -- the input is stored transposed (X^T with row pitch xs_c),
 *                i.e. 128x1 groups along the stored tensor's rows, with the
 *                codes written transposed: used for the weight-gradient GEMM,
 *                whose reduction runs over tokens; requires xs_c >= rows.
 * Alignment: x aligned to its element size, s to 4 bytes, else FP8Q_EALIGN.
 * Any pitch is accepted; the kernel uses 16-byte loads where x and its
 * pitch are 16-byte aligned and 8-byte code stores where q and ldq are
 * 8-byte aligned, element accesses otherwise (slower).
 * Size limits (else FP8Q_EUNSUPPORTED): row-contiguous input at most 2^24
 * groups per row (cols <= 2^31); transposed input fewer than 2^31 128x128
 * tiles.
 */
int fp8_quant_1x128(const void* x, int x_dtype, int64_t rows, int64_t cols,
                    int64_t xs_r, int64_t xs_c, uint8_t* q, int64_t ldq,
                    float* s, int64_t lds, hipStream_t stream);

/*
 * fp8_quant_128x128 -- 128x128 block quantization of weights
 * ("Should Fixing Deepseek Take 60 Steps?", Figure 7(a)).
 *
 * W[rows, cols] row-major with leading dimension ldw (elements, >= cols).
 * Block (i, j) covers rows [128i, 128i+128) x cols [128j, 128j+128), clipped
 * at the edges.
 *   q   : q[r*ldq + c] uint8 codes, ldq >= cols.
 *   s   : s[i*ceil(cols/128) + j] FP32 block scales (dense, row-major).
 *   q_t : optional (NULL to skip) transposed codes q_t[c*ldqt + r],
 *         ldqt >= rows -- the weight operand of the input-gradient GEMM,
 *         whose reduction runs over the weight's rows.  The block grid is
 *         symmetric under transposition, so q_t uses the same scales, read
 *         as s[j + i*ceil(cols/128)] by the GEMM's scale strides.
 * Alignment: w aligned to its element size, s to 4 bytes, else FP8Q_EALIGN;
 * pitches as for fp8_quant_1x128 (vector accesses where aligned).
 * Size limit (else FP8Q_EUNSUPPORTED): fewer than 2^31 128x128 blocks.
 */
int fp8_quant_128x128(const void* w, int w_dtype, int64_t rows, int64_t cols,
                      int64_t ldw, uint8_t* q, int64_t ldq, float* s,
                      uint8_t* q_t, int64_t ldqt, hipStream_t stream);

/*
 * fp8_blockscaled_gemm -- C[M, N] = A[M, K] * B[N, K]^T on E4M3 operands
 * with FP32 promotion of every 128-wide K interval (jp-study.kr page,
 * Figure 7(b)); serves the Fprop, Dgrad and Wgrad shapes of a linear layer
 * (Figure 6).
 *
 *   a  : E4M3 codes, a[m*lda + k]; lda >= K, multiple of 16; 16-B aligned.
 *   sa : activation (1x128) scales, sa[kb*ldsa + m], kb = k/128;
 *        ldsa >= M.
 *   b  : E4M3 codes, b[n*ldb + k]; ldb >= K, multiple of 16; 16-B aligned.
 *   sb : B scales.  FP8Q_SCALE_BLOCK128: sb[(n/128)*sbs0 + kb*sbs1]
 *        (a 128x128-block weight scale, strides allow the transposed read);
 *        FP8Q_SCALE_ROW128: sb[kb*sbs0 + n] (sbs1 ignored; sbs0 >= N).
 *   c  : output, c[m*ldc + n], element type c_dtype (FP8Q_BF16: round to
 *        nearest even; FP8Q_F32); ldc >= N and a multiple of 4; 16-B aligned.
 *   K  : a positive multiple of 128, else FP8Q_EUNSUPPORTED.
 * lda and ldb above 2^24 bytes return FP8Q_EUNSUPPORTED.
 * For every element: acc = sum over kb of (sa[m,kb]*sb[n,kb]) * P_kb, where
 * P_kb is the FP32 partial sum of the 128 products of the K block.
 */
int fp8_blockscaled_gemm(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                         const uint8_t* b, int64_t ldb, const float* sb, int b_scale_mode,
                         int64_t sbs0, int64_t sbs1,
                         void* c, int c_dtype, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * fp8_grouped_gemm -- per-group (MoE expert) block-scaled GEMM: the FP8
 * forward GEMM of the MoE up-projection, whose activations are quantized
 * before being dispatched to the experts (jp-study.kr page, passage on
 * quantizing before the MoE up-projection).
 *
 * Group g owns rows [offsets[g], offsets[g+1]) of A and C and multiplies
 * them with its own weight B_g = b + g*N*ldb (E4M3 codes [N, K], row pitch
 * ldb) scaled per 128x128 block by sb_g = sb + g*ceil(N/128)*(K/128), laid
 * out [n/128][kb].
 *   offsets : DEVICE int32[num_groups+1]; offsets[0] = 0, non-decreasing,
 *             offsets[num_groups] = M_total.  Read on the device (no host
 *             synchronization); a sequence violating this is undefined
 *             behaviour.  Empty groups are allowed.
 *   a, sa   : as fp8_blockscaled_gemm with M = M_total.
 *   c       : c[m*ldc + n] for m < M_total, n < N.
 * Alignment and K rules as fp8_blockscaled_gemm.
 */
int fp8_grouped_gemm(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                     const uint8_t* b, int64_t ldb, const float* sb,
                     const int32_t* offsets, int64_t num_groups, int64_t M_total,
                     void* c, int c_dtype, int64_t ldc, int64_t N, int64_t K,
                     hipStream_t stream);

/*
 * Power-of-two (E8M0) scale variant.  The pages ask for matrix hardware that
 * takes the fine-grained group scales and applies them inside the multiply,
 * instead of promoting partial sums (why-be.why-be.co.kr page,
 * hardware-design passage).  gfx950's scaled FP8 matrix instruction does
 * this, with scales that are exponents only (E8M0).  The four calls below
 * are the same operations as their FP32-scale counterparts, with:
 *   - quantizers: each group's scale is s = 2^e, e the smallest integer with
 *     amax <= 448 * 2^e, clamped to [-127, 127] (an all-zero group gets
 *     2^-127), and the codes are encode(x * 2^-e) (exact scaling, then the
 *     same round-to-nearest-even saturating E4M3 encoding).  Scales are still
 *     stored as FP32 values, in the same layouts;
 *   - GEMMs: every A and B scale must be such a power of two (the mantissa
 *     bits of each scale are ignored).  The matrix instruction applies them
 *     per 32-wide K group and accumulates across K blocks in its FP32
 *     accumulator: no separate promotion step.  Result: sum over kb of
 *     (sa*sb) * P_kb as for fp8_blockscaled_gemm.
 * Arguments, layouts, alignment and error statuses are those of the
 * corresponding call above.
 */
int fp8_quant_1x128_pow2(const void* x, int x_dtype, int64_t rows, int64_t cols,
                         int64_t xs_r, int64_t xs_c, uint8_t* q, int64_t ldq,
                         float* s, int64_t lds, hipStream_t stream);
int fp8_quant_128x128_pow2(const void* w, int w_dtype, int64_t rows, int64_t cols,
                           int64_t ldw, uint8_t* q, int64_t ldq, float* s,
                           uint8_t* q_t, int64_t ldqt, hipStream_t stream);
int fp8_blockscaled_gemm_pow2(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                              const uint8_t* b, int64_t ldb, const float* sb,
                              int b_scale_mode, int64_t sbs0, int64_t sbs1,
                              void* c, int c_dtype, int64_t ldc,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream);
int fp8_grouped_gemm_pow2(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                          const uint8_t* b, int64_t ldb, const float* sb,
                          const int32_t* offsets, int64_t num_groups, int64_t M_total,
                          void* c, int c_dtype, int64_t ldc, int64_t N, int64_t K,
                          hipStream_t stream);

/*
 * fp8_dispatch_rows -- FP8 dispatch permutation.  The activations of the MoE
 * up-projection are quantized once per token and dispatched to the experts
 * in FP8, with their scales (jp-study.kr page, passage on quantizing before
 * the MoE up-projection and dispatching in FP8).  This call builds the
 * expert-ordered operand of fp8_grouped_gemm from the token-ordered output
 * of fp8_quant_1x128.  For r < rows, with t = index[r]:
 *   q_dst[r*ldq_dst + c] = q_src[t*ldq_src + c]   for c < cols;
 *   s_dst[g*lds_dst + r] = s_src[g*lds_src + t]   for g < ceil(cols/128).
 *   index : DEVICE int32[rows].  Entries outside [0, src_rows) are skipped:
 *           that output row and its scales are left unwritten (no fault).
 *   ldq_src, ldq_dst >= cols; lds_src >= src_rows; lds_dst >= rows.
 * The source and destination must not overlap.
 * Alignment: s_src, s_dst and index 4-byte aligned, else FP8Q_EALIGN.  Rows
 * move with 16-byte accesses when both code pointers and both pitches are
 * 16-byte aligned, byte accesses otherwise (slower).
 */
int fp8_dispatch_rows(const uint8_t* q_src, int64_t ldq_src, const float* s_src,
                      int64_t lds_src, int64_t src_rows, const int32_t* index,
                      int64_t rows, int64_t cols, uint8_t* q_dst, int64_t ldq_dst,
                      float* s_dst, int64_t lds_dst, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* fp8q_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
