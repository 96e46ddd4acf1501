// kernels.h -- internal launchers of libfp8q (host side).  Arguments are
// assumed validated by fp8q_api.hip; every launcher returns the HIP error of
// the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

enum { kF32 = 0, kBF16 = 1 };
enum { kTileBlock = 0, kTileCols = 1, kTileRows = 2 };
enum { kScaleBlock128 = 0, kScaleRow128 = 1 };
// Group scale rules: s = amax/448 (FP32), or the power of two 2^e with e the
// smallest integer such that amax <= 448 * 2^e (an E8M0 exponent).
enum { kRuleFP32 = 0, kRulePow2 = 1 };

// 1x128 groups along contiguous rows of x[rows, cols] (row pitch ldx elements).
// rule: kRuleFP32 (s = amax/448) or kRulePow2 (s = the power of two an E8M0
// exponent carries), as in device_common.h.
hipError_t launch_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds, int rule,
                             hipStream_t stream);

// 128x128 tiles of x[rows, cols] (row pitch ldx).  kTileBlock: one scale per
// tile, s[ti*ceil(cols/128)+tj], codes to q (row-major) and/or qt
// (transposed).  kTileCols: one scale per column per 128 rows,
// s[ti*lds + col], codes to qt only (128x256 tiles).  kTileRows: one scale per row per 128
// columns (1x128 groups), s[tj*lds + row], codes to q only.
hipError_t launch_quant_tiles(const void* x, int dtype, int mode, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                              float* s, int64_t lds, int rule, hipStream_t stream);

struct GemmParams {
    const uint8_t* a;
    int64_t lda;
    const float* sa;
    int64_t ldsa;
    const uint8_t* b;
    int64_t ldb;
    const float* sb;
    int64_t sbs0, sbs1;
    void* c;
    int64_t ldc;
    int64_t M, N, K;
    // grouped GEMM only
    const int32_t* offsets;
    int64_t num_groups;
};

// pow2: the A and B scales are powers of two applied by the matrix
// instruction (E8M0 exponents) instead of an FP32 promotion per K block.
hipError_t launch_gemm(const GemmParams& p, int scale_mode, int out_dtype, bool pow2,
                       hipStream_t stream);
hipError_t launch_grouped_gemm(const GemmParams& p, int out_dtype, bool pow2, hipStream_t stream);

// FP8 dispatch permutation: q_dst row r = q_src row index[r] (rows whose
// index lies outside [0, src_rows) are skipped), scales likewise.  vec: both
// code pointers and pitches are 16-byte aligned.
struct DispatchParams {
    const uint8_t* q_src;
    int64_t ldq_src;
    const float* s_src;
    int64_t lds_src;
    int64_t src_rows;
    const int32_t* index;
    int64_t rows, cols;
    uint8_t* q_dst;
    int64_t ldq_dst;
    float* s_dst;
    int64_t lds_dst;
    bool vec;
};

hipError_t launch_dispatch_rows(const DispatchParams& p, hipStream_t stream);

// Largest group count the grouped GEMM's on-chip tile table holds.
constexpr int64_t kMaxGroups = 4096;

}  // namespace fp8q
