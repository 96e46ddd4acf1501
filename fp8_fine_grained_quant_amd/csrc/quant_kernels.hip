// quant_kernels.hip -- fine-grained E4M3 quantizers for gfx950.
//
// Method: activations are scaled per 1x128 tile and weights per 128x128
// block; each group's largest magnitude is found at quantization time and
// mapped onto the largest E4M3 value ("Should Fixing Deepseek Take 60
// Steps?", Figure 7(a); why-be.why-be.co.kr page, passage after Figure 7(a)).
// The exact scale rule and rounding are the library contract stated in
// include/fp8q.h.
//
// All three kernels are HBM-bound streaming kernels: every input byte is read
// once, every output byte written once, with 16-byte vector accesses on the
// interior and element-guarded accesses on ragged edges.
//
//  quant_rows_kernel  -- 1x128 groups along a contiguous row.  One 16-lane
//                        DPP row per group (8 elements per lane), so the
//                        group max is a 4-step row_ror reduction with no LDS.
//  quant_tile_kernel  -- 128x128 input tiles, thread (a, b) of 256 owning the
//                        8x8 sub-tile rows 8a..8a+7, cols 8b..8b+7:
//                        MODE_BLOCK: one scale per tile (weights), codes
//                        stored row-major and/or transposed;
//                        MODE_COLS: one scale per column over the tile's 128
//                        rows (128x1 groups for the weight-gradient GEMM),
//                        codes stored transposed.
//                        The transposed store is an 8x8 byte transpose in
//                        registers, so each thread writes 8-byte runs and
//                        the 16 threads of a column run write 128 bytes.
#include "device_common.h"
#include "kernels.h"

namespace fp8q {

// group loads in flight per lane in the 1x128 row kernel
constexpr int kRowUnroll = 4;

// ---------------------------------------------------------------------------
// 1x128 groups along contiguous rows
// ---------------------------------------------------------------------------

// Streaming 16-byte load: every input byte is read exactly once, so the
// non-temporal hint keeps it from displacing reusable cache lines.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Loads the 8 elements [c0, c0+8) of a row as FP32; elements at or beyond
// `cols` read as 0 (they do not change the group max and are not stored).
// `vec`: the row start is 16-byte aligned, so full runs use vector loads.
template <int DT>
__device__ __forceinline__ void load8(const void* row, int64_t c0, int64_t cols, float v[8],
                                      bool vec) {
    if (vec && c0 + 8 <= cols) {
        if (DT == kBF16) {
            uint4 u = ld_stream16(static_cast<const uint16_t*>(row) + c0);
            uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_bits_to_float(w[i] & 0xFFFFu);
                v[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
            }
        } else {
            const float* p = static_cast<const float*>(row) + c0;
            const uint4 a = ld_stream16(p), b = ld_stream16(p + 4);
            v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
            v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
            v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
            v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int64_t c = c0 + i;
            if (c < cols) {
                v[i] = DT == kBF16 ? bf16_bits_to_float(static_cast<const uint16_t*>(row)[c])
                                   : static_cast<const float*>(row)[c];
            } else {
                v[i] = 0.0f;
            }
        }
    }
}

// Stores the 8 code bytes of [c0, c0+8) (those below `cols`); `vec`: the
// row start is 8-byte aligned, so full runs use one 8-byte store.  Plain
// (temporal) stores: the codes are read next by the GEMM, and kept in the
// memory-side cache they need not come back from HBM (measured: the Fprop
// GEMM after the quantizers runs ~1-2 % faster than after non-temporal
// stores).
__device__ __forceinline__ void store8(uint8_t* row, int64_t c0, int64_t cols, uint32_t lo,
                                       uint32_t hi, bool vec) {
    if (vec && c0 + 8 <= cols) {
        *reinterpret_cast<uint2*>(row + c0) = make_uint2(lo, hi);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (c0 + i < cols) row[c0 + i] = (uint8_t)((i < 4 ? lo >> (8 * i) : hi >> (8 * (i - 4))) & 0xFF);
        }
    }
}

// One group: 16 lanes x 8 elements.  Every lane of the DPP row takes part.
template <int DT, int RULE>
__device__ __forceinline__ void quant_group_1x128(const float v[8], uint8_t* qrow, int64_t c0,
                                                  int64_t cols, float* s_out, bool lead,
                                                  bool vout) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(fabsf(v[i])));
    m = row16_max_u32(m);
    float s, inv;
    group_scale_rule<RULE>(__uint_as_float(m), s, inv);
    uint32_t lo = enc4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    uint32_t hi = enc4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    store8(qrow, c0, cols, lo, hi, vout);
    if (lead) *s_out = s;
}

// Grid: blocks of 4 waves; wave w of block b handles rows b*4+w (grid-strided);
// within a row, the 4 DPP rows (slices) of the wave take groups g = slice,
// slice+4, ... so one wave-load covers 4 consecutive groups (1 KB of BF16).
template <int DT, int RULE>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ x, int64_t rows,
                                                         int64_t cols, int64_t ldx,
                                                         uint8_t* __restrict__ q, int64_t ldq,
                                                         float* __restrict__ s, int64_t lds,
                                                         bool vin, bool vout) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int slice = lane >> 4;
    const int sl = lane & 15;
    const int64_t groups = (cols + 127) >> 7;
    const size_t esz = DT == kBF16 ? 2 : 4;
    for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < rows; r += (int64_t)gridDim.x * 4) {
        const void* xr = static_cast<const char*>(x) + (size_t)r * (size_t)ldx * esz;
        uint8_t* qr = q + r * ldq;
        // kRowUnroll group loads in flight per lane before any is consumed
        for (int64_t g0 = 0; g0 < groups; g0 += 4 * kRowUnroll) {
            float v[kRowUnroll][8];
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int64_t g = g0 + 4 * u + slice;
                if (g < groups) load8<DT>(xr, g * 128 + sl * 8, cols, v[u], vin);
            }
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int64_t g = g0 + 4 * u + slice;
                if (g < groups)
                    quant_group_1x128<DT, RULE>(v[u], qr, g * 128 + sl * 8, cols, s + g * lds + r, sl == 0,
                                          vout);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 128x128 tiles: block scales (weights) or column scales (128x1 groups)
// ---------------------------------------------------------------------------

// Reads the 8x8 sub-tile rows r0..r0+7, cols c0..c0+7 of a row-major matrix;
// elements outside [rows, cols] read as 0.
template <int DT>
__device__ __forceinline__ void load_8x8(const void* x, int64_t ldx, int64_t rows, int64_t cols,
                                         int64_t r0, int64_t c0, float v[8][8], bool vin) {
    const size_t esz = DT == kBF16 ? 2 : 4;
    const bool full = (r0 + 8 <= rows) && (c0 + 8 <= cols);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const void* row = static_cast<const char*>(x) + (size_t)(r0 + p) * (size_t)ldx * esz;
        if (full) {
            load8<DT>(row, c0, cols, v[p], vin);
        } else if (r0 + p < rows) {
            load8<DT>(row, c0, cols, v[p], vin);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[p][j] = 0.0f;
        }
    }
}

// Byte j of the 8-byte row code (lo: bytes 0..3, hi: bytes 4..7).
__device__ __forceinline__ uint32_t code_byte(uint32_t lo, uint32_t hi, int j) {
    return ((j < 4 ? lo >> (8 * j) : hi >> (8 * (j - 4)))) & 0xFFu;
}

template <int DT, int MODE, int RULE>
__global__ __launch_bounds__(256) void quant_tile_kernel(const void* __restrict__ x, int64_t rows,
                                                         int64_t cols, int64_t ldx,
                                                         uint8_t* __restrict__ q, int64_t ldq,
                                                         uint8_t* __restrict__ qt, int64_t ldqt,
                                                         float* __restrict__ s, int64_t lds,
                                                         int64_t tiles_c, bool vin, bool vq,
                                                         bool vqt) {
    __shared__ uint32_t red[4 * 128];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int a = tid >> 4;   // sub-tile row group 0..15
    const int b = tid & 15;   // sub-tile col group 0..15
    const int64_t ti = blockIdx.x / tiles_c;
    const int64_t tj = blockIdx.x - ti * tiles_c;
    const int64_t r0 = ti * 128 + 8 * a;
    const int64_t c0 = tj * 128 + 8 * b;

    float v[8][8];
    load_8x8<DT>(x, ldx, rows, cols, r0, c0, v, vin);

    float inv[8];
    if (MODE == kTileBlock) {
        uint32_t m = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p)
#pragma unroll
            for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(fabsf(v[p][j])));
        m = row16_max_u32(m);
        m = max(m, (uint32_t)__shfl_xor((int)m, 16));
        m = max(m, (uint32_t)__shfl_xor((int)m, 32));
        if ((tid & 63) == 0) red[wave] = m;
        __syncthreads();
        m = max(max(red[0], red[1]), max(red[2], red[3]));
        float sc, iv;
        group_scale_rule<RULE>(__uint_as_float(m), sc, iv);
        if (tid == 0) s[ti * tiles_c + tj] = sc;
#pragma unroll
        for (int j = 0; j < 8; ++j) inv[j] = iv;
    } else {
        // per-column max over the tile's 128 rows
        uint32_t m[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            m[j] = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p) m[j] = max(m[j], __float_as_uint(fabsf(v[p][j])));
            m[j] = max(m[j], (uint32_t)__shfl_xor((int)m[j], 16));
            m[j] = max(m[j], (uint32_t)__shfl_xor((int)m[j], 32));
        }
        if ((tid & 63) < 16) {
#pragma unroll
            for (int j = 0; j < 8; ++j) red[wave * 128 + 8 * b + j] = m[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = 8 * b + j;
            uint32_t mm = max(max(red[c], red[128 + c]), max(red[256 + c], red[384 + c]));
            float sc, iv;
            group_scale_rule<RULE>(__uint_as_float(mm), sc, iv);
            inv[j] = iv;
            // logical output row = input column; scale index [tile row][column]
            if (a == 0 && c0 + j < cols) s[ti * lds + c0 + j] = sc;
        }
    }

    // codes: row p of the sub-tile as two dwords
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        lo[p] = enc4(v[p][0] * inv[0], v[p][1] * inv[1], v[p][2] * inv[2], v[p][3] * inv[3]);
        hi[p] = enc4(v[p][4] * inv[4], v[p][5] * inv[5], v[p][6] * inv[6], v[p][7] * inv[7]);
    }

    if (q != nullptr) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            if (r0 + p < rows) store8(q + (r0 + p) * ldq, c0, cols, lo[p], hi[p], vq);
        }
    }
    if (qt != nullptr) {
        // transposed: output row c0+j holds bytes of input rows r0..r0+7
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t tlo = 0, thi = 0;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                tlo |= code_byte(lo[p], hi[p], j) << (8 * p);
                thi |= code_byte(lo[p + 4], hi[p + 4], j) << (8 * p);
            }
            if (c0 + j < cols) store8(qt + (c0 + j) * ldqt, r0, rows, tlo, thi, vqt);
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static bool is_aligned(const void* p, uintptr_t a) {
    return reinterpret_cast<uintptr_t>(p) % a == 0;
}

hipError_t launch_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds, int rule,
                             hipStream_t stream) {
    int64_t blocks = (rows + 3) / 4;
    if (blocks > 65536 * 8) blocks = 65536 * 8;
    dim3 grid((unsigned)blocks), block(256);
    const int64_t esz = dtype == kBF16 ? 2 : 4;
    const bool vin = is_aligned(x, 16) && (ldx * esz) % 16 == 0;
    const bool vout = is_aligned(q, 8) && ldq % 8 == 0;
#define FP8Q_LAUNCH_ROWS(DT, RL)                                                               \
    hipLaunchKernelGGL((quant_rows_kernel<DT, RL>), grid, block, 0, stream, x, rows, cols, ldx, q, \
                       ldq, s, lds, vin, vout)
    if (dtype == kBF16) {
        if (rule == kRulePow2) FP8Q_LAUNCH_ROWS(kBF16, kRulePow2);
        else FP8Q_LAUNCH_ROWS(kBF16, kRuleFP32);
    } else {
        if (rule == kRulePow2) FP8Q_LAUNCH_ROWS(kF32, kRulePow2);
        else FP8Q_LAUNCH_ROWS(kF32, kRuleFP32);
    }
#undef FP8Q_LAUNCH_ROWS
    return hipGetLastError();
}

hipError_t launch_quant_tiles(const void* x, int dtype, int mode, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                              float* s, int64_t lds, int rule, hipStream_t stream) {
    const int64_t tr = (rows + 127) / 128, tc = (cols + 127) / 128;
    dim3 grid((unsigned)(tr * tc)), block(256);
    const int64_t esz = dtype == kBF16 ? 2 : 4;
    const bool vin = is_aligned(x, 16) && (ldx * esz) % 16 == 0;
    const bool vq = q != nullptr && is_aligned(q, 8) && ldq % 8 == 0;
    const bool vqt = qt != nullptr && is_aligned(qt, 8) && ldqt % 8 == 0;
#define FP8Q_LAUNCH_TILE(DT, MD, RL)                                                     \
    hipLaunchKernelGGL((quant_tile_kernel<DT, MD, RL>), grid, block, 0, stream, x, rows, cols, \
                       ldx, q, ldq, qt, ldqt, s, lds, tc, vin, vq, vqt)
#define FP8Q_LAUNCH_TILE_RULE(DT, MD)                          \
    do {                                                       \
        if (rule == kRulePow2) FP8Q_LAUNCH_TILE(DT, MD, kRulePow2); \
        else FP8Q_LAUNCH_TILE(DT, MD, kRuleFP32);              \
    } while (0)
    if (dtype == kBF16) {
        if (mode == kTileBlock) FP8Q_LAUNCH_TILE_RULE(kBF16, kTileBlock);
        else FP8Q_LAUNCH_TILE_RULE(kBF16, kTileCols);
    } else {
        if (mode == kTileBlock) FP8Q_LAUNCH_TILE_RULE(kF32, kTileBlock);
        else FP8Q_LAUNCH_TILE_RULE(kF32, kTileCols);
    }
#undef FP8Q_LAUNCH_TILE_RULE
#undef FP8Q_LAUNCH_TILE
    return hipGetLastError();
}

}  // namespace fp8q
