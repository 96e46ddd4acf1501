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
//  quant_rows_kernel  -- 1x128 groups along contiguous rows.  One 16-lane
//                        DPP row per group (8 elements per lane), so the
//                        group max is a 4-step row_ror reduction with no
//                        LDS; a grid of resident waves strides over the
//                        groups.
//  quant_tile_kernel  -- 128x128 input tiles, thread (a, b) of 256 owning the
//                        8x8 sub-tile rows 8a..8a+7, cols 8b..8b+7:
//                        kTileBlock: one scale per tile (weights), codes
//                        stored row-major and/or transposed;
//                        kTileRows: 32x128 tiles, one scale per row (1x128
//                        groups, the 16 lanes of a DPP row), codes stored
//                        row-major -- the 1x128 quantizer on matrices of
//                        128 rows or more.
//                        The transposed copy of kTileBlock goes through LDS,
//                        so that every wave writes whole 128-byte runs of
//                        output rows.
//  quant_cols_kernel  -- 128x1 groups (one scale per column over 128 rows,
//                        for the weight-gradient GEMM), codes stored
//                        transposed: 128x256 tiles, one 128x64 strip per
//                        wave, a column's 128 rows in one wave, and each
//                        lane's 16 codes of a column one 16-byte run of its
//                        output row.
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace fp8q {

// group loads in flight per lane in the 1x128 row kernel
constexpr int kRowUnroll = 2;

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

// Eight consecutive elements of a row, as raw 16-byte runs (BF16: one run,
// FP32: two).  Loading is split from unpacking so that a thread issues all
// of its loads before it consumes any: a load whose result is used right
// away would make every load of the thread wait for the one before.
struct Run8 {
    uint4 a, b;
};
template <int DT>
__device__ __forceinline__ void issue8(const void* row, int64_t c0, Run8& r) {
    if (DT == kBF16) {
        r.a = ld_stream16(static_cast<const uint16_t*>(row) + c0);
    } else {
        const float* p = static_cast<const float*>(row) + c0;
        r.a = ld_stream16(p);
        r.b = ld_stream16(p + 4);
    }
}
template <int DT>
__device__ __forceinline__ void unpack8(const Run8& r, float v[8]) {
    if (DT == kBF16) {
        const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_float(w[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
        }
    } else {
        v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
        v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
        v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
        v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
    }
}
// Element-wise fallback (unaligned rows, ragged edges): [c0, c0+8) as FP32,
// elements at or beyond `cols` read as 0 (they change neither the group
// max nor any stored code).
template <int DT>
__device__ __forceinline__ void load8_elems(const void* row, int64_t c0, int64_t cols, float v[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t c = c0 + i;
        v[i] = c < cols ? (DT == kBF16 ? bf16_bits_to_float(static_cast<const uint16_t*>(row)[c])
                                       : static_cast<const float*>(row)[c])
                        : 0.0f;
    }
}

// Stores the 8 code bytes of [c0, c0+8) (those below `cols`); `vec`: the
// row start is 8-byte aligned, so full runs use one 8-byte store.  Plain
// (temporal) stores by default: the codes are read next by the GEMM, and
// kept in the memory-side cache they need not come back from HBM (measured:
// the Fprop GEMM after the quantizers runs ~1-2 % faster than after
// non-temporal stores).  `nt`: non-temporal, for outputs too large for that
// cache.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8(uint8_t* row, int64_t c0, int64_t cols, uint32_t lo,
                                       uint32_t hi, bool vec, bool nt = false) {
    if (vec && c0 + 8 <= cols) {
        if (nt) __builtin_nontemporal_store((u32x2){lo, hi}, reinterpret_cast<u32x2*>(row + c0));
        else *reinterpret_cast<uint2*>(row + c0) = make_uint2(lo, hi);
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
    const uint32_t lo = enc4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t hi = enc4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    store8(qrow, c0, cols, lo, hi, vout);
    if (lead) *s_out = s;
}

// Division by a launch constant d (the groups per row) as a multiply-high:
// n / d = (umulhi(n, m) + n) >> l for every 32-bit n, with l = ceil(log2 d)
// and m = floor(2^32 (2^l - d) / d) + 1 (Granlund and Montgomery, "Division
// by invariant integers using multiplication", 1994).
struct DivMagic {
    uint32_t m, l;
};
__device__ __forceinline__ uint32_t div_magic(uint32_t n, DivMagic d) {
    return (uint32_t)(((uint64_t)__umulhi(n, d.m) + n) >> d.l);
}

// Groups are numbered in bands of 4 rows, gi = (band * gpr + g) * 4 + rsub
// (gpr groups per row, fewer than 2^31 per launch), so the 4 slices of a
// wave (slice = lane / 16) take group g of 4 consecutive rows: each reads a
// 256-byte row run and their 4 scales S[g][r..r+3] go out as one 16-byte
// run (row-major numbering wrote every scale to a line of its own).  The
// grid is a few resident rounds of waves striding over the groups; a wave
// takes kRowUnroll such steps per pass (groups g, g+1, ...), issuing all of
// its loads before it consumes any, and every wave gets the same share
// however the rows fall.  Rows past the last one in the final band are
// skipped.
template <int DT, int RULE>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ x, int64_t cols,
                                                         int64_t ldx, uint8_t* __restrict__ q,
                                                         int64_t ldq, float* __restrict__ s,
                                                         int64_t lds, uint32_t total, uint32_t gpr,
                                                         DivMagic dm, bool vin, bool vout, uint32_t nrows) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int slice = lane >> 4;
    const int sl = lane & 15;
    const size_t esz = DT == kBF16 ? 2 : 4;
    const uint32_t step = gridDim.x * 4u * 4u * kRowUnroll;
    for (uint32_t base = (blockIdx.x * 4u + wave) * 4u * kRowUnroll; base < total; base += step) {
        Run8 raw[kRowUnroll];
        uint32_t rr[kRowUnroll], gg[kRowUnroll];
        bool vec[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            // bands of 4 rows: gi = (band * gpr + g) * 4 + rsub
            const uint32_t gi = base + 4 * u + slice;
            const uint32_t bg = gi >> 2;
            const uint32_t band = div_magic(bg, dm);
            gg[u] = bg - band * gpr;
            rr[u] = band * 4 + (gi & 3);
            const int64_t c0 = (int64_t)gg[u] * 128 + sl * 8;
            vec[u] = vin && gi < total && rr[u] < nrows && c0 + 8 <= cols;
            if (vec[u]) issue8<DT>(static_cast<const char*>(x) + (size_t)rr[u] * (size_t)ldx * esz, c0, raw[u]);
        }
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
            const uint32_t gi = base + 4 * u + slice;
            if (gi >= total || rr[u] >= nrows) continue;
            const int64_t c0 = (int64_t)gg[u] * 128 + sl * 8;
            float v[8];
            if (vec[u]) unpack8<DT>(raw[u], v);
            else load8_elems<DT>(static_cast<const char*>(x) + (size_t)rr[u] * (size_t)ldx * esz, c0, cols, v);
            quant_group_1x128<DT, RULE>(v, q + (int64_t)rr[u] * ldq, c0, cols,
                                        s + (int64_t)gg[u] * lds + rr[u], sl == 0, vout);
        }
    }
}

// ---------------------------------------------------------------------------
// 128x128 tiles: block scales (weights) or column scales (128x1 groups)
// ---------------------------------------------------------------------------

// Reads the NRx8 sub-tile rows r0..r0+NR-1, cols c0..c0+7 of a row-major
// matrix; elements outside [rows, cols] read as 0.  An interior sub-tile of
// an aligned matrix issues all of its row loads before unpacking any.
template <int DT, int NR>
__device__ __forceinline__ void load_rows8(const void* x, int64_t ldx, int64_t rows, int64_t cols,
                                           int64_t r0, int64_t c0, float v[NR][8], bool vin) {
    const size_t esz = DT == kBF16 ? 2 : 4;
    if (vin && r0 + NR <= rows && c0 + 8 <= cols) {
        Run8 raw[NR];
#pragma unroll
        for (int p = 0; p < NR; ++p)
            issue8<DT>(static_cast<const char*>(x) + (size_t)(r0 + p) * (size_t)ldx * esz, c0, raw[p]);
#pragma unroll
        for (int p = 0; p < NR; ++p) unpack8<DT>(raw[p], v[p]);
        return;
    }
#pragma unroll
    for (int p = 0; p < NR; ++p) {
        if (r0 + p < rows) {
            load8_elems<DT>(static_cast<const char*>(x) + (size_t)(r0 + p) * (size_t)ldx * esz, c0,
                            cols, v[p]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[p][j] = 0.0f;
        }
    }
}

// Tile of workgroup b in a one-tile-per-workgroup grid of n: workgroups are
// dealt to the 8 XCDs round-robin (b % 8), so XCD x takes the contiguous
// tiles [start(x), start(x) + count(x)) instead of every eighth one, and
// tiles that are neighbours in a row run on one XCD at about the same time.
// A bijection on [0, n): XCD x has count(x) = n/8 + (x < n%8) workgroups.
// (128x128 blocks of W_e [524288,7168]: 2110 -> 1946 us; tokens [32768,7168]
// 110.8 -> 107.6 us; the 128x1 kernel is 2 % faster without it.)
__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t n) {
    const uint32_t x = b & 7, i = b >> 3, q = n >> 3, r = n & 7;
    return x * q + min(x, r) + i;
}

// Byte j of the 8-byte row code (lo: bytes 0..3, hi: bytes 4..7).
__device__ __forceinline__ uint32_t code_byte(uint32_t lo, uint32_t hi, int j) {
    return ((j < 4 ? lo >> (8 * j) : hi >> (8 * (j - 4)))) & 0xFFu;
}

// Stores the 16 code bytes [c0, c0+16) of an output row (those below
// `cols`); vec: 2 -- row start and pitch 16-byte aligned, 1 -- 8-byte, 0 --
// neither.
__device__ __forceinline__ void store16(uint8_t* row, int64_t c0, int64_t cols, uint4 v, int vec) {
    if (vec == 2 && c0 + 16 <= cols) {
        *reinterpret_cast<uint4*>(row + c0) = v;
        return;
    }
    store8(row, c0, cols, v.x, v.y, vec == 1);
    store8(row, c0 + 8, cols, v.z, v.w, vec == 1);
}

// The tile's transposed codes in LDS: output row c (input column c of the
// tile) is 16 chunks of 8 bytes, chunk k holding input rows 8k..8k+7, stored
// at position k ^ (c / 8 % 16).  The swizzle spreads the 16 lanes of a DPP
// row, which write the same chunk of 16 different output rows, over all 32
// banks; a chunk pair 2m, 2m+1 stays one aligned 16-byte word (swapped when
// the swizzle is odd).
constexpr int kTBufChunks = 128 * 16;

// Tile height of the 1x128 mode: a group needs a tile's full 128 columns but
// not its 128 rows, and shorter tiles leave a smaller last round of
// workgroups (one-wave workgroups: A [8192,7168] 34.2 -> 33.5 us, tokens
// [32768,7168] 112.1 -> 110.6 us against 128-row tiles; 64 rows in between).
constexpr int kRowTileH = 32;

// TH: tile height (rows), 128 except in kTileRows mode; the workgroup has
// 2*TH threads.
template <int DT, int MODE, int RULE, int TH = 128>
__global__ __launch_bounds__(2 * TH) void quant_tile_kernel(const void* __restrict__ x, int64_t rows,
                                                         int64_t cols, int64_t ldx,
                                                         uint8_t* __restrict__ q, int64_t ldq,
                                                         uint8_t* __restrict__ qt, int64_t ldqt,
                                                         float* __restrict__ s, int64_t lds,
                                                         int64_t tiles_c, bool vin, int vq,
                                                         int vqt) {
    static_assert(MODE == kTileBlock || MODE == kTileRows, "128x1 groups: quant_cols_kernel");
    static_assert(TH == 128 || MODE == kTileRows, "only 1x128 groups allow short tiles");
    __shared__ uint32_t red[MODE == kTileRows ? 1 : 4];
    __shared__ __attribute__((aligned(16))) uint2 tbuf[MODE == kTileRows ? 1 : kTBufChunks];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int a = tid >> 4;   // sub-tile row group 0..TH/8-1
    const int b = tid & 15;   // sub-tile col group 0..15
    const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t ti = tile / tiles_c;
    const int64_t tj = tile - ti * tiles_c;
    const int64_t r0 = ti * TH + 8 * a;
    const int64_t c0 = tj * 128 + 8 * b;

    float v[8][8];
    load_rows8<DT, 8>(x, ldx, rows, cols, r0, c0, v, vin);

    // inverse scales: kTileBlock -- inv[j] of column j, all equal; kTileRows --
    // inv[p] of row p
    float inv[8];
    if constexpr (MODE == kTileBlock) {
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
        // row p of the sub-tile: its group is the row's 128 columns, held by
        // the 16 lanes b = 0..15 of this DPP row
        float sc[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(fabsf(v[p][j])));
            m = row16_max_u32(m);
            group_scale_rule<RULE>(__uint_as_float(m), sc[p], inv[p]);
        }
        // lane b < 8 stores the scale of row r0 + b: scale index [group][row]
        float mine = sc[0];
#pragma unroll
        for (int p = 1; p < 8; ++p)
            if (b == p) mine = sc[p];
        if (b < 8 && r0 + b < rows) s[tj * lds + r0 + b] = mine;
    }

    // codes: row p of the sub-tile as two dwords
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        if (MODE == kTileRows) {
            lo[p] = enc4(v[p][0] * inv[p], v[p][1] * inv[p], v[p][2] * inv[p], v[p][3] * inv[p]);
            hi[p] = enc4(v[p][4] * inv[p], v[p][5] * inv[p], v[p][6] * inv[p], v[p][7] * inv[p]);
        } else {
            lo[p] = enc4(v[p][0] * inv[0], v[p][1] * inv[1], v[p][2] * inv[2], v[p][3] * inv[3]);
            hi[p] = enc4(v[p][4] * inv[4], v[p][5] * inv[5], v[p][6] * inv[6], v[p][7] * inv[7]);
        }
    }

    if (q != nullptr) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            if (r0 + p < rows) store8(q + (r0 + p) * ldq, c0, cols, lo[p], hi[p], vq != 0, vq == 2);
        }
    }
    if (MODE == kTileBlock && qt != nullptr) {
        // transposed: output row c0+j holds bytes of input rows r0..r0+7,
        // chunk a of LDS row 8b+j
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t tlo = 0, thi = 0;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                tlo |= code_byte(lo[p], hi[p], j) << (8 * p);
                thi |= code_byte(lo[p + 4], hi[p + 4], j) << (8 * p);
            }
            tbuf[(8 * b + j) * 16 + (a ^ b)] = make_uint2(tlo, thi);
        }
        __syncthreads();
        // 128 output rows x 8 runs of 16 bytes: thread tid takes runs
        // tid, tid + 256, ...; 8 consecutive lanes cover one output row
        const int64_t oc0 = tj * 128, or0 = ti * 128;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = it * 256 + tid;
            const int c = idx >> 3;    // output row within the tile
            const int k = idx & 7;     // 16-byte run: input rows 16k .. 16k+15
            const int sw = (c >> 3) & 15;
            const uint4 w = *reinterpret_cast<const uint4*>(&tbuf[c * 16 + ((2 * k) ^ (sw & ~1))]);
            const uint4 run = (sw & 1) ? make_uint4(w.z, w.w, w.x, w.y) : w;
            if (oc0 + c < cols) store16(qt + (oc0 + c) * ldqt, or0 + 16 * k, rows, run, vqt);
        }
    }
}

// 128x1 groups (one scale per column over 128 rows: the weight-gradient
// operands), codes stored transposed.  A workgroup takes a 128-row x
// 256-column tile, each of its four waves a 128 x 64 strip; lane (a, b) =
// (lane / 8, lane % 8) of a wave owns rows 16a..16a+15 and columns
// 8b..8b+7 of the strip.  So:
//  - a wave's load instruction reads 8 rows, each a whole 128-byte segment
//    (BF16), and the four waves read the rows' adjacent segments together;
//  - a column's 128 rows lie in one wave, and its max takes three lane
//    exchanges over the 8 row groups (no LDS, no barrier);
//  - the 16 codes a lane holds of one column are 16 consecutive bytes of
//    that column's output row: one 16-byte store, and the 8 lanes of a
//    column group write one whole 128-byte output segment.
// A/B against 128x128 tiles with an LDS exchange, bitwise identical: X^T
// [7168 x 8192 tokens] 37.8 -> 34.3 us, dY^T [2048 x 8192] 13.6 -> 11.7 us;
// one-wave workgroups (128 x 64 tiles) lose on X^T (40.6 us), and eight-wave
// ones too (40.8 us).  Three waves per SIMD (168 VGPRs) against two: X^T 35.8
// -> 34.3 us; four spill.
constexpr int kColStripW = 64;
constexpr int kColWaves = 4;

template <int DT, int RULE>
__global__ __launch_bounds__(64 * kColWaves, 3) void quant_cols_kernel(
        const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* __restrict__ qt,
        int64_t ldqt, float* __restrict__ s, int64_t lds, int64_t tiles_c, bool vin, int vqt, bool vs) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int a = lane >> 3;   // row group 0..7
    const int b = lane & 7;    // column group 0..7
    const int64_t ti = blockIdx.x / tiles_c;
    const int64_t tj = blockIdx.x - ti * tiles_c;
    const int64_t r0 = ti * 128 + 16 * a;
    const int64_t c0 = (tj * kColWaves + wave) * kColStripW + 8 * b;

    float v[16][8];
    load_rows8<DT, 16>(x, ldx, rows, cols, r0, c0, v, vin);

    float sc[8], inv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int p = 0; p < 16; ++p) m = max(m, __float_as_uint(fabsf(v[p][j])));
        m = max(m, (uint32_t)__shfl_xor((int)m, 8));
        m = max(m, (uint32_t)__shfl_xor((int)m, 16));
        m = max(m, (uint32_t)__shfl_xor((int)m, 32));
        group_scale_rule<RULE>(__uint_as_float(m), sc[j], inv[j]);
    }
    // logical output row = input column; scale index [tile row][column]
    if (a == 0) {
        float* sp = s + ti * lds + c0;
        if (vs && c0 + 8 <= cols) {
            reinterpret_cast<float4*>(sp)[0] = make_float4(sc[0], sc[1], sc[2], sc[3]);
            reinterpret_cast<float4*>(sp)[1] = make_float4(sc[4], sc[5], sc[6], sc[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (c0 + j < cols) sp[j] = sc[j];
        }
    }
    // output row c0+j, bytes r0..r0+15: the column's codes in row order
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = enc4(v[4 * q][j] * inv[j], v[4 * q + 1][j] * inv[j], v[4 * q + 2][j] * inv[j],
                        v[4 * q + 3][j] * inv[j]);
        if (c0 + j < cols) store16(qt + (c0 + j) * ldqt, r0, rows, make_uint4(w[0], w[1], w[2], w[3]), vqt);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static bool is_aligned(const void* p, uintptr_t a) {
    return reinterpret_cast<uintptr_t>(p) % a == 0;
}

// Resident workgroups of quant_rows_kernel<DT, RL> on the current device
// (cached per device).
// Threads may race to fill an entry; they all store the same value.
template <int DT, int RL>
static int64_t rows_resident_blocks() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 2048;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_rows_kernel<DT, RL>, 256, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 4;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        v = per_cu * cus;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

static DivMagic make_div_magic(uint32_t d) {
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    const uint64_t m = ((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d) + 1;
    return DivMagic{(uint32_t)m, l};
}

template <int DT, int RL>
static hipError_t launch_rows_t(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds, bool vin,
                                bool vout, hipStream_t stream) {
    const int64_t esz = DT == kBF16 ? 2 : 4;
    const int64_t gpr = (cols + 127) / 128;
    if (rows <= 0 || gpr <= 0) return hipSuccess;
    const DivMagic dm = make_div_magic((uint32_t)gpr);
    // four resident rounds of workgroups (measured best among 1, 2, 4, 8)
    const int64_t cap = 4 * rows_resident_blocks<DT, RL>();
    // rows per launch: fewer than 2^31 groups, so 32-bit group indices
    const int64_t chunk = (((int64_t)1 << 31) / gpr - 4) / 4 * 4;
    for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
        const int64_t nr = rows - r0 < chunk ? rows - r0 : chunk;
        const int64_t total = (nr + 3) / 4 * 4 * gpr;   // bands of 4 rows
        int64_t blocks = (total + 16 * kRowUnroll - 1) / (16 * kRowUnroll);
        if (blocks > cap) blocks = cap;
        hipLaunchKernelGGL((quant_rows_kernel<DT, RL>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const char*>(x) + r0 * ldx * esz, cols, ldx, q + r0 * ldq,
                           ldq, s + r0, lds, (uint32_t)total, (uint32_t)gpr, dm, vin, vout, (uint32_t)nr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds, int rule,
                             hipStream_t stream) {
    // 128 rows or more: kRowTileH x 128 tiles (kTileRows), whose loads and
    // stores are those of the weight quantizer; fewer rows: the row-striding
    // kernel
    if (rows >= 128 && (rows + kRowTileH - 1) / kRowTileH * ((cols + 127) / 128) <= 0x7FFFFFFF)
        return launch_quant_tiles(x, dtype, kTileRows, rows, cols, ldx, q, ldq, nullptr, 0, s, lds,
                                  rule, stream);
    const int64_t esz = dtype == kBF16 ? 2 : 4;
    const bool vin = is_aligned(x, 16) && (ldx * esz) % 16 == 0;
    const bool vout = is_aligned(q, 8) && ldq % 8 == 0;
    if (dtype == kBF16) {
        if (rule == kRulePow2)
            return launch_rows_t<kBF16, kRulePow2>(x, rows, cols, ldx, q, ldq, s, lds, vin, vout, stream);
        return launch_rows_t<kBF16, kRuleFP32>(x, rows, cols, ldx, q, ldq, s, lds, vin, vout, stream);
    }
    if (rule == kRulePow2)
        return launch_rows_t<kF32, kRulePow2>(x, rows, cols, ldx, q, ldq, s, lds, vin, vout, stream);
    return launch_rows_t<kF32, kRuleFP32>(x, rows, cols, ldx, q, ldq, s, lds, vin, vout, stream);
}

// Code output size above which the tile kernel stores codes non-temporally.
constexpr int64_t kNtCodeBytes = int64_t(256) << 20;

hipError_t launch_quant_tiles(const void* x, int dtype, int mode, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                              float* s, int64_t lds, int rule, hipStream_t stream) {
    const int64_t esz = dtype == kBF16 ? 2 : 4;
    const bool vin = is_aligned(x, 16) && (ldx * esz) % 16 == 0;
    // row-major codes: 0 byte stores, 1 8-byte stores, 2 8-byte non-temporal
    // stores (outputs larger than the 256 MB memory-side cache cannot stay
    // there for the next kernel, and ordinary stores would only evict what
    // can: MoE W_e codes, 3.76 GB, 1940 -> 1880 us; the 235 MB of MoE token
    // codes stay ordinary, 107 against 120 us non-temporal)
    const int vq = q == nullptr || !is_aligned(q, 8) || ldq % 8 != 0 ? 0
                   : rows * cols > kNtCodeBytes                     ? 2
                                                                    : 1;
    const int vqt = qt == nullptr ? 0
                    : (is_aligned(qt, 16) && ldqt % 16 == 0) ? 2
                    : (is_aligned(qt, 8) && ldqt % 8 == 0) ? 1
                                                           : 0;
    if (mode == kTileCols) {
        const int64_t tw = kColStripW * kColWaves;
        const int64_t tc = (cols + tw - 1) / tw;
        const dim3 grid((unsigned)((rows + 127) / 128 * tc)), block(64 * kColWaves);
        const bool vs = is_aligned(s, 16) && lds % 4 == 0;
#define FP8Q_LAUNCH_COLS(DT, RL)                                                                   \
    hipLaunchKernelGGL((quant_cols_kernel<DT, RL>), grid, block, 0, stream, x, rows, cols, ldx, qt, \
                       ldqt, s, lds, tc, vin, vqt, vs)
        if (dtype == kBF16) {
            if (rule == kRulePow2) FP8Q_LAUNCH_COLS(kBF16, kRulePow2);
            else FP8Q_LAUNCH_COLS(kBF16, kRuleFP32);
        } else {
            if (rule == kRulePow2) FP8Q_LAUNCH_COLS(kF32, kRulePow2);
            else FP8Q_LAUNCH_COLS(kF32, kRuleFP32);
        }
#undef FP8Q_LAUNCH_COLS
        return hipGetLastError();
    }
    const int64_t th = mode == kTileRows ? kRowTileH : 128;
    const int64_t tr = (rows + th - 1) / th, tc = (cols + 127) / 128;
    dim3 grid((unsigned)(tr * tc)), block((unsigned)(2 * th));
#define FP8Q_LAUNCH_TILE(DT, MD, RL)                                                          \
    hipLaunchKernelGGL((quant_tile_kernel<DT, MD, RL, MD == kTileRows ? kRowTileH : 128>), grid, \
                       block, 0, stream, x, rows, cols, ldx, q, ldq, qt, ldqt, s, lds, tc, vin, vq, vqt)
#define FP8Q_LAUNCH_TILE_RULE(DT, MD)                          \
    do {                                                       \
        if (rule == kRulePow2) FP8Q_LAUNCH_TILE(DT, MD, kRulePow2); \
        else FP8Q_LAUNCH_TILE(DT, MD, kRuleFP32);              \
    } while (0)
#define FP8Q_LAUNCH_TILE_MODE(DT)                                      \
    do {                                                               \
        if (mode == kTileBlock) FP8Q_LAUNCH_TILE_RULE(DT, kTileBlock); \
        else FP8Q_LAUNCH_TILE_RULE(DT, kTileRows);                     \
    } while (0)
    if (dtype == kBF16) FP8Q_LAUNCH_TILE_MODE(kBF16);
    else FP8Q_LAUNCH_TILE_MODE(kF32);
#undef FP8Q_LAUNCH_TILE_MODE
#undef FP8Q_LAUNCH_TILE_RULE
#undef FP8Q_LAUNCH_TILE
    return hipGetLastError();
}

}  // namespace fp8q
