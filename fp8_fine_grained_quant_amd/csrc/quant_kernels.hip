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
//                        MODE_BLOCK: one scale per tile (weights), codes
//                        stored row-major and/or transposed;
//                        MODE_COLS: one scale per column over the tile's 128
//                        rows (128x1 groups for the weight-gradient GEMM),
//                        codes stored transposed.
//                        The transposed store is an 8x8 byte transpose in
//                        registers, so each thread writes 8-byte runs and
//                        the 16 threads of a column run write 128 bytes.
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

// Reads the 8x8 sub-tile rows r0..r0+7, cols c0..c0+7 of a row-major matrix;
// elements outside [rows, cols] read as 0.  An interior sub-tile of an
// aligned matrix issues its eight row loads before unpacking any.
template <int DT>
__device__ __forceinline__ void load_8x8(const void* x, int64_t ldx, int64_t rows, int64_t cols,
                                         int64_t r0, int64_t c0, float v[8][8], bool vin) {
    const size_t esz = DT == kBF16 ? 2 : 4;
    if (vin && r0 + 8 <= rows && c0 + 8 <= cols) {
        Run8 raw[8];
#pragma unroll
        for (int p = 0; p < 8; ++p)
            issue8<DT>(static_cast<const char*>(x) + (size_t)(r0 + p) * (size_t)ldx * esz, c0, raw[p]);
#pragma unroll
        for (int p = 0; p < 8; ++p) unpack8<DT>(raw[p], v[p]);
        return;
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        if (r0 + p < rows) {
            load8_elems<DT>(static_cast<const char*>(x) + (size_t)(r0 + p) * (size_t)ldx * esz, c0,
                            cols, v[p]);
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
