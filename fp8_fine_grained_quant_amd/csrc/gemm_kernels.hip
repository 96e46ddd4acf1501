// gemm_kernels.hip -- FP8 (E4M3) block-scaled GEMM for gfx950.
//
// C[M,N] = A[M,K] * B[N,K]^T where every 128-wide K interval's partial sum is
// multiplied by the activation tile scale sa[m,kb] and the weight scale
// sb[n,kb] and accumulated in FP32 -- the "promotion" of partial results to
// FP32 with the scales applied at that point (jp-study.kr page, Figure 7(b);
// scales per 1x128 activation tile and 128x128 weight block from "Should
// Fixing Deepseek Take 60 Steps?", Figure 7(a)).
//
// The pages' kernel was built around another vendor's asynchronous matrix
// instructions, with a second warp group promoting while the first multiplies.
// On CDNA4 the same goal -- matrix cores never idle while the vector units
// promote -- is met inside each wave: an MFMA retires into a short-lived
// partial-sum register set and independent VALU FMAs fold the previous
// partial into the FP32 accumulator while the next MFMA runs.
//
// All of them -- BLOCK128 (Fprop, Dgrad, the grouped MoE GEMM) and ROW128
// (Wgrad) -- run the ping-pong kernel gemm_pp_kernel.
//
// Design (256x256 output tiles; a persistent workgroup of 8 waves, 2 per
// SIMD, on each compute unit loops over its tiles):
//  * K step 128 = exactly one scale block, so each K step is one
//    16x16x128 FP8 matrix instruction per 16x16 output block: the plain
//    v_mfma_f32_16x16x128_f8f6f4 with FP32 block scales, which the
//    promotion FMA applies, or v_mfma_scale_f32_16x16x128_f8f6f4 carrying
//    power-of-two scales.
//  * A and B K-slabs (256x128 bytes each) go HBM -> LDS with
//    global_load_lds_dwordx4 (no VGPR staging), double buffered: the next
//    slab streams in while the current one is multiplied.  Rows are 128
//    bytes with an XOR chunk swizzle that keeps both the copies (8 lanes per
//    row) coalesced and the fragment reads free of bank conflicts (see swz).
//  * Wave tile 64(M) x 128(N): 4 x 8 blocks of 16x16, 128 FP32 accumulator
//    VGPRs (64 x 112 in the 224-wide tiles of the ROW128 GEMM).  The MFMA is
//    issued with the B slab as its first operand, so a lane's four result
//    registers are four CONSECUTIVE output columns of one row and the
//    128x128-block weight scale is a wave-uniform scalar.  The epilogue
//    turns the block around through LDS and stores whole row segments.
//  * A tile's last two K steps already copy the next tile's first two, so a
//    workgroup moves from tile to tile without a prologue.
//  * Workgroup -> tile mapping keeps each XCD on a contiguous range of tiles
//    and walks them in groups of 8 tile rows so that concurrently running
//    tiles share A rows and B columns in that XCD's L2.
//  * Tails in M and N: loads clamp the row index (never read out of bounds),
//    stores are masked.
#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 512;
constexpr int kWaveM = 64;
constexpr int kSlabBytes = BM * BK;          // one operand, one stage
constexpr int kStageBytes = 2 * kSlabBytes;  // A + B
constexpr int kGroupM = 8;                   // tile rows per swizzle group

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// Wave-uniform 64-bit pointer, made provably uniform (lives in SGPRs).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// HBM -> LDS copies (global_load_lds): lane l's 16 (or 4) bytes at
// base + voff land at LDS address m0 + 16*l (or 4*l).  Written as inline
// assembly so that the compiler does not treat the copy in flight as a
// pending write to every LDS location (it would then wait for it before
// each LDS read); completion is awaited explicitly with vmcnt before the
// barrier that publishes a stage.  The compiler loads M0 itself ("{m0}").
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// LDS layout of a 256-row x 128-byte operand slab: row r at r*128, its
// 16-byte K chunk c at slot c ^ f(r) with f(r) = (r & 7) ^ ((r >> 3) & 1).
// A fragment read (ds_read_b128) has the 16 rows of a block in one 16-lane
// quarter of the wave, all at the same logical chunk.  f is a permutation
// of 0..7 on rows 0..7 and on rows 8..15, and on each row-parity class of
// the 16 rows (whose 128-byte rows fall alternately into the two halves of
// a 256-byte bank window), so every 8-lane group and every 16-lane quarter
// touches distinct banks: the read runs at the full LDS rate (measured with
// the SQ_LDS_BANK_CONFLICT counter, zero conflict cycles, where f(r) =
// (r >> 1) & 7 or f(r) = r & 7 alone cost two-way conflicts).  The copy side
// stays fully coalesced: 8 consecutive lanes fetch one row's 128 bytes.
// Lane l = 16*kq + r of a wave holds, for block b, row 16b + r, K chunks
// 2kq and 2kq+1 (32 bytes).  The matrix instruction sums over its 128 K
// positions in the same order for both operands, so any K assignment shared
// by A and B gives the same dot products.
__device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
}

__device__ __forceinline__ v8i frag32(const uint8_t* __restrict__ slab, int block, int lane) {
    const int row = block * 16 + (lane & 15);
    const int kq = lane >> 4;
    const uint8_t* rb = slab + row * BK;
    const uint4 x0 = *reinterpret_cast<const uint4*>(rb + (swz(row, 2 * kq) << 4));
    const uint4 x1 = *reinterpret_cast<const uint4*>(rb + (swz(row, 2 * kq + 1) << 4));
    return (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                 (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// The partial sum of one 128-wide K block, unscaled.  Zero scale operands
// make the compiler emit the plain v_mfma_f32_16x16x128_f8f6f4, which has
// no scale operands; it is bitwise equal to the scaled form with unit (E8M0
// 127) scales (tests/probes/mfma_forms.hip: 262,144 random outputs), and it
// issues faster (Fprop 781.6 -> 774.8 us, Dgrad 821.6 -> 813.7 us, Wgrad
// 118.8 -> 115.1 us, bitwise identical).
__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        a, b, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
}

// Power-of-two scales applied by the instruction itself: lane l's scale
// operands are the E8M0 exponents of its operand-A row (l & 15) and
// operand-B row (l & 15), used for every 32-wide K group of the lane's
// fragment; the product accumulates onto c.
__device__ __forceinline__ v4f mfma_f8_scaled(const v8i& a, const v8i& b, const v4f& c,
                                              uint32_t scale_a, uint32_t scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, (int)scale_a, 0,
                                                            (int)scale_b);
}

// E8M0 exponent of an FP32 power of two 2^e, e in [-127, 127]: its biased
// exponent field (2^-127, an FP32 subnormal, gives 0).  Mantissa bits are
// ignored.
__device__ __forceinline__ uint32_t e8m0_of(float s) { return (__float_as_uint(s) >> 23) & 0xFFu; }

// Everything a wave needs to stream one K step of A, B and the scales into
// an LDS stage.
struct LoadCtx {
    const uint8_t* a_base;  // A + m0*lda (wave-uniform)
    const uint8_t* b_base;  // B + n0*ldb (wave-uniform)
    uint32_t a_off[4];      // per copy instruction: row*lda + K byte offset
    uint32_t b_off[4];
    const float* s_base;    // scale row of K step 0 (sa, or sb in ROW128 mode)
    uint32_t s_off;         // this lane's element offset, in bytes
    int64_t s_kstride;      // scale elements per K step
};

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Barrier that publishes/releases a stage: this wave's own LDS reads and
// copies are complete, then all waves meet.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Copy instruction q (0..8) of one K step into an LDS stage: q < 4 moves
// 8 rows of the A slab, 4 <= q < 8 8 rows of the B slab, q == 8 the scales.
__device__ __forceinline__ void issue_copy(int q, const LoadCtx& lc, int64_t koff, int kb,
                                           uint8_t* st_a, uint8_t* st_b, float* st_s,
                                           int wave) {
    if (q < 4)
        dma16(lc.a_base + koff, lc.a_off[q], lds_addr(st_a + (wave * 4 + q) * 1024));
    else if (q < 8)
        dma16(lc.b_base + koff, lc.b_off[q - 4], lds_addr(st_b + (wave * 4 + q - 4) * 1024));
    else
        dma4(uniform_ptr(lc.s_base + (int64_t)kb * lc.s_kstride), lc.s_off, lds_addr(st_s + (wave & 3) * 64));
}

// Promotion of one 16x16 block: acc += partial * scale (ROW128: the scale of
// each of the lane's four columns differs).
template <int SCALE_MODE>
__device__ __forceinline__ void promote(v4f& a, const v4f& pp, float sci, const float4& sbq) {
    if (SCALE_MODE == kScaleBlock128) {
        a[0] = fmaf(pp[0], sci, a[0]);
        a[1] = fmaf(pp[1], sci, a[1]);
        a[2] = fmaf(pp[2], sci, a[2]);
        a[3] = fmaf(pp[3], sci, a[3]);
    } else {
        a[0] = fmaf(pp[0], sci * sbq.x, a[0]);
        a[1] = fmaf(pp[1], sci * sbq.y, a[1]);
        a[2] = fmaf(pp[2], sci * sbq.z, a[2]);
        a[3] = fmaf(pp[3], sci * sbq.w, a[3]);
    }
}

// Read-only memory seen through the constant address space: uniform
// accesses become scalar loads (lgkmcnt), which leave the counted vmcnt
// waits on the copies in flight undisturbed.
typedef __attribute__((address_space(4))) const GemmParams* ConstParamsPtr;
typedef __attribute__((address_space(4))) const int32_t* ConstI32Ptr;

// The kernel's GemmParams, read from the kernel argument segment at the point
// of use.  The persistent kernel needs most arguments again for every tile;
// the empty asm hides where the pointer comes from, so the compiler reloads
// them (scalar loads, cached) instead of pinning ~30 SGPRs for the whole
// kernel.
static_assert(sizeof(GemmParams) == 16 * 8, "kparams() copies each of GemmParams' 16 fields");
__device__ __forceinline__ GemmParams kparams() {
    ConstParamsPtr q = (ConstParamsPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(q));
    GemmParams r;
    r.a = q->a; r.lda = q->lda; r.sa = q->sa; r.ldsa = q->ldsa;
    r.b = q->b; r.ldb = q->ldb; r.sb = q->sb; r.sbs0 = q->sbs0; r.sbs1 = q->sbs1;
    r.c = q->c; r.ldc = q->ldc; r.M = q->M; r.N = q->N; r.K = q->K;
    r.offsets = q->offsets; r.num_groups = q->num_groups;
    return r;
}

// An output tile: rows [m0, m_end) of C (m_end: the end of the tile's group,
// or M), columns from n0, and the weight codes and block scales it uses.
struct Tile {
    int64_t m0, m_end, n0;
    const uint8_t* b;
    const float* sb;
};

// Dense tile t: each XCD gets a contiguous range of tiles (workgroups are
// dealt to the XCDs round-robin), walked in groups of kGroupM tile rows so
// that tiles running together share A rows and B columns in L2.
// The tile count is below 2^31 (checked by the host), so the index
// arithmetic runs in 32 bits.
template <int TBN>
__device__ __forceinline__ Tile dense_tile(const GemmParams& p, uint32_t t) {
    const uint32_t tiles_n = (uint32_t)((p.N + TBN - 1) / TBN);
    const uint32_t tiles_m = (uint32_t)((p.M + BM - 1) / BM);
    const uint32_t T = tiles_m * tiles_n;
    if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
    const uint32_t grp = t / (kGroupM * tiles_n);
    const uint32_t first_m = grp * kGroupM;
    const uint32_t gm = min(tiles_m - first_m, (uint32_t)kGroupM);
    const uint32_t rem = t - grp * kGroupM * tiles_n;
    return Tile{(int64_t)(first_m + rem % gm) * BM, p.M, (int64_t)(rem / gm) * TBN, p.b, p.sb};
}

// Grouped GEMM tile table in LDS: group g owns tiles [tile_start[g],
// tile_start[g+1]), ceil(rows_g/BM) * tiles_n of them.  Built once per
// workgroup from the device offsets (a block-wide scan); returns the total
// tile count.
template <int TBN>
__device__ __forceinline__ int32_t grouped_table(const GemmParams& p, int32_t* tile_start,
                                                 int32_t* wave_tot, int tid, int lane, int wave) {
    const int64_t G = p.num_groups;
    const int32_t tiles_n = (int32_t)((p.N + TBN - 1) / TBN);
    const int per = (int)((G + kThreads - 1) / kThreads);
    const int g0 = tid * per;
    int32_t local = 0;
    for (int g = g0; g < g0 + per && g < G; ++g) {
        const int32_t rows = p.offsets[g + 1] - p.offsets[g];
        local += (rows + BM - 1) / BM * tiles_n;
    }
    int32_t incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int32_t v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wave_tot[w];
    int32_t run = base + incl - local;
    for (int g = g0; g < g0 + per && g < G; ++g) {
        tile_start[g] = run;
        const int32_t rows = p.offsets[g + 1] - p.offsets[g];
        run += (rows + BM - 1) / BM * tiles_n;
    }
    if (tid == kThreads - 1) tile_start[G] = run;
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(tile_start[G]);
}

// Grouped tile t < tile_start[G].  As for dense tiles, each XCD gets a
// contiguous range of the table (when the tile count and the grid are
// multiples of 8, which keeps a workgroup's tiles increasing), and a group's
// tiles are walked in groups of kGroupM tile rows: without this every XCD
// took one tile column of every group and all eight read each A tile (3.5-6 %
// slower on 262,144-row problems).  The tile's group is the last g with
// tile_start[g] <= t.  A workgroup's tiles only increase, so the search runs
// upward from gc (the previous tile's group), 64 table entries per step: the
// entries <= t form a prefix of the window, counted with a ballot.
template <int TBN>
__device__ __forceinline__ Tile grouped_tile(const GemmParams& p, const int32_t* tile_start,
                                             int32_t t, int& gc, int lane) {
    const int G = (int)p.num_groups;
    const int32_t T = __builtin_amdgcn_readfirstlane(tile_start[G]);
    if ((T & 7) == 0 && (gridDim.x & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
    for (int it = 0; it <= G / 64 + 1; ++it) {
        const int gi = gc + 1 + lane;
        const bool le = gi <= G && tile_start[gi] <= t;
        const int k = __popcll(__ballot(le));
        gc = __builtin_amdgcn_readfirstlane(gc + k);
        if (k < 64) break;
    }
    const int g = gc;
    const int64_t N = p.N;
    const int32_t tiles_n = (int32_t)((N + TBN - 1) / TBN);
    const int32_t first_t = __builtin_amdgcn_readfirstlane(tile_start[g]);
    const int32_t local_t = t - first_t;
    const int32_t tiles_m = (__builtin_amdgcn_readfirstlane(tile_start[g + 1]) - first_t) / tiles_n;
    const int32_t grp = local_t / (kGroupM * tiles_n);
    const int32_t first_m = grp * kGroupM;
    const int32_t gm = min(tiles_m - first_m, (int32_t)kGroupM);
    const int32_t rem = local_t - grp * kGroupM * tiles_n;
    const int32_t tm = first_m + rem % gm;
    const int32_t tn = rem / gm;
    const ConstI32Ptr offs = (ConstI32Ptr)p.offsets;   // scalar loads (g is uniform)
    return Tile{(int64_t)offs[g] + (int64_t)tm * BM, (int64_t)offs[g + 1], (int64_t)tn * TBN,
                p.b + (int64_t)g * N * p.ldb, p.sb + (int64_t)g * ((N + 127) / 128) * (p.K / 128)};
}

// Epilogue: the wave's 64 x kWN output block goes to C through a 4 KiB LDS
// buffer of its own, in passes of 16 rows x 256 bytes.  A matrix instruction
// leaves each lane 4 consecutive columns of one row, so a direct store writes
// 16 rows x 32 bytes (BF16) per instruction: 16 partial-line requests.  After
// the round trip through LDS a lane holds 16 consecutive bytes and a store
// instruction covers 4 whole 256-byte row segments.  The 16-byte chunks of a
// buffer row are XOR-swizzled with the row (chunk ^ (row & 15)), which keeps
// both the fragment-order writes and the row-order reads free of bank
// conflicts.  Rows past m_end and columns past N are not written.  Whole
// 16-byte chunks go out as non-temporal stores: C is written once, and kept
// out of the memory-side cache it leaves the A and B codes there for the
// other tiles that re-read them (Fprop 858 -> 843 us, Dgrad 899 -> 891 us,
// bitwise identical).
template <int OUT, int NJ>
__device__ __forceinline__ void store_tile(const GemmParams& p, const v4f (&acc)[4][NJ], uint8_t* buf,
                                           int64_t m_base, int64_t m_end, int64_t n_base, int lane) {
    // (opaque: the per-lane address terms are computed here, per tile, not
    // hoisted out of the tile loop and kept live through the K loop)
    asm volatile("" : "+v"(lane));
    const int64_t N = p.N;
    const int r16 = lane & 15, kq = lane >> 4;
    const int q = lane & 15;           // read side: 16-byte chunk of a buffer row
    const int rq = lane >> 4;          // read side: row within a group of 4
    // passes: BF16 -- one per row block i (NJ blocks of 16 columns = 2*NJ
    // chunks); FP32 -- one per row block and half (up to 4 blocks = 16 chunks)
    constexpr int kHalves = OUT == kF32 ? 2 : 1;
#pragma unroll
    for (int pass = 0; pass < 4 * kHalves; ++pass) {
        const int i = pass / kHalves, h = pass % kHalves;
        const int j0 = h * 4;
        const int nj = OUT == kF32 ? (NJ - j0 < 4 ? NJ - j0 : 4) : NJ;
        // this pass's row segment: columns n_base + ccol0 .. + 8*chunks - 1
        const int ccol0 = OUT == kF32 ? j0 * 16 : 0;
        const int nchunk = OUT == kF32 ? 4 * nj : 2 * nj;
        asm volatile("" ::: "memory");   // the previous pass's reads stay before these writes
#pragma unroll
        for (int jj = 0; jj < 4 * 2; ++jj) {
            if (jj >= nj) continue;
            const v4f v = acc[i][j0 + jj];
            if constexpr (OUT == kF32) {
                const int ch = 4 * jj + kq;
                *reinterpret_cast<float4*>(buf + r16 * 256 + ((ch ^ r16) << 4)) =
                    make_float4(v[0], v[1], v[2], v[3]);
            } else {
                const int ch = 2 * jj + (kq >> 1);
                *reinterpret_cast<uint2*>(buf + r16 * 256 + ((ch ^ r16) << 4) + (kq & 1) * 8) =
                    make_uint2(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]));
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int rl = 4 * t + rq;
            const uint4 v = *reinterpret_cast<const uint4*>(buf + rl * 256 + ((q ^ rl) << 4));
            const int64_t m = m_base + i * 16 + rl;
            if (q >= nchunk || m >= m_end) continue;
            if constexpr (OUT == kF32) {
                const int64_t n = n_base + ccol0 + 4 * q;
                if (n >= N) continue;
                float* cp = static_cast<float*>(p.c) + m * p.ldc + n;
                if (n + 4 <= N) {
                    __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(cp));
                } else {
                    const float f[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                        __uint_as_float(v.w)};
                    for (int e = 0; e < 4 && n + e < N; ++e) cp[e] = f[e];
                }
            } else {
                const int64_t n = n_base + 8 * q;
                if (n >= N) continue;
                uint16_t* cp = static_cast<uint16_t*>(p.c) + m * p.ldc + n;
                if (n + 8 <= N) {
                    if ((p.ldc & 7) == 0) {
                        __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(cp));
                    } else {   // ldc % 8 == 4: rows alternate between 16- and 8-byte alignment
                        reinterpret_cast<uint2*>(cp)[0] = make_uint2(v.x, v.y);
                        reinterpret_cast<uint2*>(cp)[1] = make_uint2(v.z, v.w);
                    }
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                    for (int e = 0; e < 8 && n + e < N; ++e) cp[e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Ping-pong schedule.
//
// The two waves that share a SIMD belong to different groups: waves 0-3
// (group 0) own the tile's output columns 0-127, waves 4-7 (group 1) columns
// 128-255.  The groups alternate between a memory slot -- LDS fragment reads
// and issuing the global -> LDS copies of later K steps -- and a compute slot
// -- 16 matrix instructions on register-resident fragments, with their
// promotions -- and every slot ends at a workgroup barrier.  On each SIMD one
// wave therefore feeds the matrix pipe while the other one is held up by
// memory traffic (with one schedule for all waves, both would stall on their
// copies at the same time).  A wave runs, per K step kb,
//   MEM(kb,0)  A fragments, B fragments of column blocks 0-3, the scales;
//              issues the copies of its own 32 B rows of step kb+1 (into
//              stage kb+1, whose B rows its group finished reading two
//              slots earlier)
//   COMP(kb,0) column blocks 0-3
//   MEM(kb,1)  B fragments of column blocks 4-7 (ROW128: and the column
//              scales of that half); issues the copies of its 32 A rows and
//              its scale copy of step kb+2 (A rows into stage kb, which both
//              groups have read by then; scales into the scale stage of
//              step kb -- BLOCK128 -- whose scales are read only in
//              MEM(kb,0), or -- ROW128, three scale stages -- of step kb-1,
//              because group 1 reads step kb's column scales in this same
//              slot while waves 6 and 7 issue the copy)
//   COMP(kb,1) column blocks 4-7
// with group 1 one slot behind group 0.  Every copy is issued at least four
// slots before its first reader; each wave waits for its own copies with a
// counted vmcnt before the barrier that publishes them:
//   group 0, after COMP(kb,1): vmcnt(5) -- all but the 5 copies of step kb+3
//     (4 A rows + 1 scale) issued in MEM(kb,1) have landed: step kb+1's A
//     rows, scales and B rows are complete for MEM(kb+1,0);
//   both groups, after MEM(kb,1): vmcnt(9) -- their A rows and scale of
//     step kb+1 have landed (the 4 B copies of step kb+1 and 5 copies of step
//     kb+2 may still fly): group 1's before group 0 reads step kb+1 in the
//     next slot.  Group 0 needs this only at its next wait, but one wait for
//     both groups keeps the compute slot free of a branch (2-3 % faster on
//     Fprop and Dgrad, bitwise identical);
//   group 1, after COMP(kb,1): vmcnt(5) -- its B rows of step kb+1 too.
// Every accumulator sees the same operations in the same order as in a
// plain one-wave-per-tile schedule, so results do not depend on it.
// ---------------------------------------------------------------------------

// Slot boundaries.  The scheduling barriers keep instructions (the matrix
// instructions included, which have no memory effects) inside their slot.
__device__ __forceinline__ void slot_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void slot_barrier_vm5() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void slot_barrier_vm9() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Distance, in matrix instructions, between a partial sum's instruction and
// the FMAs that promote it (the ring of partial sums holds distance + 1).
// An FMA that reads a result still in flight holds up the wave's in-order
// issue, and with it the matrix pipe; at distance 4 the result has landed.
// The dense kernels run the same at 4, 5 and 6 (ROW128: 121.7, 122.6, 123.0
// us on Wgrad).  The grouped kernel ran 2-4 % faster at 6 while it issued
// the scaled matrix instruction; with the plain one, 4 is ~1 % faster than 6
// on the MoE routing (3451 against 3485 us, bitwise identical).
constexpr int kPromoteDist = 4;

// Column scales of the current compute half in ROW128 mode: for column block
// jj, this lane's 4 FP32 column scales, or (POW2) the E8M0 exponent of the
// block's B row r16.  Empty for BLOCK128.
template <bool ROW>
struct RowScales {
    __device__ uint32_t e8m0(int, uint32_t block_e) const { return block_e; }
    __device__ float4 col(int) const { return make_float4(1.f, 1.f, 1.f, 1.f); }
};
template <>
struct RowScales<true> {
    float4 q[4];
    uint32_t e[4];
    // s: the wave's 128 column scales in LDS; h: the compute half
    template <bool POW2>
    __device__ __forceinline__ void load(const float* s, int h, int r16, int kq) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int c = (4 * h + jj) * 16;
            if constexpr (POW2) e[jj] = e8m0_of(s[c + r16]);
            else q[jj] = *reinterpret_cast<const float4*>(&s[c + kq * 4]);
        }
    }
    __device__ uint32_t e8m0(int jj, uint32_t) const { return e[jj]; }
    __device__ float4 col(int jj) const { return q[jj]; }
};

// SM: B scale granularity, kScaleBlock128 (one per 128x128 weight block) or
// kScaleRow128 (one per B row = output column, per K step: the Wgrad GEMM).
template <int OUT, bool POW2, bool GROUPED, int SM, int TBN = BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_pp_kernel(GemmParams p) {
    constexpr bool ROW = SM == kScaleRow128;
    // TBN: tile width, 256 or (ROW128 only) 224.  A wave owns kWN = TBN/2
    // columns in NJ blocks of 16: 4 in the first compute half, NJ1 in the
    // second.
    static_assert(TBN == BN || (ROW && TBN == 224), "224-wide tiles need per-column scales");
    constexpr int kWN = TBN / 2;
    constexpr int NJ = kWN / 16;
    constexpr int NJ1 = NJ - 4;
    // VALU instructions of one promotion: FMAs, plus (ROW128) the products of
    // the row scale with the four column scales
    constexpr int kPromoteValu = ROW ? 8 : 4;
    constexpr int kPartRing = kPromoteDist + 1;
    __shared__ __attribute__((aligned(1024))) uint8_t smem_ab[2][kStageBytes];
    // [stage][0..255]: sa of the tile's rows.  [stage][256 + c]: BLOCK128 --
    // c = g, the weight block scale of column half g (lane l fetches block
    // n0/128 + (l & 1)); ROW128 -- the scale of the tile's column c.
    // Scale stages: two (with the A/B stages) for BLOCK128; three for
    // ROW128, where step kb+2's column scales are copied in the slot in which
    // group 1 still reads step kb's (MEM(kb,1)).
    constexpr int kSStages = ROW ? 3 : 2;
    __shared__ __attribute__((aligned(16))) float smem_s[kSStages][BM + BN];
    __shared__ int32_t tile_start[GROUPED ? (kMaxGroups + 1) : 1];
    __shared__ int32_t wave_tot[kThreads / 64];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave & 3;       // wave row (64 rows each)
    const int g = wave >> 2;       // group == wave column (128 columns each)
    const int r16 = lane & 15;
    const int kq = lane >> 4;

    const int64_t N = p.N;
    const int nkb = (int)(p.K / BK);

    // Persistent: workgroup b runs tiles b, b + gridDim.x, ...  Tile counts
    // are below 2^31 (checked by the host), so t + gridDim.x fits 32 bits.
    uint32_t t = blockIdx.x;
    uint32_t total;
    int gc = 0;   // grouped: group of the current tile
    if constexpr (GROUPED) total = (uint32_t)grouped_table<TBN>(p, tile_start, wave_tot, tid, lane, wave);
    else total = (uint32_t)(((p.M + BM - 1) / BM) * ((N + TBN - 1) / TBN));
    if (t >= total) return;  // whole workgroup: uniform exit
    auto locate = [&](uint32_t tt) -> Tile {
        if constexpr (GROUPED) return grouped_tile<TBN>(kparams(), tile_start, (int32_t)tt, gc, lane);
        else return dense_tile<TBN>(kparams(), (uint32_t)tt);
    };
    Tile cur = locate(t);

    // Copy sources: copy qd of wave w moves rows 8*(4w+qd) .. +7 of a slab
    // (group 0: B rows 0-127, group 1: 128-255); rows past the tile's end
    // are clamped.
    LoadCtx lc;
    auto set_lc = [&](const Tile& tl) {
        const GemmParams p = kparams();
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));   // computed here, not hoisted (as in store_tile)
        const int64_t N = p.N;
        const int64_t nb_last = (N + 127) / 128 - 1;
        const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)tl.m0) |
                           ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)tl.m0 >> 32)) << 32);
        const int64_t n0 = tl.n0, m_end = tl.m_end;
        lc.a_base = uniform_ptr(p.a + m0 * p.lda);
        lc.b_base = uniform_ptr(tl.b + n0 * p.ldb);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int row = (wave * 4 + qd) * 8 + (lane >> 3);
            const uint32_t kbyte = (uint32_t)(swz(row, lane & 7) * 16);
            lc.a_off[qd] = (uint32_t)((min(m0 + row, m_end - 1) - m0) * p.lda) + kbyte;
            lc.b_off[qd] = (uint32_t)((min(n0 + row, N - 1) - n0) * p.ldb) + kbyte;
        }
        if (g == 1) {
            if constexpr (ROW) {
                // the tile's 256 column scales: wave 4+w, lane l -> column 64w + l
                lc.s_base = uniform_ptr(tl.sb + n0);
                lc.s_off = (uint32_t)(min(n0 + (wave & 3) * 64 + lane, N - 1) - n0) * 4u;
                lc.s_kstride = p.sbs0;
            } else {
                lc.s_base = uniform_ptr(tl.sb);
                lc.s_off = (uint32_t)(min((n0 >> 7) + (lane & 1), nb_last) * p.sbs0) * 4u;
                lc.s_kstride = p.sbs1;
            }
        } else {
            lc.s_base = uniform_ptr(p.sa + m0);
            lc.s_off = (uint32_t)(min(m0 + wm * 64 + lane, m_end - 1) - m0) * 4u;
            lc.s_kstride = p.ldsa;
        }
    };
    set_lc(cur);
    const int s_half = g == 1 ? BM : 0;
    auto stage_a = [&](int st) { return smem_ab[st]; };
    auto stage_b = [&](int st) { return smem_ab[st] + kSlabBytes; };
    auto stage_s = [&](int sst) { return &smem_s[sst][s_half]; };
    // Copy instructions q0 .. q1-1 (0-3 A rows, 4-7 B rows, 8 scales) of
    // step kb - kboff of the tile lc points at, A and B rows into stage st,
    // scales into scale stage sst.  kboff is 0, or nkb once lc has moved on
    // to the next tile; steps past the last one refill it (harmless: nothing
    // reads them).
    int kboff = 0;
    auto copies = [&](int q0, int q1, int kb, int st, int sst) {
        int kbc = kb - kboff;
        if (kbc >= nkb) kbc = nkb - 1;
#pragma unroll
        for (int q = 0; q < 9; ++q)
            if (q >= q0 && q < q1)
                issue_copy(q, lc, (int64_t)kbc * BK, kbc, stage_a(st), stage_b(st), stage_s(sst),
                           wave);
    };

    v4f acc[4][NJ];
    v8i af[4], bf[4];
    float sc[4];
    uint32_t sab[4] = {}, sbb = 0;   // POW2: E8M0 exponents of the sa rows and of sb
    // ROW128: the half's column scales (empty for BLOCK128)
    RowScales<ROW> rs;

    // COMP(kb,h): the 16 blocks (i, 4h+jj).  FP32 scales: each partial sum is
    // promoted kPromoteDist instructions after it was issued.
    auto comp = [&](int h) {
        const int nj = h == 0 ? 4 : NJ1;    // column blocks of this half
        if constexpr (POW2) {
#pragma unroll
            for (int tt = 0; tt < 16; ++tt)
                if ((tt & 3) < nj)
                    acc[tt >> 2][4 * h + (tt & 3)] = mfma_f8_scaled(
                        bf[tt & 3], af[tt >> 2], acc[tt >> 2][4 * h + (tt & 3)],
                        rs.e8m0(tt & 3, sbb), sab[tt >> 2]);
        } else {
            v4f part[kPartRing];
#pragma unroll
            for (int tt = 0; tt < 16 + kPromoteDist; ++tt) {
                if (tt < 16 && (tt & 3) < nj) part[tt % kPartRing] = mfma_f8(bf[tt & 3], af[tt >> 2]);
                if (tt >= kPromoteDist && ((tt - kPromoteDist) & 3) < nj) {
                    const int u = tt - kPromoteDist;
                    if constexpr (ROW)
                        promote<kScaleRow128>(acc[u >> 2][4 * h + (u & 3)], part[u % kPartRing],
                                              sc[u >> 2], rs.col(u & 3));
                    else
                        promote<kScaleBlock128>(acc[u >> 2][4 * h + (u & 3)], part[u % kPartRing],
                                                sc[u >> 2], make_float4(1.f, 1.f, 1.f, 1.f));
                }
            }
            // issue order pinned: kPromoteDist matrix instructions, then
            // each further one followed by the four FMAs of an earlier
            // partial (left to itself the scheduler packs the FMAs right
            // behind their own instruction, into hazard wait states)
#pragma unroll
            for (int tt = 0; tt < 16 + kPromoteDist; ++tt) {
                if (tt < 16 && (tt & 3) < nj) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (tt >= kPromoteDist && ((tt - kPromoteDist) & 3) < nj)
                    __builtin_amdgcn_sched_group_barrier(0x002, kPromoteValu, 0);
            }
        }
        // pins the half's accumulators here, so that none of the slot's
        // (memory-free) instructions is sunk past its closing barrier
        const int j0 = 4 * h;
        if (nj == 4) {
            asm volatile("" : "+v"(acc[0][j0]), "+v"(acc[0][j0 + 1]), "+v"(acc[0][j0 + 2]),
                              "+v"(acc[0][j0 + 3]), "+v"(acc[1][j0]), "+v"(acc[1][j0 + 1]),
                              "+v"(acc[1][j0 + 2]), "+v"(acc[1][j0 + 3]), "+v"(acc[2][j0]),
                              "+v"(acc[2][j0 + 1]), "+v"(acc[2][j0 + 2]), "+v"(acc[2][j0 + 3]),
                              "+v"(acc[3][j0]), "+v"(acc[3][j0 + 1]), "+v"(acc[3][j0 + 2]),
                              "+v"(acc[3][j0 + 3]));
        } else {
            asm volatile("" : "+v"(acc[0][j0]), "+v"(acc[0][j0 + 1]), "+v"(acc[0][j0 + 2]),
                              "+v"(acc[1][j0]), "+v"(acc[1][j0 + 1]), "+v"(acc[1][j0 + 2]),
                              "+v"(acc[2][j0]), "+v"(acc[2][j0 + 1]), "+v"(acc[2][j0 + 2]),
                              "+v"(acc[3][j0]), "+v"(acc[3][j0 + 1]), "+v"(acc[3][j0 + 2]));
        }
    };

    // Stage of step kb of the current tile: (kb + sbase) & 1.  The first
    // tile's prologue: step 0 complete; step 1's A rows and scales (its B
    // rows come with MEM(0,0)).  A later tile's step 0 and step 1 A rows and
    // scales are copied during the last two steps of the tile before it
    // (when K spans at least two steps), so it starts without a prologue.
    // ROW128: the scale stage of step kb is (kb + s3base) % 3.
    int sbase = 0, s3base = 0;
    auto sstage = [&](int kb, int st) { return ROW ? (kb + s3base) % 3 : st; };
    copies(0, 9, 0, 0, sstage(0, 0));
    copies(0, 4, 1, 1, sstage(1, 1));
    copies(8, 9, 1, 1, sstage(1, 1));
    stage_barrier();
    for (;;) {
        const uint32_t t_next = t + gridDim.x;
        const bool ahead = nkb >= 2 && t_next < total;   // next tile copied during this one
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
        kboff = 0;
        if (g == 1) slot_barrier();      // group 1 starts one slot later

        // The K loop starts on a 64-byte boundary.  Its placement relative to
        // the instruction fetch lines is worth 3-4 %: the same instructions,
        // shifted by an unrelated change elsewhere in the file, ran 915-923 us
        // instead of 874-886 us on the Fprop GEMM.
        asm volatile(".p2align 6");
        for (int kb = 0; kb < nkb; ++kb) {
            const int cur_st = (kb + sbase) & 1;
            const int cur_ss = sstage(kb, cur_st);   // scale stage of step kb
            {   // MEM(kb,0)
                const uint8_t* sa_ = stage_a(cur_st);
                const uint8_t* sb_ = stage_b(cur_st);
#pragma unroll
                for (int i = 0; i < 4; ++i) af[i] = frag32(sa_, wm * 4 + i, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) bf[j] = frag32(sb_, g * NJ + j, lane);
                if constexpr (POW2) {
                    if constexpr (!ROW) sbb = e8m0_of(smem_s[cur_ss][BM + g]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) sab[i] = e8m0_of(smem_s[cur_ss][wm * kWaveM + i * 16 + r16]);
                } else if constexpr (ROW) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[i] = smem_s[cur_ss][wm * kWaveM + i * 16 + r16];
                } else {
                    const float sbv = smem_s[cur_ss][BM + g];
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[i] = smem_s[cur_ss][wm * kWaveM + i * 16 + r16] * sbv;
                }
                if constexpr (ROW) rs.template load<POW2>(&smem_s[cur_ss][BM + g * kWN], 0, r16, kq);
                copies(4, 8, kb + 1, cur_st ^ 1, 0);
            }
            slot_barrier();
            comp(0);
            slot_barrier();
            {   // MEM(kb,1)
                const uint8_t* sb_ = stage_b(cur_st);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (j < NJ1) bf[j] = frag32(sb_, g * NJ + 4 + j, lane);
                if constexpr (ROW) rs.template load<POW2>(&smem_s[cur_ss][BM + g * kWN], 1, r16, kq);
                if (ahead && kb == nkb - 2) {   // from here on, copies fetch the next tile
                    // (opaque to the compiler, so that the next tile's copy
                    // offsets are computed here and not kept live through
                    // the whole loop)
                    uint32_t tn = t_next;
                    asm volatile("" : "+s"(tn));
                    set_lc(locate(tn));
                    kboff = nkb;
                }
                copies(0, 4, kb + 2, cur_st, 0);
                copies(8, 9, kb + 2, cur_st, sstage(kb + 2, cur_st));
            }
            // both groups: the same wait (for group 0 stricter than it needs,
            // see the schedule above), so no branch ahead of the compute slot
            slot_barrier_vm9();
            comp(1);
            slot_barrier_vm5();
        }
        if (g == 0) slot_barrier();      // group 0's idle last slot
        wait_vm_all();

        // ---- epilogue ----
        // Every wave's copies have landed (the next tile's steps 0 and 1, or
        // refills past the last step) and are published.  Each wave stores
        // its block through its own 32 B rows of the stage the last step
        // used, which nothing is copied into before the next tile's MEM(0,0)
        // (issued by the same wave, after its epilogue).
        __syncthreads();
        const int last_st = (nkb - 1 + sbase) & 1;
        store_tile<OUT, NJ>(kparams(), acc, stage_b(last_st) + wave * 4096, cur.m0 + wm * kWaveM,
                            cur.m_end, cur.n0 + g * kWN, lane);
        if (t_next >= total) break;
        t = t_next;
        sbase = (sbase + nkb) & 1;
        if constexpr (ROW) s3base = (s3base + nkb) % 3;
        cur = locate(t);
        if (!ahead) {
            // K spans one step: the next tile's prologue, once every wave's
            // epilogue has read its LDS buffer
            set_lc(cur);
            kboff = 0;
            __syncthreads();
            copies(0, 9, 0, sbase, sstage(0, sbase));
            copies(0, 4, 1, sbase ^ 1, sstage(1, sbase ^ 1));
            copies(8, 9, 1, sbase ^ 1, sstage(1, sbase ^ 1));
            stage_barrier();
        }
    }
}

// Compute units of the current device (cached per device; racing threads
// store the same value).
static int device_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Tile width of the ROW128 GEMM: the one with fewer column-passes,
// ceil(tiles / CUs) * width (ties: 256).
static int row_tile_n(int64_t M, int64_t N) {
    const int64_t cus = device_cu_count();
    const int64_t tm = (M + BM - 1) / BM;
    auto cost = [&](int64_t w) { return ((tm * ((N + w - 1) / w) + cus - 1) / cus) * w; };
    return cost(224) < cost(256) ? 224 : 256;
}

// Persistent grid: one workgroup per compute unit (a workgroup takes most of
// a CU's LDS), or fewer when there are fewer tiles.
static unsigned persistent_grid(int64_t tiles) {
    return (unsigned)std::min<int64_t>(tiles, device_cu_count());
}

hipError_t launch_gemm(const GemmParams& p, int scale_mode, int out_dtype, bool pow2,
                       hipStream_t stream) {
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    dim3 grid(persistent_grid(tiles)), block(kThreads);
    if (scale_mode == kScaleBlock128) {
        // dense Fprop / Dgrad: ping-pong schedule
        if (out_dtype == kBF16) {
            if (pow2) hipLaunchKernelGGL((gemm_pp_kernel<kBF16, true, false, kScaleBlock128>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((gemm_pp_kernel<kBF16, false, false, kScaleBlock128>), grid, block, 0, stream, p);
        } else {
            if (pow2) hipLaunchKernelGGL((gemm_pp_kernel<kF32, true, false, kScaleBlock128>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((gemm_pp_kernel<kF32, false, false, kScaleBlock128>), grid, block, 0, stream, p);
        }
        return hipGetLastError();
    }
    // ROW128 (Wgrad): per-column B scales; 224-wide tiles where they take
    // fewer column-passes over the chip (ceil(tiles / CUs) * width), e.g.
    // 2048 x 7168: 224 tiles of 256 on 256 CUs become 256 tiles of 224
    const int tbn = row_tile_n(p.M, p.N);
    dim3 g2(persistent_grid(((p.M + BM - 1) / BM) * ((p.N + tbn - 1) / tbn)));
#define FP8Q_ROW(OD, P2)                                                                                    \
    do {                                                                                                    \
        if (tbn == 224) hipLaunchKernelGGL((gemm_pp_kernel<OD, P2, false, kScaleRow128, 224>), g2, block, 0, stream, p); \
        else hipLaunchKernelGGL((gemm_pp_kernel<OD, P2, false, kScaleRow128, 256>), g2, block, 0, stream, p);            \
    } while (0)
    if (out_dtype == kBF16) {
        if (pow2) FP8Q_ROW(kBF16, true);
        else FP8Q_ROW(kBF16, false);
    } else {
        if (pow2) FP8Q_ROW(kF32, true);
        else FP8Q_ROW(kF32, false);
    }
#undef FP8Q_ROW
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmParams& p, int out_dtype, bool pow2, hipStream_t stream) {
    // upper bound on the tile count: sum_g ceil(rows_g/BM) <= M/BM + groups
    const int64_t tiles = ((p.M + BM - 1) / BM + p.num_groups) * ((p.N + BN - 1) / BN);
    dim3 grid(persistent_grid(tiles)), block(kThreads);
#define FP8Q_GGEMM(OD, P2) \
    hipLaunchKernelGGL((gemm_pp_kernel<OD, P2, true, kScaleBlock128>), grid, block, 0, stream, p)
    if (out_dtype == kBF16) {
        if (pow2) FP8Q_GGEMM(kBF16, true);
        else FP8Q_GGEMM(kBF16, false);
    } else {
        if (pow2) FP8Q_GGEMM(kF32, true);
        else FP8Q_GGEMM(kF32, false);
    }
#undef FP8Q_GGEMM
    return hipGetLastError();
}

}  // namespace fp8q
