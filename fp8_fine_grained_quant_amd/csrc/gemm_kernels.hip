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
// Design (one workgroup = one 256x256 output tile, 8 waves, 2 per SIMD):
//  * K step 128 = exactly one scale block, so each K step is one
//    v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 output block (scale
//    operands set to 1.0; the FP32 block scales are applied by the
//    promotion FMA).
//  * A and B K-slabs (256x128 bytes each) go HBM -> LDS with
//    global_load_lds_dwordx4 (no VGPR staging), double buffered: the next
//    slab streams in while the current one is multiplied.  LDS rows are
//    128 bytes; 16-byte chunk c of row r is stored at slot c ^ (r & 7) so
//    that the fragment reads (16 rows, same chunk) hit distinct banks.
//  * Wave tile 64(M) x 128(N): 4 x 8 blocks of 16x16, 128 FP32 accumulator
//    VGPRs.  The MFMA is issued with the B slab as its first operand, so a
//    lane's four result registers are four CONSECUTIVE output columns of one
//    row: the epilogue writes 16-byte (FP32) or 8-byte (BF16) runs, and the
//    128x128-block weight scale is a wave-uniform scalar.
//  * Workgroup -> tile mapping keeps each XCD on a contiguous range of tiles
//    and walks them in groups of 8 tile rows so that concurrently running
//    tiles share A rows and B columns in that XCD's L2.
//  * Tails in M and N: loads clamp the row index (never read out of bounds),
//    stores are masked.
#include "device_common.h"
#include "kernels.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 512;
constexpr int kWaveM = 64;
constexpr int kWaveN = 128;
constexpr int kSlabBytes = BM * BK;          // one operand, one stage
constexpr int kStageBytes = 2 * kSlabBytes;  // A + B
constexpr int kGroupM = 8;                   // tile rows per swizzle group
constexpr unsigned kOneE8M0 = 127;           // MFMA block scale 2^0

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

__device__ __forceinline__ v8i frag32(const uint8_t* __restrict__ slab, int row, int kq) {
    // 32 bytes of row `row` of a 128-byte-per-row swizzled slab: logical
    // 16-byte chunks 2*kq and 2*kq+1 (stored at chunk ^ (row & 7)).
    const uint8_t* rb = slab + row * BK;
    const uint4 x0 = *reinterpret_cast<const uint4*>(rb + (((2 * kq) ^ (row & 7)) << 4));
    const uint4 x1 = *reinterpret_cast<const uint4*>(rb + (((2 * kq + 1) ^ (row & 7)) << 4));
    return (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                 (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        a, b, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0, kOneE8M0, 0, kOneE8M0);
}

// Everything a wave needs to stream one K step of A, B and the scales into
// an LDS stage.
struct LoadCtx {
    const uint8_t* a_base;  // A + m0*lda (wave-uniform)
    const uint8_t* b_base;  // B + n0*ldb (wave-uniform)
    uint32_t a_off[4];      // per 8-row block: row*lda + swizzled chunk offset
    uint32_t b_off[4];
    const float* s_base;    // scale row of K step 0 (sa, or sb in ROW128 mode)
    uint32_t s_off;         // this lane's element offset, in bytes
    int64_t s_kstride;      // scale elements per K step
};

// One K step: issue the HBM -> LDS copy of step kb+1 into `nxt_*` (when
// `issue`), then multiply the operands of step kb held in `cur_*`.  The
// restrict-qualified stage pointers let the compiler see that the copy in
// flight never writes the stage being read, so it does not wait for it;
// completion is awaited explicitly (vmcnt) before the next step's barrier.
template <int SCALE_MODE>
__device__ __forceinline__ void kstep(const uint8_t* __restrict__ cur_a,
                                      const uint8_t* __restrict__ cur_b,
                                      const float* __restrict__ cur_sa,
                                      const float* __restrict__ cur_sb,
                                      uint8_t* __restrict__ nxt_a, uint8_t* __restrict__ nxt_b,
                                      float* __restrict__ nxt_s, bool issue, int64_t koff_next,
                                      int kb_next, const LoadCtx& lc, int wave, int wm, int wn,
                                      int lane, v4f (&acc)[4][8]) {
    if (issue) {
        const uint8_t* ab = lc.a_base + koff_next;
        const uint8_t* bb = lc.b_base + koff_next;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
            dma16(ab, lc.a_off[qd], lds_addr(nxt_a + (wave * 4 + qd) * 1024));
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
            dma16(bb, lc.b_off[qd], lds_addr(nxt_b + (wave * 4 + qd) * 1024));
        dma4(lc.s_base + (int64_t)kb_next * lc.s_kstride, lc.s_off,
             lds_addr(nxt_s + (wave & 3) * 64));
    }

    const int r16 = lane & 15;
    const int kq = lane >> 4;
    v8i af[4];
    float sc[4];
    const float sbv = SCALE_MODE == kScaleBlock128 ? cur_sb[wn] : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wm * kWaveM + i * 16 + r16;
        af[i] = frag32(cur_a, row, kq);
        sc[i] = cur_sa[row];
        if (SCALE_MODE == kScaleBlock128) sc[i] *= sbv;
    }
    // Two partial-sum sets: the MFMAs of column block j run while the
    // promotion FMAs of block j-1 retire.
    v4f part[2][4];
    v8i bf = frag32(cur_b, wn * kWaveN + r16, kq);
#pragma unroll
    for (int i = 0; i < 4; ++i) part[0][i] = mfma_f8(bf, af[i]);
#pragma unroll
    for (int j = 1; j <= 8; ++j) {
        const int cb = j & 1, pb = cb ^ 1;
        if (j < 8) {
            bf = frag32(cur_b, wn * kWaveN + j * 16 + r16, kq);
#pragma unroll
            for (int i = 0; i < 4; ++i) part[cb][i] = mfma_f8(bf, af[i]);
        }
        float4 sbq = make_float4(1.f, 1.f, 1.f, 1.f);
        if (SCALE_MODE == kScaleRow128)
            sbq = *reinterpret_cast<const float4*>(&cur_sb[wn * kWaveN + (j - 1) * 16 + kq * 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v4f& a = acc[i][j - 1];
            const v4f& pp = part[pb][i];
            if (SCALE_MODE == kScaleBlock128) {
                a[0] = fmaf(pp[0], sc[i], a[0]);
                a[1] = fmaf(pp[1], sc[i], a[1]);
                a[2] = fmaf(pp[2], sc[i], a[2]);
                a[3] = fmaf(pp[3], sc[i], a[3]);
            } else {
                a[0] = fmaf(pp[0], sc[i] * sbq.x, a[0]);
                a[1] = fmaf(pp[1], sc[i] * sbq.y, a[1]);
                a[2] = fmaf(pp[2], sc[i] * sbq.z, a[2]);
                a[3] = fmaf(pp[3], sc[i] * sbq.w, a[3]);
            }
        }
    }
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int SCALE_MODE, int OUT, bool GROUPED>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem_ab[2][kStageBytes];
    // [stage][0..255]: sa of the tile's rows; [stage][256..511]: ROW128: sb
    // of the tile's columns; BLOCK128: the two 128x128-block weight scales of
    // the tile's column halves, at [256] and [257] (each fetched by 32 lanes)
    __shared__ __attribute__((aligned(16))) float smem_s[2][BM + BN];
    __shared__ int32_t tile_start[GROUPED ? (kMaxGroups + 1) : 1];
    __shared__ int32_t wave_tot[kThreads / 64];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps it in SGPRs
    const int lane = tid & 63;
    const int wm = wave & 3;   // wave row (64 rows each)
    const int wn = wave >> 2;  // wave column (128 columns each)

    const int64_t N = p.N;
    const int64_t tiles_n = (N + BN - 1) / BN;
    const uint8_t* __restrict__ bptr = p.b;
    const float* __restrict__ sbptr = p.sb;
    int64_t m0, m_end, n0;

    if (!GROUPED) {
        const int64_t tiles_m = (p.M + BM - 1) / BM;
        const int64_t T = tiles_m * tiles_n;
        int64_t t = blockIdx.x;
        if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);  // contiguous range per XCD
        const int64_t grp = t / (kGroupM * tiles_n);
        const int64_t first_m = grp * kGroupM;
        const int64_t gm = min(tiles_m - first_m, (int64_t)kGroupM);
        const int64_t rem = t - grp * kGroupM * tiles_n;
        m0 = (first_m + rem % gm) * BM;
        n0 = (rem / gm) * BN;
        m_end = p.M;
    } else {
        // Tile table: group g owns tiles [tile_start[g], tile_start[g+1]),
        // ceil(rows_g/BM) * tiles_n of them, in (m-tile, n-tile) order.
        const int64_t G = p.num_groups;
        const int per = (int)((G + kThreads - 1) / kThreads);
        const int g0 = tid * per;
        int32_t local = 0;
        for (int g = g0; g < g0 + per && g < G; ++g) {
            const int32_t rows = p.offsets[g + 1] - p.offsets[g];
            local += (rows + BM - 1) / BM * (int32_t)tiles_n;
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
            run += (rows + BM - 1) / BM * (int32_t)tiles_n;
        }
        if (tid == kThreads - 1) tile_start[G] = run;
        __syncthreads();
        const int32_t t = (int32_t)blockIdx.x;
        if (t >= tile_start[G]) return;  // whole workgroup: uniform exit
        int lo = 0, hi = (int)G;         // tile_start[lo] <= t < tile_start[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tile_start[mid] <= t) lo = mid; else hi = mid;
        }
        const int g = lo;
        const int32_t local_t = t - tile_start[g];
        const int64_t tm = local_t / tiles_n;
        const int64_t tn = local_t - tm * tiles_n;
        m0 = p.offsets[g] + tm * BM;
        m_end = p.offsets[g + 1];
        n0 = tn * BN;
        bptr += (int64_t)g * N * p.ldb;
        sbptr += (int64_t)g * ((N + 127) / 128) * (p.K / 128);
    }

    const int nkb = (int)(p.K / BK);
    const int64_t nb_last = (N + 127) / 128 - 1;

    // Per-lane copy sources.  Instruction qd of wave w moves rows
    // 8*(4w+qd) .. +7 of a slab; lane l carries row +l/8, stored 16-byte
    // slot l%8, which holds logical chunk (l%8) ^ (row & 7).  Rows past the
    // tile's end are clamped (their results are never stored).
    // Offsets stay below 2^32: a tile spans 256 rows of at most 2^24 bytes
    // each (the host rejects larger leading dimensions).
    m0 = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)m0) |
         ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)m0 >> 32)) << 32);
    LoadCtx lc;
    {
        const int r_in = lane >> 3;
        const int slot = lane & 7;
        lc.a_base = uniform_ptr(p.a + m0 * p.lda);
        lc.b_base = uniform_ptr(bptr + n0 * p.ldb);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int row = (wave * 4 + qd) * 8 + r_in;
            const uint32_t chunk = (uint32_t)((slot ^ (row & 7)) * 16);
            lc.a_off[qd] = (uint32_t)((min(m0 + row, m_end - 1) - m0) * p.lda) + chunk;
            lc.b_off[qd] = (uint32_t)((min(n0 + row, N - 1) - n0) * p.ldb) + chunk;
        }
        if (SCALE_MODE == kScaleRow128 && wave >= 4) {
            lc.s_base = uniform_ptr(sbptr + n0);
            lc.s_off = (uint32_t)(min(n0 + (wave - 4) * 64 + lane, N - 1) - n0) * 4u;
            lc.s_kstride = p.sbs0;
        } else if (wave >= 4) {
            // BLOCK128: lane l fetches the weight block scale of wave column
            // l&1 (block n0/128 + (l&1)); smem_s[st][BM + wn] is then read
            // by wave column wn.
            lc.s_base = uniform_ptr(sbptr);
            lc.s_off = (uint32_t)(min((n0 >> 7) + (lane & 1), nb_last) * p.sbs0) * 4u;
            lc.s_kstride = p.sbs1;
        } else {
            lc.s_base = uniform_ptr(p.sa + m0);
            lc.s_off = (uint32_t)(min(m0 + (wave & 3) * 64 + lane, m_end - 1) - m0) * 4u;
            lc.s_kstride = p.ldsa;
        }
    }
    const int s_half = wave >= 4 ? BM : 0;  // which half of smem_s this wave fills

    v4f acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};


    // prologue: step 0 into stage 0
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
        dma16(lc.a_base, lc.a_off[qd], lds_addr(smem_ab[0] + (wave * 4 + qd) * 1024));
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
        dma16(lc.b_base, lc.b_off[qd], lds_addr(smem_ab[0] + kSlabBytes + (wave * 4 + qd) * 1024));
    dma4(lc.s_base, lc.s_off, lds_addr(&smem_s[0][s_half] + (wave & 3) * 64));

    for (int kb = 0; kb < nkb; ++kb) {
        const int st = kb & 1;
        // this wave's copies of step kb have landed; after the barrier every
        // wave's have, and every wave has finished reading stage st^1
        wait_vm_all();
        barrier();
        kstep<SCALE_MODE>(smem_ab[st], smem_ab[st] + kSlabBytes, &smem_s[st][0], &smem_s[st][BM],
                          smem_ab[st ^ 1], smem_ab[st ^ 1] + kSlabBytes, &smem_s[st ^ 1][s_half],
                          kb + 1 < nkb, (int64_t)(kb + 1) * BK, kb + 1, lc, wave, wm, wn, lane,
                          acc);
    }

    // ---- epilogue: lane holds rows m, columns n..n+3 of each 16x16 block ----
    const int r16 = lane & 15;
    const int kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * kWaveM + i * 16 + r16;
        if (m >= m_end) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t n = n0 + wn * kWaveN + j * 16 + kq * 4;
            if (n >= N) continue;
            const v4f v = acc[i][j];
            if (OUT == kF32) {
                float* cp = static_cast<float*>(p.c) + m * p.ldc + n;
                if (n + 4 <= N) {
                    *reinterpret_cast<float4*>(cp) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
                    for (int e = 0; e < 4 && n + e < N; ++e) cp[e] = v[e];
                }
            } else {
                uint16_t* cp = static_cast<uint16_t*>(p.c) + m * p.ldc + n;
                const uint32_t h0 = float_to_bf16_bits(v[0]), h1 = float_to_bf16_bits(v[1]);
                const uint32_t h2 = float_to_bf16_bits(v[2]), h3 = float_to_bf16_bits(v[3]);
                if (n + 4 <= N) {
                    *reinterpret_cast<uint2*>(cp) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
                } else {
                    const uint32_t h[4] = {h0, h1, h2, h3};
                    for (int e = 0; e < 4 && n + e < N; ++e) cp[e] = (uint16_t)h[e];
                }
            }
        }
    }
}

hipError_t launch_gemm(const GemmParams& p, int scale_mode, int out_dtype, hipStream_t stream) {
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    dim3 grid((unsigned)tiles), block(kThreads);
#define FP8Q_GEMM(SM, OD) hipLaunchKernelGGL((gemm_kernel<SM, OD, false>), grid, block, 0, stream, p)
    if (scale_mode == kScaleBlock128) {
        if (out_dtype == kBF16) FP8Q_GEMM(kScaleBlock128, kBF16);
        else FP8Q_GEMM(kScaleBlock128, kF32);
    } else {
        if (out_dtype == kBF16) FP8Q_GEMM(kScaleRow128, kBF16);
        else FP8Q_GEMM(kScaleRow128, kF32);
    }
#undef FP8Q_GEMM
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmParams& p, int out_dtype, hipStream_t stream) {
    // upper bound on the tile count: sum_g ceil(rows_g/BM) <= M/BM + groups
    const int64_t tiles = ((p.M + BM - 1) / BM + p.num_groups) * ((p.N + BN - 1) / BN);
    dim3 grid((unsigned)tiles), block(kThreads);
    if (out_dtype == kBF16)
        hipLaunchKernelGGL((gemm_kernel<kScaleBlock128, kBF16, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<kScaleBlock128, kF32, true>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fp8q
