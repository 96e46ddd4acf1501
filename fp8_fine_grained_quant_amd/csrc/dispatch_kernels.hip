// dispatch_kernels.hip -- FP8 dispatch permutation for the MoE up-projection.
//
// The activations feeding the MoE up-projection are quantized once per token
// (1x128 groups) and dispatched to the experts in FP8 together with their
// scales (jp-study.kr page, passage on quantizing before the MoE
// up-projection and dispatching in FP8).  On one GPU the dispatch is a row
// gather: row r of the expert-ordered operand is token index[r]'s row of
// codes, and its 1x128 scales follow it.
//
// HBM-bound: per output row, cols code bytes read and written, 4 bytes of
// scale read and written per 128 columns, and one index.
//
// Layout: one workgroup (4 waves) per 32 output rows.  Each wave moves whole
// rows of codes with 16-byte accesses, up to eight per lane in flight (a
// 7168-byte row in one round; four per lane took two rounds and ran ~1 %
// slower).  The loads are ordinary ones: with top-k routing every token row
// is read k times, and a token-ordered operand that fits the memory-side
// cache (32768 x 7168 codes, 235 MB) then serves the repeats from there;
// non-temporal loads, which bypass it, made the MoE dispatch 1.29x slower.
// The stores are non-temporal (the output is far larger than the cache;
// ordinary stores ~5 % slower).
// Scales are moved in a second decomposition: workgroup b takes 256 rows and
// the scale groups of slot b % 8.  Workgroups are dealt to the 8 XCDs
// round-robin, so each XCD gathers from one eighth of the source scale rows,
// which its L2 then holds (a gather of 4-byte words by token otherwise
// misses the L2 with every word).
#include "kernels.h"

namespace fp8q {

namespace {

constexpr int kDispRows = 32;
constexpr int kDispThreads = 256;
constexpr int kScaleRows = kDispThreads;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kDispThreads) void dispatch_rows_kernel(DispatchParams p) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * kDispRows;

    for (int i = wave; i < kDispRows; i += kDispThreads / 64) {
        const int64_t r = r0 + i;
        if (r >= p.rows) break;
        const int32_t t = __builtin_amdgcn_readfirstlane(p.index[r]);
        if (t < 0 || (int64_t)t >= p.src_rows) continue;   // skipped row
        const uint8_t* src = p.q_src + (int64_t)t * p.ldq_src;
        uint8_t* dst = p.q_dst + r * p.ldq_dst;
        int64_t done = 0;
        if (p.vec) {
            const int64_t n16 = p.cols >> 4;
            const u32x4* s16 = reinterpret_cast<const u32x4*>(src);
            u32x4* d16 = reinterpret_cast<u32x4*>(dst);
            for (int64_t c = lane; c < n16; c += 8 * 64) {
                u32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (c + u * 64 < n16) v[u] = s16[c + u * 64];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (c + u * 64 < n16) __builtin_nontemporal_store(v[u], d16 + c + u * 64);
            }
            done = n16 << 4;
        }
        for (int64_t c = done + lane; c < p.cols; c += 64) dst[c] = src[c];
    }

    // Scales: workgroup b gathers those of rows [kScaleRows*(b/8), +kScaleRows)
    // in the groups of slot b%8, [slot*G/8, (slot+1)*G/8), one row per thread.
    const int64_t groups = (p.cols + 127) / 128;
    const int slot = blockIdx.x & 7;
    const int64_t g0 = groups * slot / 8, g1 = groups * (slot + 1) / 8;
    const int64_t r = (int64_t)(blockIdx.x >> 3) * kScaleRows + tid;
    if (r >= p.rows || g0 == g1) return;
    const int32_t t = p.index[r];
    if (t < 0 || (int64_t)t >= p.src_rows) return;
    for (int64_t gc = g0; gc < g1; gc += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (gc + u < g1) v[u] = p.s_src[(gc + u) * p.lds_src + t];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (gc + u < g1) p.s_dst[(gc + u) * p.lds_dst + r] = v[u];
    }
}

}  // namespace

hipError_t launch_dispatch_rows(const DispatchParams& p, hipStream_t stream) {
    // 8 workgroups per 256 rows cover both decompositions (kScaleRows is 8 * kDispRows)
    static_assert(kScaleRows == 8 * kDispRows, "one grid serves codes and scales");
    const int64_t blocks = 8 * ((p.rows + kScaleRows - 1) / kScaleRows);
    hipLaunchKernelGGL(dispatch_rows_kernel, dim3((unsigned)blocks), dim3(kDispThreads), 0, stream,
                       p);
    return hipGetLastError();
}

}  // namespace fp8q
