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
// rows of codes with non-temporal 16-byte accesses, up to eight per lane in
// flight (a 7168-byte row in one round; four per lane took two rounds and
// ran ~1 % slower, temporal stores ~5 % slower);
// then the workgroup moves the scales of its 32 rows group by group, so the
// writes of 32 consecutive rows of a scale row are contiguous (the reads are
// gathered by token).
#include "kernels.h"

namespace fp8q {

namespace {

constexpr int kDispRows = 32;
constexpr int kDispThreads = 256;

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
                    if (c + u * 64 < n16) v[u] = __builtin_nontemporal_load(s16 + c + u * 64);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (c + u * 64 < n16) __builtin_nontemporal_store(v[u], d16 + c + u * 64);
            }
            done = n16 << 4;
        }
        for (int64_t c = done + lane; c < p.cols; c += 64) dst[c] = src[c];
    }

    const int64_t groups = (p.cols + 127) / 128;
    for (int64_t e = tid; e < groups * kDispRows; e += kDispThreads) {
        const int64_t g = e / kDispRows;
        const int64_t r = r0 + e % kDispRows;
        if (r >= p.rows) continue;
        const int32_t t = p.index[r];
        if (t < 0 || (int64_t)t >= p.src_rows) continue;
        p.s_dst[g * p.lds_dst + r] = p.s_src[g * p.lds_src + t];
    }
}

}  // namespace

hipError_t launch_dispatch_rows(const DispatchParams& p, hipStream_t stream) {
    const int64_t blocks = (p.rows + kDispRows - 1) / kDispRows;
    hipLaunchKernelGGL(dispatch_rows_kernel, dim3((unsigned)blocks), dim3(kDispThreads), 0, stream,
                       p);
    return hipGetLastError();
}

}  // namespace fp8q
