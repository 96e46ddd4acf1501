// mfma_rates.hip -- register-only throughput probe of the GEMM's compute
// slot on the full chip (test infrastructure; not part of the library).
//
// Every workgroup has 512 threads (8 waves, the GEMM kernel's shape and
// register budget: at most 256 VGPRs per wave, no accumulation registers),
// one workgroup per compute unit.  Each wave owns a 64x128 FP32 accumulator
// tile and repeatedly runs one K step of it on register-resident FP8
// fragments, as the GEMM's compute slots do, with no LDS or memory traffic:
//   16x16x128 : 32 v_mfma_f32_16x16x128_f8f6f4 per step (the GEMM's
//               unscaled instruction), either accumulating in place or writing a fresh
//               partial sum that an FP32 FMA promotes four instructions
//               later (the FP32-scale GEMM's promotion), or -- "row x
//               column", the weight-gradient GEMM's per-row scales on both
//               operands -- with four products of a row scale and four
//               column scales ahead of the four FMAs;
//   32x32x64  : 16 v_mfma_f32_32x32x64_f8f6f4, chained in pairs over
//               one 128-wide K block, either in place or into a partial sum
//               promoted with 16 FMAs two blocks later.
// "2 waves/SIMD": all 8 waves compute; "1 wave/SIMD": waves 4-7 leave at
// once, as in the ping-pong schedule where one wave per SIMD computes while
// the other moves data.  Prints TFLOP/s and the fraction of 5.0 PFLOP/s.
//
// Usage: mfma_rates [iterations]
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                                \
    do {                                                                                        \
        hipError_t e_ = (x);                                                                    \
        if (e_ != hipSuccess) {                                                                 \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);          \
            std::exit(1);                                                                       \
        }                                                                                       \
    } while (0)

// Zero scale operands: the compiler emits the plain (unscaled) instruction,
// as the GEMM's FP32-scale path does.
__device__ __forceinline__ v4f mf16(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v16f mf32(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

enum { k16InPlace, k16Promote, k32InPlace, k32Promote, k16PromoteRow };

template <int MODE, bool ONE_WAVE>
__global__ __launch_bounds__(512, 1) void probe(const int* __restrict__ seed, float* __restrict__ out,
                                                int iters) {
    if (ONE_WAVE && (threadIdx.x >> 6) >= 4) return;
    const int lane = threadIdx.x & 63;
    v8i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            af[i][e] = seed[(lane * 8 + e + i * 512) & 1023];
            bf[i][e] = seed[(lane * 8 + e + i * 512 + 77) & 1023];
        }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = 1.0f + 0.001f * (float)(lane + i);
    float4 cs[4];   // per-column scales of the four column blocks (row-scaled B)
#pragma unroll
    for (int j = 0; j < 4; ++j)
        cs[j] = make_float4(1.f + 0.002f * lane, 1.f - 0.001f * j, 1.f + 0.003f * j, 0.5f + 0.001f * lane);
    float sum = 0.f;
    if constexpr (MODE == k16InPlace || MODE == k16Promote || MODE == k16PromoteRow) {
        v4f acc[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (MODE == k16InPlace) {
#pragma unroll
                    for (int t = 0; t < 16; ++t)
                        acc[t >> 2][4 * h + (t & 3)] = mf16(bf[t & 3], af[t >> 2], acc[t >> 2][4 * h + (t & 3)]);
                } else {
                    constexpr int D = 4, R = D + 1;
                    v4f part[R];
#pragma unroll
                    for (int t = 0; t < 16 + D; ++t) {
                        if (t < 16) part[t % R] = mf16(bf[t & 3], af[t >> 2], (v4f){0.f, 0.f, 0.f, 0.f});
                        if (t >= D) {
                            const int u = t - D;
                            v4f& a = acc[u >> 2][4 * h + (u & 3)];
                            if constexpr (MODE == k16PromoteRow) {
                                // row scale times the lane's four column scales, then the FMAs
                                const float4 c = cs[u & 3];
                                a[0] = fmaf(part[u % R][0], sc[u >> 2] * c.x, a[0]);
                                a[1] = fmaf(part[u % R][1], sc[u >> 2] * c.y, a[1]);
                                a[2] = fmaf(part[u % R][2], sc[u >> 2] * c.z, a[2]);
                                a[3] = fmaf(part[u % R][3], sc[u >> 2] * c.w, a[3]);
                            } else {
#pragma unroll
                                for (int r = 0; r < 4; ++r) a[r] = fmaf(part[u % R][r], sc[u >> 2], a[r]);
                            }
                        }
                    }
#pragma unroll
                    for (int t = 0; t < 16 + D; ++t) {
                        if (t < 16) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (t >= D) __builtin_amdgcn_sched_group_barrier(0x002, MODE == k16PromoteRow ? 8 : 4, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // as if the fragments and scales were reloaded for every half
                // step (loop-invariant scale products would otherwise leave
                // the loop, and row x column would issue 4 VALU instructions
                // per matrix instruction instead of the GEMM's 8)
                asm volatile("" : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(bf[0]),
                                  "+v"(bf[1]), "+v"(bf[2]), "+v"(bf[3]));
                asm volatile("" : "+v"(sc[0]), "+v"(sc[1]), "+v"(sc[2]), "+v"(sc[3]));
                if constexpr (MODE == k16PromoteRow)
                    asm volatile("" : "+v"(cs[0].x), "+v"(cs[0].y), "+v"(cs[0].z), "+v"(cs[0].w),
                                      "+v"(cs[1].x), "+v"(cs[1].y), "+v"(cs[1].z), "+v"(cs[1].w),
                                      "+v"(cs[2].x), "+v"(cs[2].y), "+v"(cs[2].z), "+v"(cs[2].w),
                                      "+v"(cs[3].x), "+v"(cs[3].y), "+v"(cs[3].z), "+v"(cs[3].w));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    } else {
        // 32x32 blocks: the 64x128 tile is 2 (i) x 4 (j) blocks, a half step
        // covers j in {2h, 2h+1}; fragments af[2i + kh], bf[2jj + kh]
        v16f acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (MODE == k32InPlace) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int i = b >> 1, jj = b & 1;
                        acc[i][2 * h + jj] = mf32(bf[2 * jj], af[2 * i], acc[i][2 * h + jj]);
                        acc[i][2 * h + jj] = mf32(bf[2 * jj + 1], af[2 * i + 1], acc[i][2 * h + jj]);
                    }
                } else {
                    v16f part[3];
                    const v16f z = {};
#pragma unroll
                    for (int b = 0; b < 6; ++b) {
                        if (b < 4) {
                            const int i = b >> 1, jj = b & 1;
                            part[b % 3] = mf32(bf[2 * jj], af[2 * i], z);
                            part[b % 3] = mf32(bf[2 * jj + 1], af[2 * i + 1], part[b % 3]);
                        }
                        if (b >= 2) {
                            const int u = b - 2, i = u >> 1, jj = u & 1;
                            v16f& a = acc[i][2 * h + jj];
#pragma unroll
                            for (int e = 0; e < 16; ++e) a[e] = fmaf(part[u % 3][e], sc[i], a[e]);
                        }
                    }
#pragma unroll
                    for (int b = 0; b < 6; ++b) {
                        if (b < 4) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (b >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                        if (b < 4) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (b >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("" : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(bf[0]),
                                  "+v"(bf[1]), "+v"(bf[2]), "+v"(bf[3]));
                asm volatile("" : "+v"(sc[0]), "+v"(sc[1]));
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) sum += acc[i][j][e];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

template <int MODE, bool ONE_WAVE>
static void run(const char* name, const int* dseed, float* dout, int cus, int iters) {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int w = 0; w < 3; ++w)
        hipLaunchKernelGGL((probe<MODE, ONE_WAVE>), dim3(cus), dim3(512), 0, 0, dseed, dout, iters);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    std::vector<float> ms(5);
    for (auto& m : ms) {
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL((probe<MODE, ONE_WAVE>), dim3(cus), dim3(512), 0, 0, dseed, dout, iters);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipEventElapsedTime(&m, e0, e1));
    }
    std::sort(ms.begin(), ms.end());
    const double med = ms[2] * 1e-3;
    // per wave and iteration: 2 x 16 x (16x16x128) = 32 x 65536 FLOP, the same for 32x32x64
    const double flop = (double)cus * (ONE_WAVE ? 4 : 8) * iters * 32.0 * 65536.0;
    std::printf("%-40s %9.3f ms  %7.1f TFLOP/s  %.3f of 5.0 PFLOP/s\n", name, med * 1e3,
                flop / med / 1e12, flop / med / 5.0e15);
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
}

int main(int argc, char** argv) {
    int dev = 0, cus = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    const int iters = argc > 1 ? std::max(1, std::atoi(argv[1])) : 4000;
    std::printf("compute units %d, iterations %d\n", cus, iters);
    std::vector<int> seed(1024);
    unsigned x = 12345;
    for (auto& v : seed) {
        x = x * 1664525u + 1013904223u;
        v = (int)(x & 0x3F3F3F3Fu);   // finite E4M3 codes of magnitude below 2
    }
    int* dseed = nullptr;
    float* dout = nullptr;
    CHECK(hipMalloc(&dseed, seed.size() * sizeof(int)));
    CHECK(hipMalloc(&dout, (size_t)cus * 512 * sizeof(float)));
    CHECK(hipMemcpy(dseed, seed.data(), seed.size() * sizeof(int), hipMemcpyHostToDevice));
    for (int rep = 0; rep < 2; ++rep) {
        run<k16InPlace, false>("2 waves/SIMD 16x16x128 in place", dseed, dout, cus, iters);
        run<k16Promote, false>("2 waves/SIMD 16x16x128 + FP32 promotion", dseed, dout, cus, iters);
        run<k32InPlace, false>("2 waves/SIMD 32x32x64 in place", dseed, dout, cus, iters);
        run<k32Promote, false>("2 waves/SIMD 32x32x64 + FP32 promotion", dseed, dout, cus, iters);
        run<k16PromoteRow, false>("2 waves/SIMD 16x16x128 + row x column", dseed, dout, cus, iters);
        run<k16InPlace, true>("1 wave/SIMD 16x16x128 in place", dseed, dout, cus, iters);
        run<k16Promote, true>("1 wave/SIMD 16x16x128 + FP32 promotion", dseed, dout, cus, iters);
        run<k32InPlace, true>("1 wave/SIMD 32x32x64 in place", dseed, dout, cus, iters);
        run<k32Promote, true>("1 wave/SIMD 32x32x64 + FP32 promotion", dseed, dout, cus, iters);
        run<k16PromoteRow, true>("1 wave/SIMD 16x16x128 + row x column", dseed, dout, cus, iters);
    }
    CHECK(hipFree(dseed));
    CHECK(hipFree(dout));
    return 0;
}
