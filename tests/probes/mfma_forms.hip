// mfma_forms.hip -- the GEMM's FP32-scale path issues the 16x16x128 FP8
// matrix instruction without scale operands (the builtin with zero scale
// operands compiles to v_mfma_f32_16x16x128_f8f6f4), where the scaled form
// v_mfma_scale_f32_16x16x128_f8f6f4 would carry unit E8M0 scales (127,
// 2^0).  This probe runs both on the same random E4M3 operands and counts
// the outputs whose bit patterns agree (test infrastructure; not part of
// the library).
//
// 1024 one-wave blocks; lane i of block b reads operand words [64b + i] of
// two arrays of 8-dword fragments and writes one 4-float result per form.
// Exit status 0 if every output agrees, 3 if not, 1 on a HIP error.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                       \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                              \
        }                                                                              \
    } while (0)

__global__ __launch_bounds__(64) void forms(const v8i* a, const v8i* b, v4f* scaled, v4f* plain) {
    const int i = blockIdx.x * 64 + threadIdx.x;
    const v8i x = a[i], y = b[i];
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    scaled[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, z, 0, 0, 0, 127, 0, 127);
    plain[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, z, 0, 0, 0, 0, 0, 0);
}

int main() {
    const int blocks = 1024, n = blocks * 64;
    std::vector<int> ha((size_t)n * 8), hb((size_t)n * 8);
    unsigned s = 12345u;
    auto byte = [&]() {   // a random E4M3 byte that is not NaN (S.1111.111)
        s = s * 1664525u + 1013904223u;
        unsigned c = (s >> 24) & 0xFFu;
        return (c & 0x7Fu) == 0x7Fu ? c ^ 1u : c;
    };
    for (size_t i = 0; i < ha.size(); ++i) {
        unsigned w = 0, v = 0;
        for (int k = 0; k < 4; ++k) {
            w |= byte() << (8 * k);
            v |= byte() << (8 * k);
        }
        ha[i] = (int)w;
        hb[i] = (int)v;
    }
    v8i *da, *db;
    v4f *ds, *dp;
    CHECK(hipMalloc(&da, (size_t)n * sizeof(v8i)));
    CHECK(hipMalloc(&db, (size_t)n * sizeof(v8i)));
    CHECK(hipMalloc(&ds, (size_t)n * sizeof(v4f)));
    CHECK(hipMalloc(&dp, (size_t)n * sizeof(v4f)));
    CHECK(hipMemcpy(da, ha.data(), (size_t)n * sizeof(v8i), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, hb.data(), (size_t)n * sizeof(v8i), hipMemcpyHostToDevice));
    hipLaunchKernelGGL(forms, dim3(blocks), dim3(64), 0, 0, da, db, ds, dp);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    std::vector<float> rs((size_t)n * 4), rp((size_t)n * 4);
    CHECK(hipMemcpy(rs.data(), ds, (size_t)n * sizeof(v4f), hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(rp.data(), dp, (size_t)n * sizeof(v4f), hipMemcpyDeviceToHost));
    long same = 0, nonzero = 0;
    for (size_t i = 0; i < rs.size(); ++i) {
        same += std::memcmp(&rs[i], &rp[i], 4) == 0;
        nonzero += rs[i] != 0.f;
    }
    std::printf("outputs %zu, bitwise equal %ld, nonzero %ld\n", rs.size(), same, nonzero);
    CHECK(hipFree(da));
    CHECK(hipFree(db));
    CHECK(hipFree(ds));
    CHECK(hipFree(dp));
    return same == (long)rs.size() ? 0 : 3;
}
