// Peak probes of one MI355X: the sustained rate of the two matrix instructions the DSA kernels
// are built on and of streaming HBM reads, measured on the device itself (its clock under
// load, not the datasheet's).  They give the benchmark a second denominator beside the
// published peaks; they are not part of the attention path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_peak.h"

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;  // two waves per SIMD
constexpr int kChains = 8;     // independent accumulators per wave

// kChains independent chains of v_mfma_f32_32x32x16_bf16 per wave (32,768 FLOP each).
__global__ __launch_bounds__(kThreads) void peak_bf16_kernel(int iters, float* sink) {
    const int lane = threadIdx.x & 63;
    v8bf a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1.0f + 0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.5f - 0.001f * (float)(lane + i));
    }
    v16f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = (v16f){};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][lane & 15];
    if (s == 12345.f) sink[blockIdx.x] = s;  // keeps the chains alive; never taken for these inputs
}

// kChains independent chains of v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3, unit scales) per wave
// (65,536 FLOP each).
__global__ __launch_bounds__(kThreads) void peak_fp8_kernel(int iters, float* sink) {
    const int lane = threadIdx.x & 63;
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x38383838 + (lane & 3);  // e4m3 codes near 1.0
        b[i] = 0x30303030 + (i & 3);     // near 0.5
    }
    v4f acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = (v4f){};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][lane & 3];
    if (s == 12345.f) sink[blockIdx.x] = s;
}

// Streaming read of n16 16-byte words, grid-stride, four loads in flight per lane.
__global__ __launch_bounds__(256) void peak_read_kernel(const v4i* __restrict__ src, int64_t n16, float* sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4i x0 = __builtin_nontemporal_load(src + i);
        const v4i x1 = __builtin_nontemporal_load(src + i + stride);
        const v4i x2 = __builtin_nontemporal_load(src + i + 2 * stride);
        const v4i x3 = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= x0.x ^ x1.y ^ x2.z ^ x3.w;
    }
    for (; i < n16; i += stride) acc ^= src[i].x;
    if (acc == 0x7badf00d) sink[blockIdx.x] = (float)acc;
}

int n_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

}  // namespace

extern "C" {

int dsa_peak_mfma_bf16(int iters, float* sink, hipStream_t stream, double* flops) {
    if (iters < 1 || sink == nullptr || flops == nullptr) return 1;
    const int grid = 4 * n_cus();
    hipLaunchKernelGGL(peak_bf16_kernel, dim3(grid), dim3(kThreads), 0, stream, iters, sink);
    *flops = (double)grid * (kThreads / 64) * (double)iters * kChains * 32768.0;
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int dsa_peak_mfma_fp8(int iters, float* sink, hipStream_t stream, double* flops) {
    if (iters < 1 || sink == nullptr || flops == nullptr) return 1;
    const int grid = 4 * n_cus();
    hipLaunchKernelGGL(peak_fp8_kernel, dim3(grid), dim3(kThreads), 0, stream, iters, sink);
    *flops = (double)grid * (kThreads / 64) * (double)iters * kChains * 65536.0;
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int dsa_peak_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
    if (src == nullptr || sink == nullptr || ((uintptr_t)src & 15u) != 0 || bytes < 16) return 1;
    const int grid = 16 * n_cus();
    hipLaunchKernelGGL(peak_read_kernel, dim3(grid), dim3(256), 0, stream, (const v4i*)src,
                       (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
