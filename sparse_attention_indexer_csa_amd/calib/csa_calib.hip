// Calibration kernels (include/csa_calib.h): a bf16 MFMA loop and streaming
// read / copy kernels, for the achievable peaks that bench.py reports beside
// the datasheet ones.
#include "csa_calib.h"

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(const u32x4 *ops, float *sink, int iters)
{
    const int l = threadIdx.x & 63;
    // two A and two B fragments per lane, from the caller's operand values
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, ops[l]);
    const bf16x8 a1 = __builtin_bit_cast(bf16x8, ops[64 + l]);
    const bf16x8 b0 = __builtin_bit_cast(bf16x8, ops[128 + l]);
    const bf16x8 b1 = __builtin_bit_cast(bf16x8, ops[192 + l]);
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c3, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s += c0[r] + c1[r] + c2[r] + c3[r];
    if (l == 0)
        sink[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = s;
}

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *src, size_t n, uint32_t *sink)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    constexpr int kIn = 8;
    for (; i + (kIn - 1) * stride < n; i += kIn * stride) {
        u32x4 v[kIn];
#pragma unroll
        for (int u = 0; u < kIn; ++u)
            v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
        for (int u = 0; u < kIn; ++u)
            acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const u32x4 v = src[i];
        acc += v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4 *src, uint4 *dst, size_t n)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

} // namespace

extern "C" {

int32_t csa_calib_mfma_bf16(const void *operands, float *sink, int32_t blocks, int32_t iters, void *stream)
{
    if (!operands || !sink || blocks <= 0 || iters < 0)
        return (int32_t)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(operands), sink, iters);
    return (int32_t)hipGetLastError();
}

int32_t csa_calib_read(const void *src, size_t bytes, uint32_t *sink, int32_t blocks, void *stream)
{
    if (!src || !sink || blocks <= 0 || bytes % 16 != 0)
        return (int32_t)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), bytes / 16, sink);
    return (int32_t)hipGetLastError();
}

int32_t csa_calib_copy(const void *src, void *dst, size_t bytes, int32_t blocks, void *stream)
{
    if (!src || !dst || blocks <= 0 || bytes % 16 != 0)
        return (int32_t)hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), bytes / 16);
    return (int32_t)hipGetLastError();
}

} // extern "C"
