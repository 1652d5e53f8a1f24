// probes.hip -- measurement kernels (declared in include/mesa_probe.h).
//
// Known-work kernels for measuring the attainable MFMA rate and HBM copy
// bandwidth of the GPU the library runs on.  Each MFMA chain accumulates into
// its own registers (accumulator input == output).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "../../include/mesa_probe.h"
#include "mesa_device.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void mfma_f32_probe(int iters, float* __restrict__ sink) {
    mesa::f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mesa::f32x4{0.f, 0.f, 0.f, 0.f};
    const float a = 1e-3f * (threadIdx.x & 15), b = 1.0f + 1e-4f * (threadIdx.x >> 4);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mesa::mfma4(a, b, acc[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_bf16_probe(int iters, float* __restrict__ sink) {
    mesa::f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mesa::f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1e-3f * ((threadIdx.x + e) & 15));
        b[e] = (__bf16)(1.0f);
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy_probe(const mesa::f32x4* __restrict__ src, mesa::f32x4* __restrict__ dst,
                                                  size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        __builtin_nontemporal_store(src[i], dst + i);
}

mesa_status launched(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return MESA_ERR_HIP;
    }
    return MESA_OK;
}

}  // namespace

extern "C" {

mesa_status mesa_probe_mfma_f32(int n_workgroups, int iters, float* sink, void* stream) {
    if (n_workgroups <= 0 || iters <= 0 || !sink) return MESA_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(mfma_f32_probe, dim3(n_workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       sink);
    return launched("mfma_f32_probe");
}

mesa_status mesa_probe_mfma_bf16(int n_workgroups, int iters, float* sink, void* stream) {
    if (n_workgroups <= 0 || iters <= 0 || !sink) return MESA_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(mfma_bf16_probe, dim3(n_workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       sink);
    return launched("mfma_bf16_probe");
}

mesa_status mesa_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) % 16) != 0 ||
        (reinterpret_cast<uintptr_t>(dst) % 16) != 0)
        return MESA_ERR_INVALID_ARGUMENT;
    const size_t n = bytes / 16;
    hipLaunchKernelGGL(copy_probe, dim3(1024), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const mesa::f32x4*>(src), static_cast<mesa::f32x4*>(dst), n);
    return launched("copy_probe");
}

}  // extern "C"
