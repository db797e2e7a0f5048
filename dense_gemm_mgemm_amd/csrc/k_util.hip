// Utility kernels of the host library: fill a buffer with small exact values
// (operands for the tuner's timing runs).
#include "common.h"

namespace mgemm {
namespace {

// Value i of the pattern: one of -1, -7/8, ..., 7/8, 1 (exact in FP32, FP16
// and BF16; no denormals, no overflow in any sum of the sizes timed).
__device__ __forceinline__ float pattern(int64_t i, uint32_t seed) {
    uint32_t x = (uint32_t)i * 0x9E3779B1u ^ (uint32_t)(i >> 32) * 0x85EBCA77u ^ seed;
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    x ^= x >> 12;
    return (float)((int)(x % 17u) - 8) * 0.125f;
}

template <int DT>
__global__ __launch_bounds__(256) void k_fill(void* p, int64_t n, uint32_t seed) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float v = pattern(i, seed);
        if constexpr (DT == F32) ((float*)p)[i] = v;
        else if constexpr (DT == F16) ((uint16_t*)p)[i] = f32_to_f16_bits(v);
        else ((uint16_t*)p)[i] = f32_to_bf16_bits(v);
    }
}

}  // namespace

hipError_t launch_fill_pattern(void* p, int64_t n, int dtype, uint32_t seed, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (dtype == F32) hipLaunchKernelGGL(k_fill<F32>, dim3((unsigned)blocks), dim3(256), 0, s, p, n, seed);
    else if (dtype == F16) hipLaunchKernelGGL(k_fill<F16>, dim3((unsigned)blocks), dim3(256), 0, s, p, n, seed);
    else hipLaunchKernelGGL(k_fill<BF16>, dim3((unsigned)blocks), dim3(256), 0, s, p, n, seed);
    return hipGetLastError();
}

}  // namespace mgemm
