// mgemm_run_noalloc: the mgemm_run_variant path with its scratch memory (the
// FP32 partial results and arrival counters of the split-K and stream-K
// forms) in a static device array of this file instead of a handle's
// workspace, so that a call allocates nothing.  See include/mgemm.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>

#include "host.h"

namespace {

constexpr int64_t COUNTER_BYTES = (int64_t)MGEMM_NOALLOC_COUNTERS * 4;
constexpr int64_t PART_BYTES = (int64_t)MGEMM_NOALLOC_SCRATCH_BYTES;
static_assert(COUNTER_BYTES % 256 == 0, "partials start 256-byte aligned");

// Counters first, then the partials.  In host code `scratch` is only a
// stand-in for the symbol: its device address is looked up per device.
static __device__ __align__(256) unsigned char scratch[COUNTER_BYTES + PART_BYTES];

__global__ void k_zero_counters(unsigned* c, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) c[i] = 0u;
}

struct DeviceScratch {
    bool ready = false;
    int num_cu = 0;
    unsigned char* ptr = nullptr;     // device address of `scratch` on this device
};

std::mutex g_lock;
DeviceScratch g_dev[mgemm::MAX_DEVICES];

// Set-up of the current device on its first call: gfx950 check, CU count,
// the array's device address, and a kernel on `stream` that zeroes the
// counters.  Returns MGEMM_SUCCESS with *out filled.
mgemm_status_t device_scratch(hipStream_t stream, DeviceScratch* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MGEMM_ERR_HIP;
    if (dev < 0 || dev >= mgemm::MAX_DEVICES) return MGEMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> g(g_lock);
    DeviceScratch& d = g_dev[dev];
    if (!d.ready) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MGEMM_ERR_HIP;
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MGEMM_ERR_UNSUPPORTED;
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return MGEMM_ERR_HIP;
        const int n = (int)MGEMM_NOALLOC_COUNTERS;
        hipLaunchKernelGGL(k_zero_counters, dim3((n + 255) / 256), dim3(256), 0, stream,
                           (unsigned*)ptr, n);
        if (hipGetLastError() != hipSuccess) return MGEMM_ERR_HIP;
        d.num_cu = prop.multiProcessorCount;
        d.ptr = (unsigned char*)ptr;
        d.ready = true;
    }
    *out = d;
    return MGEMM_SUCCESS;
}

}  // namespace

extern "C" mgemm_status_t mgemm_run_noalloc(const mgemm_variant_t* v, mgemm_layout_t layoutA,
                                            mgemm_layout_t layoutB, int64_t M, int64_t N,
                                            int64_t K, float alpha, const void* A, int64_t lda,
                                            const void* B, int64_t ldb, float beta, void* C,
                                            int64_t ldc, mgemm_dtype_t dtype,
                                            mgemm_epilogue_t epilogue, hipStream_t stream) {
    DeviceScratch d;
    mgemm_status_t st = device_scratch(stream, &d);
    if (st != MGEMM_SUCCESS) return st;
    const mgemm::Workspace ws{d.ptr + COUNTER_BYTES, PART_BYTES, (unsigned*)d.ptr,
                              (int64_t)MGEMM_NOALLOC_COUNTERS};
    const mgemm_kernel_t k = v ? (mgemm_kernel_t)v->kernel : MGEMM_KERNEL_AUTO;
    const int ks = v ? v->ksplit : 0;
    return mgemm_host::run_core(d.num_cu, ws, nullptr, k, ks, layoutA, layoutB, M, N, K, alpha, A,
                                lda, B, ldb, beta, C, ldc, dtype, epilogue, stream,
                                MGEMM_ERR_SCRATCH);
}
