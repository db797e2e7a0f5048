// General GEMM kernel: any dtype, any operand order, any alignment and any
// ragged M/N/K.  It is the correctness anchor and the fallback branch.
//
// Structure: each 256-thread workgroup owns a 64x64 output tile, stages
// 64x16 slices of A' and 16x64 slices of B' through LDS as FP32 (zero-filled
// past the matrix edge, the masked last tile of "Chapter 5: Operators and
// Runtime", section 5.4.2), and each thread accumulates a 4x4 register block
// in FP32 (the register blocking of the SGEMM report's kernels K5/K6 and of
// the zwxr.cn post, section 3.4).  Scalar loads only, so no alignment rule
// applies; the epilogue applies alpha/beta and rounds once to the output type.
#include "common.h"

namespace mgemm {
namespace {

constexpr int GBM = 64, GBN = 64, GBK = 16, GNT = 256;

template <int DT>
__global__ __launch_bounds__(GNT) void k_general(Problem p) {
    using E = Elem<DT>;
    using T = typename E::T;
    __shared__ float As[GBK][GBM + 4];
    __shared__ float Bs[GBK][GBN + 4];

    const int tid = threadIdx.x;
    const int tiles_m = (int)((p.M + GBM - 1) / GBM), tiles_n = (int)((p.N + GBN - 1) / GBN);
    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tm, tn);
    const int64_t m0 = (int64_t)tm * GBM, n0 = (int64_t)tn * GBN;
    const T* A = (const T*)p.A;
    const T* B = (const T*)p.B;

    float acc[4][4] = {};
    const int ty = tid / 16, tx = tid % 16;

    for (int64_t k0 = 0; k0 < p.K; k0 += GBK) {
        // 64x16 = 1024 elements of each operand, 4 per thread; consecutive
        // threads walk the operand's contiguous direction.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int e = tid + r * GNT;
            int mi, ki;
            if (p.a_kc) { mi = e / GBK; ki = e % GBK; } else { ki = e / GBM; mi = e % GBM; }
            int64_t m = m0 + mi, k = k0 + ki;
            float v = 0.f;
            if (m < p.M && k < p.K) v = E::load(A, p.a_kc ? m * p.lda + k : k * p.lda + m);
            As[ki][mi] = v;
            int ni;
            if (p.b_kc) { ni = e / GBK; ki = e % GBK; } else { ki = e / GBN; ni = e % GBN; }
            int64_t n = n0 + ni;
            k = k0 + ki;
            float w = 0.f;
            if (n < p.N && k < p.K) w = E::load(B, p.b_kc ? n * p.ldb + k : k * p.ldb + n);
            Bs[ki][ni] = w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GBK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }

    T* C = (T*)p.C;
    with_epilogue(p.epilogue, [&](auto E) {
        constexpr int EPI = decltype(E)::value;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int64_t m = m0 + ty * 4 + i;
            if (m >= p.M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int64_t n = n0 + tx * 4 + j;
                if (n >= p.N) continue;
                int64_t idx = m * p.ldc + n;
                float v = p.alpha * acc[i][j];
                if (p.beta != 0.f) v = fmaf(p.beta, E::load(C, idx), v);
                E::store(C, idx, epilogue_op<DT, EPI>(v));
            }
        }
    });
}

// C = beta * C (K == 0 or alpha == 0: A and B are not read).
template <int DT>
__global__ __launch_bounds__(256) void k_scale(Problem p) {
    using E = Elem<DT>;
    using T = typename E::T;
    T* C = (T*)p.C;
    int64_t total = p.M * p.N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        int64_t m = e / p.N, n = e % p.N;
        int64_t idx = m * p.ldc + n;
        float v = p.beta != 0.f ? p.beta * E::load(C, idx) : 0.f;
        E::store(C, idx, apply_epilogue<DT>(v, p.epilogue));
    }
}

}  // namespace

hipError_t launch_general(const Problem& p, hipStream_t s) {
    int64_t tiles = ((p.M + GBM - 1) / GBM) * ((p.N + GBN - 1) / GBN);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)tiles), block(GNT);
    switch (p.dtype) {
    case F32: hipLaunchKernelGGL(k_general<F32>, grid, block, 0, s, p); break;
    case F16: hipLaunchKernelGGL(k_general<F16>, grid, block, 0, s, p); break;
    case BF16: hipLaunchKernelGGL(k_general<BF16>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_scale(const Problem& p, hipStream_t s) {
    int64_t total = p.M * p.N;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    dim3 grid((unsigned)blocks), block(256);
    switch (p.dtype) {
    case F32: hipLaunchKernelGGL(k_scale<F32>, grid, block, 0, s, p); break;
    case F16: hipLaunchKernelGGL(k_scale<F16>, grid, block, 0, s, p); break;
    case BF16: hipLaunchKernelGGL(k_scale<BF16>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mgemm
