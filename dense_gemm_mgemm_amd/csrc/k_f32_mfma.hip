// FP32 GEMM on the FP32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// gfx950 runs FP32 matrix FMA at the same 256 flop/clk/CU as packed FP32
// vector FMA, and this library is built without packed FP32 vector
// instructions, so the matrix cores are the only route to the FP32 peak.  The
// SGEMM report ("SGEMM measurements and three ledgers") climbs the same ladder
// on CUDA cores: shared-memory tiles (K3), register blocking (K5), wide loads
// (K6); here the "register block" is an MFMA accumulator.
//
// Per workgroup: a BM x BN output tile, 4 waves in a WM x WN grid, each wave a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA blocks held in accumulator
// registers.  K advances in slices of 16: a 16 x BM slice of A' and 16 x BN
// of B' are staged in LDS, K-major with the M/N index contiguous (a lane of
// the MFMA reads one element per operand, so 32 lanes read 32 consecutive
// words: no bank conflict; 4 words of padding per row keep the transposing
// writes conflict-light).  Two LDS slots alternate: while the waves compute
// on one, the next slice is fetched from global memory into registers and
// then written to the other (the two-slot pipeline of "Chapter 5: Operators
// and Runtime", section 5.3.2; the register prefetch of the MTT S4000 write-up,
// section 4).  Loads are scalar and masked, so any operand order, leading
// dimension, alignment and ragged edge is handled (the masked last tile of
// Chapter 5, section 5.4.2).
#include "common.h"

namespace mgemm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 2) void k_f32_mfma(Problem p) {
    constexpr int NT = 64 * WM * WN;
    constexpr int BK = 16, PAD = 4;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int LA = BM * BK / NT, LB = BN * BK / NT;
    static_assert(LA * NT == BM * BK && LB * NT == BN * BK, "tile must split evenly");

    __shared__ float As[2][BK][BM + PAD];
    __shared__ float Bs[2][BK][BN + PAD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
    int tm_, tn_;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tm_, tn_);
    const int64_t m0 = (int64_t)tm_ * BM, n0 = (int64_t)tn_ * BN;

    const float* __restrict__ A = (const float*)p.A;
    const float* __restrict__ B = (const float*)p.B;

    // Fixed per-thread element assignment: consecutive threads walk the
    // operand's contiguous direction so global reads coalesce.
    int64_t a_off[LA], b_off[LB];
    int a_mi[LA], a_ki[LA], b_ni[LB], b_ki[LB];
    bool a_ok[LA], b_ok[LB];
#pragma unroll
    for (int r = 0; r < LA; ++r) {
        int e = tid + r * NT;
        int mi, ki;
        if (p.a_kc) { mi = e / BK; ki = e % BK; } else { ki = e / BM; mi = e % BM; }
        a_mi[r] = mi; a_ki[r] = ki;
        int64_t m = m0 + mi;
        a_ok[r] = m < p.M;
        a_off[r] = p.a_kc ? m * p.lda + ki : (int64_t)ki * p.lda + m;
    }
#pragma unroll
    for (int r = 0; r < LB; ++r) {
        int e = tid + r * NT;
        int ni, ki;
        if (p.b_kc) { ni = e / BK; ki = e % BK; } else { ki = e / BN; ni = e % BN; }
        b_ni[r] = ni; b_ki[r] = ki;
        int64_t n = n0 + ni;
        b_ok[r] = n < p.N;
        b_off[r] = p.b_kc ? n * p.ldb + ki : (int64_t)ki * p.ldb + n;
    }
    const int64_t a_step = p.a_kc ? BK : (int64_t)BK * p.lda;
    const int64_t b_step = p.b_kc ? BK : (int64_t)BK * p.ldb;

    float ra[LA], rb[LB];
    auto fetch = [&](int64_t k0, int64_t kt) {
#pragma unroll
        for (int r = 0; r < LA; ++r)
            ra[r] = (a_ok[r] && k0 + a_ki[r] < p.K) ? A[a_off[r] + kt * a_step] : 0.f;
#pragma unroll
        for (int r = 0; r < LB; ++r)
            rb[r] = (b_ok[r] && k0 + b_ki[r] < p.K) ? B[b_off[r] + kt * b_step] : 0.f;
    };
    auto stash = [&](int slot) {
#pragma unroll
        for (int r = 0; r < LA; ++r) As[slot][a_ki[r]][a_mi[r]] = ra[r];
#pragma unroll
        for (int r = 0; r < LB; ++r) Bs[slot][b_ki[r]][b_ni[r]] = rb[r];
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    const int64_t nk = (p.K + BK - 1) / BK;
    const int lrow = lane >> 5, lcol = lane & 31;
    if (nk > 0) {
        fetch(0, 0);
        stash(0);
        __syncthreads();
    }
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) fetch((kt + 1) * BK, kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK / 2; ++kk) {
            float a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = As[cur][2 * kk + lrow][wm * WTM + i * 32 + lcol];
#pragma unroll
            for (int j = 0; j < TN; ++j) b[j] = Bs[cur][2 * kk + lrow][wn * WTN + j * 32 + lcol];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) stash(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: register r of lane l holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the block.
    float* C = (float*)p.C;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + wn * WTN + j * 32 + lcol;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lrow + (r & 3);
                if (m < p.M && n < p.N) {
                    const int64_t idx = m * p.ldc + n;
                    float v = p.alpha * acc[i][j][r];
                    if (p.beta != 0.f) v = fmaf(p.beta, C[idx], v);
                    C[idx] = v;
                }
            }
        }
    }
}

constexpr int F_BM = 128, F_BN = 128;

}  // namespace

bool f32_mfma_supports(const Problem& p) { return p.dtype == F32; }

hipError_t launch_f32_mfma(const Problem& p, hipStream_t s) {
    int64_t tiles = ((p.M + F_BM - 1) / F_BM) * ((p.N + F_BN - 1) / F_BN);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_f32_mfma<F_BM, F_BN, 2, 2>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace mgemm
