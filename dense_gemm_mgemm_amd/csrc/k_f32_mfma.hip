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

// ---------------------------------------------------------------------------
// Fast FP32 path for the canonical NN problem with 16-byte aligned operands
// (A' K-contiguous, B' N-contiguous, lda % 4 == 0, ldb % 4 == 0, 16-byte
// aligned bases, N % 4 == 0, K % BK == 0).
//
//  * Global loads are 16 bytes per lane (4 floats); edge rows/columns of a
//    tile are read from the last valid row/4-column chunk instead of being
//    masked (their results are never stored), so the K loop has no
//    per-element conditions.
//  * A is kept in LDS as [m][k] rows of BK+4 floats, written with one
//    16-byte store per load; B as [k][n] rows of BN+4 floats.  The MFMA only
//    needs A and B to agree on which k each (lane-half, step) stands for, so
//    lane-half g at step s uses k = g*BK/2 + s: a lane then reads its BK/2
//    consecutive A values with 16-byte LDS reads, and the 20-float row
//    stride keeps those reads free of bank conflicts.
// ---------------------------------------------------------------------------
namespace mgemm {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int BM, int BN, int BK, int WM, int WN, int OCC>
__global__ __launch_bounds__(64 * WM * WN, OCC) void k_f32_fast(Problem p) {
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int AROW = BK + 4, BROW = BN + 4;            // padded LDS rows (floats)
    constexpr int ACH = BM * BK / 4, BCH = BK * BN / 4;     // 16-byte chunks per slice
    constexpr int LA = ACH / NT, LB = BCH / NT;
    constexpr int HALF = BK / 2;                            // k values per lane-half per slice
    static_assert(LA * NT == ACH && LB * NT == BCH, "tile must split evenly");
    static_assert(HALF % 4 == 0, "BK must be a multiple of 8");

    __shared__ __align__(16) float As[2][BM * AROW];
    __shared__ __align__(16) float Bs[2][BK * BROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
    int tmi, tni;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tmi, tni);
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const int mlim = (int)(p.M - m0 < BM ? p.M - m0 : BM);
    const int nlim = (int)(p.N - n0 < BN ? p.N - n0 : BN);

    const float* __restrict__ A = (const float*)p.A;
    const float* __restrict__ B = (const float*)p.B;

    // Per-thread 16-byte chunks (fixed across K slices).
    const float* a_src[LA];
    int a_dst[LA];
#pragma unroll
    for (int r = 0; r < LA; ++r) {
        const int c = tid + r * NT;
        const int mi = c / (BK / 4), kc = (c % (BK / 4)) * 4;
        const int mm = mi < mlim ? mi : mlim - 1;
        a_src[r] = A + (m0 + mm) * p.lda + kc;
        a_dst[r] = mi * AROW + kc;
    }
    const float* b_src[LB];
    int b_dst[LB];
#pragma unroll
    for (int r = 0; r < LB; ++r) {
        const int c = tid + r * NT;
        const int ki = c / (BN / 4), nc = (c % (BN / 4)) * 4;
        const int nn = nc + 4 <= nlim ? nc : nlim - 4;
        b_src[r] = B + (int64_t)ki * p.ldb + n0 + nn;
        b_dst[r] = ki * BROW + nc;
    }
    const int64_t b_kstep = (int64_t)BK * p.ldb;

    f32x4v ra[LA], rb[LB];
    auto fetch = [&](int64_t kt) {
#pragma unroll
        for (int r = 0; r < LA; ++r) ra[r] = *(const f32x4v*)(a_src[r] + kt * BK);
#pragma unroll
        for (int r = 0; r < LB; ++r) rb[r] = *(const f32x4v*)(b_src[r] + kt * b_kstep);
    };
    auto stash = [&](int slot) {
#pragma unroll
        for (int r = 0; r < LA; ++r) *(f32x4v*)(&As[slot][a_dst[r]]) = ra[r];
#pragma unroll
        for (int r = 0; r < LB; ++r) *(f32x4v*)(&Bs[slot][b_dst[r]]) = rb[r];
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    const int64_t nk = p.K / BK;
    const int lrow = lane >> 5, lcol = lane & 31;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) fetch(kt + 1);
        const float* as = &As[cur][(wm * WTM + lcol) * AROW + lrow * HALF];
        const float* bs = &Bs[cur][(lrow * HALF) * BROW + wn * WTN + lcol];
#pragma unroll
        for (int s0 = 0; s0 < HALF; s0 += 4) {
            f32x4v a4[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) a4[i] = *(const f32x4v*)(as + i * 32 * AROW + s0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float b[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j) b[j] = bs[(s0 + s) * BROW + j * 32];
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[i][s], b[j], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) stash(cur ^ 1);
        __syncthreads();
    }

    float* C = (float*)p.C;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int ni = wn * WTN + j * 32 + lcol;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int mi = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lrow + (r & 3);
                if (mi < mlim && ni < nlim) {
                    const int64_t idx = (m0 + mi) * p.ldc + n0 + ni;
                    float v = p.alpha * acc[i][j][r];
                    if (p.beta != 0.f) v = fmaf(p.beta, C[idx], v);
                    C[idx] = v;
                }
            }
        }
    }
}

// Two instantiations: a 256x256x32 tile on 16 waves (one workgroup per CU)
// for grids that fill the chip, and a 128x128x16 tile on 4 waves (two
// workgroups per CU) for smaller grids.
struct BigCfg { static constexpr int BM = 256, BN = 256, BK = 32, WM = 4, WN = 4, OCC = 1; };
struct SmallCfg { static constexpr int BM = 128, BN = 128, BK = 16, WM = 2, WN = 2, OCC = 2; };

template <class CF>
bool fast_supports(const Problem& p) {
    if (p.dtype != F32 || !p.a_kc || p.b_kc) return false;
    if (p.K <= 0 || p.K % CF::BK != 0 || p.N % 4 != 0) return false;
    if (p.lda % 4 != 0 || p.ldb % 4 != 0) return false;
    if (((uintptr_t)p.A & 15) != 0 || ((uintptr_t)p.B & 15) != 0) return false;
    const int64_t tiles = ((p.M + CF::BM - 1) / CF::BM) * ((p.N + CF::BN - 1) / CF::BN);
    return tiles > 0 && tiles <= 0x7fffffff;
}
template <class CF>
hipError_t fast_launch(const Problem& p, hipStream_t s) {
    const int64_t tiles = ((p.M + CF::BM - 1) / CF::BM) * ((p.N + CF::BN - 1) / CF::BN);
    hipLaunchKernelGGL((k_f32_fast<CF::BM, CF::BN, CF::BK, CF::WM, CF::WN, CF::OCC>),
                       dim3((unsigned)tiles), dim3(64 * CF::WM * CF::WN), 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool f32_fast_supports(const Problem& p, bool big) {
    return big ? fast_supports<BigCfg>(p) : fast_supports<SmallCfg>(p);
}

hipError_t launch_f32_fast(const Problem& p, bool big, hipStream_t s) {
    return big ? fast_launch<BigCfg>(p, s) : fast_launch<SmallCfg>(p, s);
}

}  // namespace mgemm
