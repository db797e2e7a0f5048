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
    with_epilogue(p.epilogue, [&](auto E) {
        constexpr int EPI = decltype(E)::value;
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
                        C[idx] = epilogue_op<F32, EPI>(v);
                    }
                }
            }
        }
    });
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
// Fast FP32 path for the canonical NN problem (A' K-contiguous, B'
// N-contiguous), in two forms:
//   * k_f32_fast<..., 4, 4>: 16-byte aligned operands (lda % 4 == 0,
//     ldb % 4 == 0, 16-byte aligned bases, N % 4 == 0) and K % BK == 0;
//   * the same kernel with narrower global loads for operands that are not
//     16-byte aligned (VA = 1 float per A load, VB = 1 or 2 floats per B
//     load, chosen from the alignment of the bases and leading dimensions;
//     not both single floats) and any K: the last, partial K slice is
//     fetched element by element, zero beyond K.  This is the ragged row of the pages' workloads
//     (lda = 4095, ldb = 12290: A rows 4-byte and B rows 8-byte aligned).
//
//  * Edge rows/columns of a tile are read from the last valid row / column
//    chunk instead of being masked (their results are never stored), so the
//    full K slices have no per-element conditions.
//  * A is kept in LDS as [m][k] rows of BK+4 floats; B as [k][n] rows of
//    BN+4 floats.  The MFMA only needs A and B to agree on which k each
//    (lane-half, step) stands for, so lane-half g at step s uses
//    k = g*BK/2 + s: a lane then reads its BK/2 consecutive A values with
//    16-byte LDS reads, and the 36-float row stride keeps those reads free
//    of bank conflicts.
// ---------------------------------------------------------------------------
namespace mgemm {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
template <int V> struct VecT;
template <> struct VecT<1> { typedef float T; };
template <> struct VecT<2> { typedef f32x2v T; };
template <> struct VecT<4> { typedef f32x4v T; };
template <int V>
__device__ __forceinline__ float lane_of(const typename VecT<V>::T& v, int e) {
    if constexpr (V == 1) return v;
    else return v[e];
}
template <int V>
__device__ __forceinline__ void set_lane(typename VecT<V>::T& v, int e, float x) {
    if constexpr (V == 1) v = x;
    else v[e] = x;
}

// Stream-K form (SK): the grid has one workgroup per CU, and the T = tiles * nk
// (tile, K slice) pairs, tile-major in the M-grouped tile order, are dealt out
// in equal contiguous shares: workgroup g takes pairs [g*T/G, (g+1)*T/G).  A
// share covers the end of one tile, whole tiles and the start of another; a
// whole tile is stored as usual.  Each piece of a split tile is published as
// an FP32 partial in the workspace, the contributors count their arrivals on
// the tile's counter, and the last to arrive sums the pieces in K order
// (contributor order) and stores C.  No workgroup ever waits for another.
// Shares are numbered XCD-major (the workgroups on one XCD take consecutive
// shares, hence neighbouring tiles that share A and B panels in its L2).
struct SKArgs {
    float* part;        // [G][2] partial tiles of BM*BN floats in register order
    int part_bytes;     // bytes of `part` (bounds the buffer accesses)
    unsigned* cnt;      // [tiles] arrival counters, zero between calls
};

// Operand layouts (LAY, 16-byte loads only, K % BK == 0): 0 = the canonical
// NN form (A' K-contiguous, B' N-contiguous); 1 = B' K-contiguous (a
// row-major A times a column-major B); 2 = A' M-contiguous (column-major A
// times row-major B, after the transpose identity).  Forms 1 and 2 load four
// consecutive k of one column of B' (four consecutive m of one column of A')
// and write them to the same [k][n] ([m][k]) LDS rows as form 0, one float at
// a time; the MFMA loop is the same.
template <int BM, int BN, int BK, int WM, int WN, int OCC, int VA, int VB, bool TAIL, bool SK,
          int LAY = 0>
__global__ __launch_bounds__(64 * WM * WN, OCC) void k_f32_fast(Problem p, SKArgs sk) {
    typedef typename VecT<VA>::T TA;
    typedef typename VecT<VB>::T TB;
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int AROW = BK + 4, BROW = BN + 4;            // padded LDS rows (floats)
    constexpr int ACH = BM * BK / VA, BCH = BK * BN / VB;   // loads per slice
    constexpr int LA = ACH / NT, LB = BCH / NT;
    constexpr int HALF = BK / 2;                            // k values per lane-half per slice
    static_assert(LA * NT == ACH && LB * NT == BCH, "tile must split evenly");
    static_assert(HALF % 4 == 0, "BK must be a multiple of 8");

    __shared__ __align__(16) float As[2][BM * AROW];
    __shared__ __align__(16) float Bs[2][BK * BROW];
    __shared__ int last_arrival;

    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
    const int64_t nfull = p.K / BK, nk = (p.K + BK - 1) / BK;

    const float* __restrict__ A = (const float*)p.A;
    const float* __restrict__ B = (const float*)p.B;

    // Load positions: load r of a thread covers A row a_mi0 + r*A_RS (columns
    // a_kc..a_kc+VA-1 of the slice) and B row b_ki0 + r*B_RS (columns
    // b_nc..b_nc+VB-1).  Only these few integers stay live across the K loop.
    constexpr int AK = BK / VA, A_RS = NT / AK;
    constexpr int BNV = BN / VB, B_RS = NT / BNV;
    static_assert(NT % AK == 0 && NT % BNV == 0, "loads must tile the slice");
    static_assert(LAY == 0 || (VA == 4 && VB == 4 && !TAIL && !SK), "layout forms are 16-byte only");
    // Form 1: B' column n = b_nj + r*B_NRS, k = b_k4..b_k4+3 of the slice.
    // Form 2: sixteen lanes cover 64 consecutive m of one K row of A' (256
    // contiguous bytes); load r of thread t is unit U = t/16 + r*NT/16, K row
    // U % BK, m = 64*(U / BK) + 4*(t % 16) .. +3.  In LDS element (m, k) sits
    // at column k ^ 4*((m >> 3) & 7) of row m: aligned groups of four k stay
    // together (the MFMA loop reads them as one 16-byte read, of eight lanes
    // with the same m >> 3: still conflict-free), and the scattered writes of
    // a wave spread over the banks (at most two lanes per bank instead of 32).
    constexpr int BKV = BK / 4, B_NRS = NT / BKV;
    static_assert(LAY != 1 || (NT % BKV == 0 && LB * B_NRS == BN), "form 1 must tile the slice");
    static_assert(LAY != 2 || ((NT / 16) * LA == BK * (BM / 64) && BK == 32),
                  "form 2 must tile the slice");

    f32x16 acc[TM][TN];
    // Thread-chunk c of the accumulators: 4 consecutive values of one MFMA
    // block (the unit of the partial exchange).
    constexpr int NCH = TM * TN * 4;
    auto chunk = [&](int c) -> f32x4 {
        const f32x16& v = acc[c / (TN * 4)][(c / 4) % TN];
        const int e = 4 * (c % 4);
        return f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
    };
    auto set_chunk = [&](int c, f32x4 x) {
        f32x16& v = acc[c / (TN * 4)][(c / 4) % TN];
        const int e = 4 * (c % 4);
        v[e] = x[0]; v[e + 1] = x[1]; v[e + 2] = x[2]; v[e + 3] = x[3];
    };

    // Slices [k0, k1) of tile (tmi, tni) into acc; if they are all of K, the
    // epilogue stores C, otherwise (stream-K only) the piece is exchanged.
    // Everything derived from the thread id is formed here, from `tid` as
    // passed in: the stream-K loop passes it through an empty asm on every
    // tile, so that these values are not hoisted out of that loop and kept
    // live (with the accumulators) across it.
    auto tile_pass = [&](int tid, int tmi, int tni, int64_t k0, int64_t k1, int64_t t, int64_t g,
                         int64_t T, int64_t G) {
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / WN, wn = wave % WN;
        const int a_mi0 = tid / AK, a_kc = (tid % AK) * VA;
        const int b_ki0 = tid / BNV, b_nc = (tid % BNV) * VB;
        const int lrow = lane >> 5, lcol = lane & 31;
        const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
        const int mlim = (int)(p.M - m0 < BM ? p.M - m0 : BM);
        const int nlim = (int)(p.N - n0 < BN ? p.N - n0 : BN);
        const int b_nn = b_nc + VB <= nlim ? b_nc : nlim - VB;
        const float* a_base = A + m0 * p.lda + a_kc;
        const float* b_base = B + (int64_t)b_ki0 * p.ldb + n0 + b_nn;
        auto a_ptr = [&](int r) {
            const int mi = a_mi0 + r * A_RS;
            return a_base + (int64_t)(mi < mlim ? mi : mlim - 1) * p.lda;
        };
        auto b_ptr = [&](int r) { return b_base + (int64_t)(r * B_RS) * p.ldb; };

        TA ra[LA];
        TB rb[LB];
        // With 16-byte loads on both operands the per-load pointers are
        // computed once (they fit in the registers of a 16-wave workgroup and
        // save the address arithmetic in the loop); with narrower loads there
        // are too many, and the slice bases pass through an empty asm so that
        // the compiler forms each load address here instead of keeping LA + LB
        // loop-invariant 64-bit pointers live across the K loop.
        constexpr bool WIDE = VA == 4 && VB == 4;
        const float* a_src[WIDE ? LA : 1];
        const float* b_src[WIDE ? LB : 1];
        const int b_nj = tid / BKV, b_k4 = (tid % BKV) * 4;
        auto amc_k = [&](int r) { return ((tid >> 4) + r * (NT / 16)) % BK; };
        auto amc_m = [&](int r) { return 64 * (((tid >> 4) + r * (NT / 16)) / BK) + 4 * (tid & 15); };
        if constexpr (WIDE) {
            if constexpr (LAY == 2) {
                // Columns past M read the last valid 4-float chunk (M % 4 == 0).
#pragma unroll
                for (int r = 0; r < LA; ++r) {
                    const int m = amc_m(r), mm = m + 4 <= mlim ? m : mlim - 4;
                    a_src[r] = A + (int64_t)amc_k(r) * p.lda + m0 + mm;
                }
            } else {
#pragma unroll
                for (int r = 0; r < LA; ++r) a_src[r] = a_ptr(r);
            }
            if constexpr (LAY == 1) {
                // Columns past N read the last valid column.
#pragma unroll
                for (int r = 0; r < LB; ++r) {
                    const int nj = b_nj + r * B_NRS;
                    b_src[r] = B + (n0 + (nj < nlim ? nj : nlim - 1)) * p.ldb + b_k4;
                }
            } else {
#pragma unroll
                for (int r = 0; r < LB; ++r) b_src[r] = b_ptr(r);
            }
        }
        const int64_t a_step = LAY == 2 ? (int64_t)BK * p.lda : BK;
        const int64_t b_step = LAY == 1 ? (int64_t)BK : (int64_t)BK * p.ldb;
        auto fetch = [&](int64_t kt) {
            if constexpr (WIDE) {
#pragma unroll
                for (int r = 0; r < LA; ++r) ra[r] = *(const TA*)(a_src[r] + kt * a_step);
#pragma unroll
                for (int r = 0; r < LB; ++r) rb[r] = *(const TB*)(b_src[r] + kt * b_step);
            } else {
                const float* ab = a_base + kt * BK;
                const float* bb = b_base + kt * BK * p.ldb;
                asm volatile("" : "+v"(ab), "+v"(bb));
#pragma unroll
                for (int r = 0; r < LA; ++r) {
                    const int mi = a_mi0 + r * A_RS;
                    ra[r] = *(const TA*)(ab + (int64_t)(mi < mlim ? mi : mlim - 1) * p.lda);
                }
#pragma unroll
                for (int r = 0; r < LB; ++r) rb[r] = *(const TB*)(bb + (int64_t)(r * B_RS) * p.ldb);
            }
        };
        // The partial last slice: element by element, zero where k >= K (the
        // address is clamped to k = K-1 so that nothing past the operands is read).
        auto fetch_tail = [&](int64_t kt) {
            const int64_t kb = kt * BK;
#pragma unroll
            for (int r = 0; r < LA; ++r)
#pragma unroll
                for (int e = 0; e < VA; ++e) {
                    const int64_t k = kb + a_kc + e;
                    const float x = a_ptr(r)[(k < p.K ? k : p.K - 1) - a_kc];
                    set_lane<VA>(ra[r], e, k < p.K ? x : 0.f);
                }
#pragma unroll
            for (int r = 0; r < LB; ++r) {
                const int64_t k = kb + b_ki0 + r * B_RS;
                const float* row = b_base + ((k < p.K ? k : p.K - 1) - b_ki0) * p.ldb;
#pragma unroll
                for (int e = 0; e < VB; ++e) set_lane<VB>(rb[r], e, k < p.K ? row[e] : 0.f);
            }
        };
        auto stash = [&](int slot) {
            if constexpr (LAY == 2) {
#pragma unroll
                for (int r = 0; r < LA; ++r) {
                    const int m = amc_m(r), kk = amc_k(r) ^ (4 * ((m >> 3) & 7));
#pragma unroll
                    for (int e = 0; e < 4; ++e) As[slot][(m + e) * AROW + kk] = lane_of<VA>(ra[r], e);
                }
            } else {
#pragma unroll
                for (int r = 0; r < LA; ++r) *(TA*)(&As[slot][(a_mi0 + r * A_RS) * AROW + a_kc]) = ra[r];
            }
            if constexpr (LAY == 1) {
#pragma unroll
                for (int r = 0; r < LB; ++r)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Bs[slot][(b_k4 + e) * BROW + b_nj + r * B_NRS] = lane_of<VB>(rb[r], e);
            } else {
#pragma unroll
                for (int r = 0; r < LB; ++r) *(TB*)(&Bs[slot][(b_ki0 + r * B_RS) * BROW + b_nc]) = rb[r];
            }
        };
        auto load = [&](int64_t kt) {
            if constexpr (TAIL) {
                if (kt < nfull) fetch(kt);
                else fetch_tail(kt);
            } else {
                fetch(kt);          // K % BK == 0 (host-checked)
            }
        };

#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

        load(k0);
        stash(0);
        __syncthreads();
        for (int64_t kt = k0; kt < k1; ++kt) {
            const int cur = (int)((kt - k0) & 1);
            if (kt + 1 < k1) load(kt + 1);
            const float* as = &As[cur][(wm * WTM + lcol) * AROW + (LAY == 2 ? 0 : lrow * HALF)];
            const float* bs = &Bs[cur][(lrow * HALF) * BROW + wn * WTN + lcol];
#pragma unroll
            for (int s0 = 0; s0 < HALF; s0 += 4) {
                f32x4v a4[TM];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if constexpr (LAY == 2) {
                        // Row m = wm*WTM + lcol + 32i: its swizzle 4*((m >> 3) & 7).
                        const int sw = 4 * ((((wm * WTM + lcol) >> 3) + 4 * i) & 7);
                        a4[i] = *(const f32x4v*)(as + i * 32 * AROW + ((lrow * HALF + s0) ^ sw));
                    } else {
                        a4[i] = *(const f32x4v*)(as + i * 32 * AROW + s0);
                    }
                }
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
            if (kt + 1 < k1) stash(cur ^ 1);
            __syncthreads();
        }

        if constexpr (SK) {
            if (k0 != 0 || k1 != nk) {
                // Owner of pair x: the largest g with g*T/G <= x.
                auto owner = [&](int64_t x) { return ((x + 1) * G - 1) / T; };
                const int64_t first = owner(t * nk), last = owner((t + 1) * nk - 1);
                const int nc = (int)(last - first + 1);
                // A contributor's piece is the end of its share (slot 1) if its
                // share began before this tile, else the start (slot 0).
                auto slot_base = [&](int64_t gg) {
                    const int64_t sl = gg * T / G < t * nk ? 1 : 0;
                    return (unsigned)((gg * 2 + sl) * (int64_t)(BM * BN * 4));
                };
                const __amdgpu_buffer_rsrc_t ws =
                    __builtin_amdgcn_make_buffer_rsrc(sk.part, 0, sk.part_bytes, 0x00020000);
                const unsigned mine = slot_base(g) + (unsigned)tid * 16u;
#pragma unroll
                for (int c = 0; c < NCH; ++c) store_coherent(ws, mine + (unsigned)(c * NT * 16), chunk(c));
                __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): stores done
                __syncthreads();
                if (tid == 0) {
                    const unsigned old = __hip_atomic_fetch_add(sk.cnt + t, 1u, __ATOMIC_RELAXED,
                                                                __HIP_MEMORY_SCOPE_AGENT);
                    last_arrival = old == (unsigned)(nc - 1);
                }
                __syncthreads();
                if (!last_arrival) return;
                if (tid == 0) sk.cnt[t] = 0u;
                // Sum the pieces in contributor (= K) order, all of them
                // (this one's too) read back from the workspace, GRP chunks per
                // round with their loads in flight.
                constexpr int GRP = 8;
#pragma unroll
                for (int c0 = 0; c0 < NCH; c0 += GRP) {
                    f32x4 tot[GRP];
                    const unsigned b0 = slot_base(first) + (unsigned)tid * 16u;
#pragma unroll
                    for (int q = 0; q < GRP; ++q) tot[q] = load_coherent(ws, b0 + (unsigned)((c0 + q) * NT * 16));
                    for (int cc = 1; cc < nc; ++cc) {
                        const unsigned base = slot_base(first + cc) + (unsigned)tid * 16u;
                        f32x4 v[GRP];
#pragma unroll
                        for (int q = 0; q < GRP; ++q) v[q] = load_coherent(ws, base + (unsigned)((c0 + q) * NT * 16));
#pragma unroll
                        for (int q = 0; q < GRP; ++q) tot[q] = tot[q] + v[q];
                    }
#pragma unroll
                    for (int q = 0; q < GRP; ++q) set_chunk(c0 + q, tot[q]);
                }
            }
        }

        float* C = (float*)p.C;
        with_epilogue(p.epilogue, [&](auto E) {
            constexpr int EPI = decltype(E)::value;
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
                            C[idx] = epilogue_op<F32, EPI>(v);
                        }
                    }
                }
            }
        });
    };

    if constexpr (!SK) {
        int tmi, tni;
        tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tmi, tni);
        tile_pass((int)threadIdx.x, tmi, tni, 0, nk, 0, 0, 1, 1);
    } else {
        const int64_t G = gridDim.x;
        const int64_t T = (int64_t)tiles_m * tiles_n * nk;
        const int64_t g = xcd_linear(blockIdx.x, (int)G);
        int64_t it = g * T / G;
        const int64_t end = (g + 1) * T / G;
        while (it < end) {
            const int64_t t = it / nk, k0 = it - t * nk;
            const int64_t k1 = nk - k0 < end - it ? nk : k0 + (end - it);
            int tmi, tni;
            tile_from_linear((int)t, tiles_m, tiles_n, 8, tmi, tni);
            int tid = (int)threadIdx.x;
            asm volatile("" : "+v"(tid));
            tile_pass(tid, tmi, tni, k0, k1, t, g, T, G);
            it += k1 - k0;
        }
    }
}

// Tile shapes: 256x256x32 on 16 waves (one workgroup per CU) for aligned
// grids that fill the chip, 128x128x16 on 4 waves (two workgroups per CU) for
// smaller aligned grids, and 256x256x32 on 8 waves of 128x64 for the
// unaligned form, whose narrower loads need more staging registers than a
// 16-wave workgroup leaves a wave (128).
struct BigCfg { static constexpr int BM = 256, BN = 256, BK = 32, WM = 4, WN = 4, OCC = 1; };
struct SmallCfg { static constexpr int BM = 128, BN = 128, BK = 16, WM = 2, WN = 2, OCC = 2; };
struct UnalignedCfg { static constexpr int BM = 256, BN = 256, BK = 32, WM = 2, WN = 4, OCC = 1; };
// Stream-K tiles for short M (M <= 32, 64, 128): 32, 64 or 128 rows by 256
// columns on 4, 8 or 8 waves, so that a few rows do not pay for 256 rows of
// MFMA work; the K shares then stream B with one workgroup per CU.
struct SkinnyCfg32 { static constexpr int BM = 32, BN = 256, BK = 32, WM = 1, WN = 4, OCC = 1; };
struct SkinnyCfg64 { static constexpr int BM = 64, BN = 256, BK = 32, WM = 2, WN = 4, OCC = 1; };
struct SkinnyCfg128 { static constexpr int BM = 128, BN = 256, BK = 32, WM = 2, WN = 4, OCC = 1; };

// Operand form of the 16-byte kernels (the LAY parameter), -1 if none.
int fast_layout(const Problem& p) {
    if (p.a_kc && !p.b_kc) return 0;
    if (p.a_kc && p.b_kc) return 1;
    if (!p.a_kc && !p.b_kc) return 2;
    return -1;
}
template <class CF>
bool fast_supports(const Problem& p, bool any_layout) {
    if (p.dtype != F32) return false;
    const int lay = fast_layout(p);
    if (lay < 0 || (lay != 0 && !any_layout)) return false;
    if (p.K <= 0 || p.K % CF::BK != 0) return false;
    if (lay != 1 && p.N % 4 != 0) return false;      // B' rows read as 4-float chunks
    if (lay == 2 && p.M % 4 != 0) return false;      // A' columns read as 4-float chunks
    if (p.lda % 4 != 0 || p.ldb % 4 != 0) return false;
    if (((uintptr_t)p.A & 15) != 0 || ((uintptr_t)p.B & 15) != 0) return false;
    const int64_t tiles = ((p.M + CF::BM - 1) / CF::BM) * ((p.N + CF::BN - 1) / CF::BN);
    return tiles > 0 && tiles <= 0x7fffffff;
}
template <class CF, int VA, int VB, bool TAIL, int LAY = 0>
hipError_t fast_launch(const Problem& p, hipStream_t s) {
    const int64_t tiles = ((p.M + CF::BM - 1) / CF::BM) * ((p.N + CF::BN - 1) / CF::BN);
    hipLaunchKernelGGL((k_f32_fast<CF::BM, CF::BN, CF::BK, CF::WM, CF::WN, CF::OCC, VA, VB, TAIL, false, LAY>),
                       dim3((unsigned)tiles), dim3(64 * CF::WM * CF::WN), 0, s, p, SKArgs{});
    return hipGetLastError();
}
// Stream-K: one workgroup per CU (the 256x256 tiles hold one per CU).
template <class CF, int VA, int VB, bool TAIL>
hipError_t sk_launch(const Problem& p, const Workspace& ws, hipStream_t s) {
    // At most one workgroup per (tile, slice) pair, so that every share is
    // non-empty and the contributors to a tile are consecutive workgroups.
    const int64_t tiles = ((p.M + CF::BM - 1) / CF::BM) * ((p.N + CF::BN - 1) / CF::BN);
    const int64_t pairs = tiles * ((p.K + CF::BK - 1) / CF::BK);
    const int64_t cus = p.num_cu > 0 ? p.num_cu : 256;
    const int G = (int)(pairs < cus ? pairs : cus);
    SKArgs a{(float*)ws.part, (int)(ws.part_bytes < 0x7fffffff ? ws.part_bytes : 0x7fffffff),
             ws.counters};
    hipLaunchKernelGGL((k_f32_fast<CF::BM, CF::BN, CF::BK, CF::WM, CF::WN, CF::OCC, VA, VB, TAIL, true>),
                       dim3((unsigned)G), dim3(64 * CF::WM * CF::WN), 0, s, p, a);
    return hipGetLastError();
}
template <class CF>
bool sk_fits(const Problem& p, const Workspace& ws) {
    const int64_t G = p.num_cu > 0 ? p.num_cu : 256;
    const int64_t tiles = ((p.M + CF::BM - 1) / CF::BM) * ((p.N + CF::BN - 1) / CF::BN);
    return ws.part != nullptr && ws.counters != nullptr && tiles <= ws.ncounters &&
           G * 2 * CF::BM * CF::BN * (int64_t)sizeof(float) <= ws.part_bytes;
}

// Widest loads the operands allow: A loads of 4 floats need 16-byte aligned
// rows; B loads of VB floats need VB*4-byte aligned rows and N % VB == 0 (the
// last chunk of a row is shifted inside the row, never past it).
int unaligned_va(const Problem& p) {
    return (p.lda % 4 == 0 && ((uintptr_t)p.A & 15) == 0) ? 4 : 1;
}
int unaligned_vb(const Problem& p) {
    if (p.ldb % 4 == 0 && ((uintptr_t)p.B & 15) == 0 && p.N % 4 == 0) return 4;
    if (p.ldb % 2 == 0 && ((uintptr_t)p.B & 7) == 0 && p.N % 2 == 0) return 2;
    return 1;
}

}  // namespace

bool f32_fast_supports(const Problem& p, bool big) {
    return big ? fast_supports<BigCfg>(p, true) : fast_supports<SmallCfg>(p, false);
}

hipError_t launch_f32_fast(const Problem& p, bool big, hipStream_t s) {
    if (!big) return fast_launch<SmallCfg, 4, 4, false>(p, s);
    switch (fast_layout(p)) {
    case 1: return fast_launch<BigCfg, 4, 4, false, 1>(p, s);
    case 2: return fast_launch<BigCfg, 4, 4, false, 2>(p, s);
    default: return fast_launch<BigCfg, 4, 4, false>(p, s);
    }
}

bool f32_unaligned_supports(const Problem& p) {
    if (p.dtype != F32 || !p.a_kc || p.b_kc || p.K <= 0) return false;
    if (((uintptr_t)p.A & 3) != 0 || ((uintptr_t)p.B & 3) != 0) return false;
    // Single-float loads on both operands need more registers than a wave
    // has here; that case stays with k_f32_mfma.
    if (unaligned_va(p) == 1 && unaligned_vb(p) == 1) return false;
    const int64_t tiles = ((p.M + UnalignedCfg::BM - 1) / UnalignedCfg::BM) *
                          ((p.N + UnalignedCfg::BN - 1) / UnalignedCfg::BN);
    return tiles > 0 && tiles <= 0x7fffffff;
}

hipError_t launch_f32_unaligned(const Problem& p, hipStream_t s) {
    const int va = unaligned_va(p), vb = unaligned_vb(p);
    using U = UnalignedCfg;
    if (va == 4) {
        if (vb == 4) return fast_launch<U, 4, 4, true>(p, s);
        if (vb == 2) return fast_launch<U, 4, 2, true>(p, s);
        return fast_launch<U, 4, 1, true>(p, s);
    }
    if (vb == 4) return fast_launch<U, 1, 4, true>(p, s);
    return fast_launch<U, 1, 2, true>(p, s);           // (1, 1) is declined by the supports check
}

bool f32_sk_fits(const Problem& p, const Workspace& ws) {
    if (p.M <= 32) return sk_fits<SkinnyCfg32>(p, ws);
    if (p.M <= 64) return sk_fits<SkinnyCfg64>(p, ws);
    if (p.M <= 128) return sk_fits<SkinnyCfg128>(p, ws);
    return sk_fits<UnalignedCfg>(p, ws);
}

template <class U>
hipError_t sk_launch_loads(const Problem& p, const Workspace& ws, hipStream_t s) {
    const int va = unaligned_va(p), vb = unaligned_vb(p);
    if (va == 4) {
        if (vb == 4) return sk_launch<U, 4, 4, true>(p, ws, s);
        if (vb == 2) return sk_launch<U, 4, 2, true>(p, ws, s);
        return sk_launch<U, 4, 1, true>(p, ws, s);
    }
    if (vb == 4) return sk_launch<U, 1, 4, true>(p, ws, s);
    return sk_launch<U, 1, 2, true>(p, ws, s);
}

hipError_t launch_f32_sk(const Problem& p, const Workspace& ws, hipStream_t s) {
    if (p.M <= 32) return sk_launch_loads<SkinnyCfg32>(p, ws, s);
    if (p.M <= 64) return sk_launch_loads<SkinnyCfg64>(p, ws, s);
    if (p.M <= 128) return sk_launch_loads<SkinnyCfg128>(p, ws, s);
    return sk_launch_loads<UnalignedCfg>(p, ws, s);
}

}  // namespace mgemm
