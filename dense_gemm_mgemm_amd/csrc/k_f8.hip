// FP8 (E4M3FN) path for gfx950: per-row quantisation and the FP8 GEMM.
//
// Format ("Chapter 5: Operators and Runtime", section 5.4.3, Example 5-7):
// sign, 4 exponent bits (bias 7), 3 mantissa bits; largest finite value 448,
// no infinity, 0x7F/0xFF are NaN.
//
// Quantisation (Example 5-7): a row's scale comes from the largest magnitude
// of the whole row, found before any element is quantised.  Rows of up to
// 16384 16-bit (8192 FP32) elements with aligned 16-byte chunks: one workgroup
// per row holds the row in registers; otherwise one wave per row reads the
// row once for the maximum and again (from L2) to quantise.
// Element x is scaled by the row's factor, t = x * r with r = 448 / amax
// (both FP32, r correctly rounded once per row), and rounded to the nearest
// E4M3 value with ties to the even mantissa; the row's dequantisation scale
// amax / 448 is stored as FP32.  A separate kernel rather than a fused one because each output
// tile would otherwise re-read the wide input (section 5.4.4, Example 5-8:
// with 128x128 tiles 444 vs 620 MiB; with 256-wide tiles the fused form still
// reads the 16-bit input once per column block).
//
// GEMM (section 5.4.4, Example 5-8): C = alpha * sa[m] * sb[n] * sum_k
// qa[m,k] qb[n,k] + beta * C with both code matrices K-contiguous (qb holds
// the weights one output column per row).  The scales factor out of the K
// sum, so the contraction runs on v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// block scales and the row/column scales are applied in the epilogue.  The
// tile loop is the four-slot direct-to-LDS ring of k_h_dma.hip with both
// operands staged like its A: 256x256 output tiles, four waves of 128x128,
// K = 64 bytes per slice (a 64-byte row per operand row, 16 KiB per operand
// per slot), one MFMA K-step per slice, fragments read one slice ahead, the
// copies and fragment reads spread evenly between the MFMAs.  BN = 192 (four
// waves of 128x96) exists for grids that a 256-wide tile fills badly: the
// 1024x12288 FFN projection is 192 tiles of 256x256 on 256 CUs but 256 of
// 256x192.
// Restrictions of the MFMA kernel (host-checked): K >= 64 (a last partial
// slice is staged by ordinary loads with zero codes past K), lda and ldb
// multiples of 16, 16-byte aligned code buffers; k_f8_general takes the rest.
#include "f8_tiles.h"

namespace mgemm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// E4M3 encode / decode
// ---------------------------------------------------------------------------
// Nearest E4M3 code of t (ties to the even mantissa; magnitudes >= 448
// saturate to 448; NaN -> 0x7F; the sign of zero is kept).
__device__ __forceinline__ uint32_t e4m3_code(float t) {
    const uint32_t sign = (__float_as_uint(t) >> 24) & 0x80u;
    const float a = fabsf(t);
    if (!(a == a)) return 0x7Fu;
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0x1p-6f) {
        // Subnormals are multiples of 2^-9: scale exactly, round to an
        // integer 0..8 (8 is the smallest normal, code 0x08).
        return sign | (uint32_t)__builtin_rintf(a * 512.0f);
    }
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);          // round the mantissa to 3 bits, ties to even
    const uint32_t e = (b >> 23) - 127u + 7u;  // 1..15 (a < 448 cannot round past 448)
    return sign | (e << 3) | ((b >> 20) & 7u);
}

// Four codes packed little-endian into a word.  gfx950 converts FP32 pairs
// to E4M3 in hardware (v_cvt_pk_fp8_f32, round to nearest even); the inputs
// are clamped to +-448 first (infinities saturate like e4m3_code) and the
// code of a NaN is set to 0x7F afterwards.  The parity tests check every code
// against the oracle's encoder.
#ifndef MGEMM_F8_HW_CVT
#define MGEMM_F8_HW_CVT 1
#endif
__device__ __forceinline__ uint32_t e4m3_word(float a, float b, float c, float d) {
#if MGEMM_F8_HW_CVT
    auto clamp = [](float t) { return fminf(fmaxf(t, -448.0f), 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(a), clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(c), clamp(d), w, true);
    uint32_t u = (uint32_t)w;
    if (a != a) u = (u & 0xFFFFFF00u) | 0x7Fu;
    if (b != b) u = (u & 0xFFFF00FFu) | 0x7F00u;
    if (c != c) u = (u & 0xFF00FFFFu) | 0x7F0000u;
    if (d != d) u = (u & 0x00FFFFFFu) | 0x7F000000u;
    return u;
#else
    return e4m3_code(a) | (e4m3_code(b) << 8) | (e4m3_code(c) << 16) | (e4m3_code(d) << 24);
#endif
}

// Value of an E4M3 code (exact in FP32).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v;
    if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
    else if (e == 0u) v = (float)m * 0x1p-9f;
    else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------------------
// Per-row quantisation: one wave per row, four rows per workgroup.
// ---------------------------------------------------------------------------
template <int XT>
__device__ __forceinline__ float load_x(const void* x, int64_t i) {
    if constexpr (XT == F32) return ((const float*)x)[i];
    else if constexpr (XT == F16) return f16_bits_to_f32(((const uint16_t*)x)[i]);
    else return bf16_bits_to_f32(((const uint16_t*)x)[i]);
}

// Largest magnitude, NaN if either is NaN.
__device__ __forceinline__ float amax2(float a, float b) {
    return (a != a || b != b) ? __uint_as_float(0x7FC00000u) : fmaxf(a, b);
}

template <int XT, bool VEC>
__global__ __launch_bounds__(256) void k_quant_rows(int64_t M, int64_t K, const void* X, int64_t ldx,
                                                    uint8_t* Q, int64_t ldq, float* scales) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    constexpr int ES = XT == F32 ? 4 : 2;
    constexpr int V = 16 / ES;                    // elements per 16-byte load
    const unsigned char* xr = (const unsigned char*)X + row * ldx * ES;
    auto vec_at = [&](int64_t k, float (&v)[V]) {
        const i32x4 w = *(const i32x4*)(xr + k * ES);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            if constexpr (XT == F32) v[e] = __int_as_float(w[e]);
            else {
                const uint16_t h = (uint16_t)((uint32_t)w[e / 2] >> (16 * (e & 1)));
                v[e] = XT == F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
            }
        }
    };
    // Pass 1: the row's largest magnitude.
    float m = 0.0f;
    if constexpr (VEC) {
        for (int64_t k = (int64_t)lane * V; k < K; k += 64 * V) {
            float v[V];
            vec_at(k, v);
#pragma unroll
            for (int e = 0; e < V; ++e) m = amax2(m, fabsf(v[e]));
        }
    } else {
        for (int64_t k = lane; k < K; k += 64) m = amax2(m, fabsf(load_x<XT>(xr, k)));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = amax2(m, __shfl_xor(m, off, 64));
    if (lane == 0) scales[row] = m / 448.0f;
    // Pass 2: codes.  A zero row keeps its (signed) zeros.
    uint8_t* qr = Q + row * ldq;
    const float r = 448.0f / m;
    auto sc = [&](float x) { return m == 0.0f ? x : x * r; };       // scaled value
    if constexpr (VEC) {
        for (int64_t k = (int64_t)lane * V; k < K; k += 64 * V) {
            float v[V];
            vec_at(k, v);
            uint32_t w[V / 4];
#pragma unroll
            for (int g = 0; g < V / 4; ++g)
                w[g] = e4m3_word(sc(v[4 * g]), sc(v[4 * g + 1]), sc(v[4 * g + 2]), sc(v[4 * g + 3]));
            if constexpr (V == 8) *(uint2*)(qr + k) = make_uint2(w[0], w[1]);
            else *(uint32_t*)(qr + k) = w[0];
        }
    } else {
        for (int64_t k = lane; k < K; k += 64) qr[k] = (uint8_t)e4m3_code(sc(load_x<XT>(xr, k)));
    }
}

// One workgroup per row with the row held in registers: thread t loads the
// 16-byte chunks t, t + 256, ... (up to R of them, all issued at once), the
// four waves combine their maxima through LDS, and the codes are formed from
// the registers, so the row crosses HBM once and each thread waits for one
// round of loads (rows of up to 16384 16-bit or 8192 FP32 elements).
template <int XT, int R>
__global__ __launch_bounds__(256) void k_quant_rows_reg(int64_t /*M: one workgroup per row*/, int64_t K, const void* X,
                                                        int64_t ldx, uint8_t* Q, int64_t ldq,
                                                        float* scales) {
    constexpr int ES = XT == F32 ? 4 : 2;
    constexpr int V = 16 / ES;
    __shared__ float wmax[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t row = blockIdx.x;
    const int64_t chunks = K / V;
    const unsigned char* xr = (const unsigned char*)X + row * ldx * ES;
    float v[R][V];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t c = tid + 256 * i;
        if (c < chunks) {
            const i32x4 w = *(const i32x4*)(xr + c * 16);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if constexpr (XT == F32) v[i][e] = __int_as_float(w[e]);
                else {
                    const uint16_t hb = (uint16_t)((uint32_t)w[e / 2] >> (16 * (e & 1)));
                    v[i][e] = XT == F16 ? f16_bits_to_f32(hb) : bf16_bits_to_f32(hb);
                }
                m = amax2(m, fabsf(v[i][e]));
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = amax2(m, __shfl_xor(m, off, 64));
    if (lane == 0) wmax[tid >> 6] = m;
    __syncthreads();
    m = amax2(amax2(wmax[0], wmax[1]), amax2(wmax[2], wmax[3]));
    if (tid == 0) scales[row] = m / 448.0f;
    const float r = 448.0f / m;
    uint8_t* qr = Q + row * ldq;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t c = tid + 256 * i;
        if (c < chunks) {
            uint32_t w[V / 4];
#pragma unroll
            for (int g = 0; g < V / 4; ++g) {
                float t[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) t[b] = m == 0.0f ? v[i][4 * g + b] : v[i][4 * g + b] * r;
                w[g] = e4m3_word(t[0], t[1], t[2], t[3]);
            }
            if constexpr (V == 8) *(uint2*)(qr + c * V) = make_uint2(w[0], w[1]);
            else *(uint32_t*)(qr + c * V) = w[0];
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 GEMM on the matrix cores
// ---------------------------------------------------------------------------
#ifndef MGEMM_F8_SLOTS
#define MGEMM_F8_SLOTS 4
#endif
constexpr int BK = 64, NT = 256;
constexpr int SLOTS = MGEMM_F8_SLOTS, AHEAD = SLOTS - 1;   // slices in flight
constexpr int ROW = BK;                          // bytes per operand row per slice

// BMT is the tile height: 256 (the four waves laid out 2x2 hold 128 x BN/2
// each), or 128 with the 192-wide slot (64 x 96 per wave) for products whose
// 256-row grid would leave CUs idle.
template <int BN, int BMT = 256>
struct F8Cfg {
    static_assert(BN == 256 || BN == 192, "tile width");
    static_assert(BMT == 256 || (BMT == 128 && BN == 192), "tile height");
    static constexpr int A_BYTES = BMT * ROW;    // 16 or 8 KiB of A per slot
    static constexpr int A_COPIES = BMT / 64;    // 1 KiB copies of A per wave per slice
    static constexpr int WROWS = BMT / 2;        // rows per wave
    static constexpr int TM = WROWS / 32;        // 32-row blocks per wave
    static constexpr int B_COPIES = BN / 64;     // 1 KiB copies of B per wave per slice
    static constexpr int COPIES = A_COPIES + B_COPIES;
    static constexpr int SLOT_BYTES = A_BYTES + BN * ROW;
    static constexpr int TN = BN / 64;           // 32-column blocks per wave (BN/2 columns)
    static constexpr int READS = 2 * (TM + TN);  // 16-byte fragment reads per slice
};

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Wait until at most n slices of L copies each are still in flight.
template <int L>
__device__ __forceinline__ void wait_slices(int n) {
    static_assert(3 * L < 64, "vmcnt range");
    if (n <= 0) wait_vm<0>();
    else if (n == 1) wait_vm<L>();
    else if (n == 2) wait_vm<2 * L>();
    else wait_vm<3 * L>();
}
__device__ __forceinline__ void fence_sched() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void slice_barrier() {
    fence_sched();
    __builtin_amdgcn_s_barrier();
    fence_sched();
}

template <int TM, int TN>
struct Frags {
    i32x4 a[TM][2];
    i32x4 b[TN][2];
};

__device__ __forceinline__ f32x16 mfma8(const i32x4 (&x)[2], const i32x4 (&y)[2], f32x16 c) {
    const i32x8 xa = __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const i32x8 ya = __builtin_shufflevector(y[0], y[1], 0, 1, 2, 3, 4, 5, 6, 7);
    // Both operands E4M3 (format 0), no block scales: with both scale
    // operands 0 the compiler emits the unscaled v_mfma_f32_32x32x64_f8f6f4
    // (plain E4M3 products; the parity tests compare against the oracle bit
    // for bit on integer codes).
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa, ya, c, 0, 0, 0, 0, 0, 0);
}

struct F8Args {
    const float* sa;      // M scales of A's rows
    const float* sb;      // N scales of B's rows (output columns)
    float* part;          // split K: [tile][range][chunk][thread] f32x4 partial sums
    int ksplit;           // K ranges (1: no split)
    int nks;              // 64-slices per range (the last range may hold fewer)
};
// Tile order of split launches: groups two M-tiles deep, so an XCD that holds
// all K ranges of its tiles streams little of A twice.
constexpr int SPLIT_GROUP_M = 2;
// Unsplit launches group tiles four M-tiles deep, as in k_h_dma.hip (FP8
// 4096x16384x4096 267 against 321 us with groups of 8, 4096^3 68 against
// 71, 16384x4096x4096 260 against 272; 8192^3 and 4096x1536x4096 1-2%).
constexpr int UNSPLIT_GROUP_M = 4;

template <int CT>
__device__ __forceinline__ void store4(void* C, int64_t ldc, int64_t m, int64_t n, int nlim_n,
                                       bool vec_ok, float beta, float (&v)[4]) {
    if constexpr (CT == F32) {
        float* c = (float*)C + m * ldc + n;
        const bool full = vec_ok && nlim_n >= 4;
        if (beta != 0.f) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < nlim_n) v[e] = fmaf(beta, c[e], v[e]);
        }
        if (full) *(f32x4*)c = f32x4{v[0], v[1], v[2], v[3]};
        else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < nlim_n) c[e] = v[e];
        }
    } else {
        store_out4<CT, EPI_NONE>((uint16_t*)C + m * ldc, (int)n, (int)n + nlim_n, vec_ok, beta, v);
    }
}

// Scaled output of one wave's 128 x BN/2 block.  The lane's scales are
// loaded before the stores to C that follow them (a load the compiler cannot
// prove disjoint from an earlier store waits for that store: measured,
// 10 us per call when every column's scale was loaded next to its store).
// The 256-wide tile does this in two halves of its columns to stay within
// the registers.
template <int CT, int BN, int BMT>
__device__ __forceinline__ void f8_epilogue(const f32x16 (&acc)[BMT / 64][BN / 64], const Problem& p,
                                            const float* sa, const float* sb, void* C, int lane,
                                            int wm, int wn, int64_t m0, int64_t n0, int mlim,
                                            int nlim) {
    constexpr int TM = BMT / 64, TN = BN / 64, WROWS = BMT / 2;
    constexpr int PH = BN == 256 ? 2 : 1, TNP = TN / PH;    // column phases
    const int fr = lane & 31, nq = 4 * (lane >> 5);
    const int es = CT == F32 ? 4 : 2;
    const bool vec_ok = (p.ldc % 4 == 0) && (((uintptr_t)C & (4 * es - 1)) == 0);
    const bool sb_vec = ((uintptr_t)sb & 15) == 0;
    float sav[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int mi = WROWS * wm + 32 * tm + fr;
        sav[tm] = mi < mlim ? sa[m0 + mi] : 0.0f;
    }
#pragma unroll
    for (int ph = 0; ph < PH; ++ph) {
        f32x4 sbv[TNP][4];
#pragma unroll
        for (int t = 0; t < TNP; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ni = BN / 2 * wn + 32 * (ph * TNP + t) + 8 * q + nq;
                if (sb_vec && ni + 4 <= nlim) {
                    sbv[t][q] = *(const f32x4*)(sb + n0 + ni);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sbv[t][q][e] = ni + e < nlim ? sb[n0 + ni + e] : 0.0f;
                }
            }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int mi = WROWS * wm + 32 * tm + fr;
            if (mi >= mlim) continue;
#pragma unroll
            for (int t = 0; t < TNP; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int tn = ph * TNP + t;
                    const int ni = BN / 2 * wn + 32 * tn + 8 * q + nq;
                    if (ni >= nlim) continue;
                    const int nn = nlim - ni < 4 ? nlim - ni : 4;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = p.alpha * ((acc[tm][tn][4 * q + e] * sav[tm]) * sbv[t][q][e]);
                    store4<CT>(C, p.ldc, m0 + mi, n0 + ni, nn, vec_ok, p.beta, v);
                }
        }
    }
}

template <int CT, int BN, bool PARTIAL, int BMT = 256>
__global__ __launch_bounds__(NT, 1) void k_f8_dma(Problem p, F8Args f) {
    using G = F8Cfg<BN, BMT>;
    constexpr int BM = BMT, TM = G::TM, TN = G::TN, COPIES = G::COPIES, SLOT_BYTES = G::SLOT_BYTES;
    constexpr int A_COPIES = G::A_COPIES, A_BYTES = G::A_BYTES, WROWS = G::WROWS;
    using Fr = Frags<TM, TN>;
    extern __shared__ __align__(16) unsigned char smem[];
    const ClockStamp stamp0 = clock_stamp_begin();
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
    // Position tile * ksplit + range in an order where each XCD's workgroups
    // are consecutive: all K ranges of a tile run on one XCD, and the second
    // phase sums each tile on that XCD (as in k_h_dma.hip's split of K).
    const int pos = xcd_linear(blockIdx.x, gridDim.x);
    const int split = pos % f.ksplit;
    int tmi, tni;
    tile_from_linear(pos / f.ksplit, tiles_m, tiles_n, f.ksplit > 1 ? SPLIT_GROUP_M : UNSPLIT_GROUP_M,
                     tmi, tni);
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const int mlim = (int)(p.M - m0 < BM ? p.M - m0 : BM);
    const int nlim = (int)(p.N - n0 < BN ? p.N - n0 : BN);
    const int64_t k0 = (int64_t)split * f.nks * BK;         // first K of this range
    const uint8_t* __restrict__ A = (const uint8_t*)p.A + k0;
    const uint8_t* __restrict__ B = (const uint8_t*)p.B + k0;

    // Copies of this wave: rows [64w, 64w+64) of the A tile and
    // [BN/4*w, BN/4*(w+1)) of the B tile, 16 rows per copy (lane l: row
    // 16i + l/4, 16-byte chunk l%4 stored at the swizzled chunk position).
    // Rows past the edge repeat the last row.
    const uint8_t* src[COPIES];
    int dst[COPIES];
#pragma unroll
    for (int i = 0; i < A_COPIES; ++i) {
        const int r = BM / 4 * wave + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ swz(r);
        const int ra = r < mlim ? r : mlim - 1;
        src[i] = A + (m0 + ra) * p.lda + 16 * c;
        dst[i] = (BM / 4 * wave + 16 * i) * ROW;
    }
#pragma unroll
    for (int i = 0; i < G::B_COPIES; ++i) {
        const int r = BN / 4 * wave + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ swz(r);
        const int rb = r < nlim ? r : nlim - 1;
        src[A_COPIES + i] = B + (n0 + rb) * p.ldb + 16 * c;
        dst[A_COPIES + i] = A_BYTES + (BN / 4 * wave + 16 * i) * ROW;
    }
    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    auto copy = [&](int s, int i) {
        copy_to_lds(src[i] + (int64_t)s * BK, lds0 + (unsigned)(s % SLOTS) * SLOT_BYTES + dst[i]);
    };
    // Fragment offsets: lane l holds 32 K-consecutive bytes (chunks
    // 2*(l/32) and 2*(l/32)+1) of row l%32 of its 32-row block.
    int a_off[TM][2], b_off[TN][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = 2 * (lane >> 5) + h;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int ra = WROWS * wm + 32 * t + (lane & 31);
            a_off[t][h] = ra * ROW + ((c ^ swz(ra)) << 4);
        }
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const int rb = BN / 2 * wn + 32 * t + (lane & 31);
            b_off[t][h] = A_BYTES + rb * ROW + ((c ^ swz(rb)) << 4);
        }
    }
    // Read r of a slice: A0, B0..B(TN-1), A1..A3, two 16-byte halves each.
    auto read = [&](Fr& fr, int s, int r) {
        const unsigned char* base = smem + (s % SLOTS) * SLOT_BYTES;
        const int item = r >> 1, h = r & 1;
        if (item == 0) fr.a[0][h] = *(const i32x4*)(base + a_off[0][h]);
        else if (item <= TN) fr.b[item - 1][h] = *(const i32x4*)(base + b_off[item - 1][h]);
        else fr.a[item - TN][h] = *(const i32x4*)(base + a_off[item - TN][h]);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    // One slice: the TM*TN MFMAs on `use`; read r of slice rs into `nxt`
    // follows MFMA r*NM/READS and copy c of slice cs follows MFMA c*NM/COPIES.
    constexpr int NM = TM * TN, NR = G::READS;
    auto step = [&](const Fr& use, Fr& nxt, bool do_read, int rs, bool do_copy, int cs) {
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            // Row-wise snake order, as in k_h_dma.hip: fewer operand changes
            // between consecutive MFMAs at the power limit.
            const int tm = i / TN, tn = (tm & 1) ? TN - 1 - i % TN : i % TN;
            acc[tm][tn] = mfma8(use.b[tn], use.a[tm], acc[tm][tn]);
            if (do_copy) {
#pragma unroll
                for (int c = 0; c < COPIES; ++c)
                    if (c * NM / COPIES == i) copy(cs, c);
            }
            if (do_read) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    if (r * NM / NR == i) read(nxt, rs, r);
            }
            fence_sched();
        }
    };

    const int nk_all = (int)(p.K / BK);
    const int nk = nk_all - split * f.nks < f.nks ? nk_all - split * f.nks : f.nks;
    const int npro = nk < AHEAD ? nk : AHEAD;
    for (int s = 0; s < npro; ++s)
        for (int i = 0; i < COPIES; ++i) copy(s, i);
    wait_slices<COPIES>(npro - 1);
    slice_barrier();
    Fr f0, f1;
#pragma unroll
    for (int r = 0; r < NR; ++r) read(f0, 0, r);

    // Pairs of slices (the fragment buffers alternate); every slice waits
    // for this wave's copies of the next slice, then a barrier makes them
    // visible to all waves and frees the slot of the slice before.
    int j = 0;
    for (; j + 1 + AHEAD < nk; j += 2) {
        wait_slices<COPIES>(AHEAD - 2);
        slice_barrier();
        step(f0, f1, true, j + 1, true, j + AHEAD);
        wait_slices<COPIES>(AHEAD - 2);
        slice_barrier();
        step(f1, f0, true, j + 2, true, j + 1 + AHEAD);
    }
    for (; j < nk; j += 2) {        // the last slices: copies only while any remain
        int left = nk - j - 2;
        if (j + 1 < nk) {
            wait_slices<COPIES>(left < AHEAD - 2 ? left : AHEAD - 2);
            slice_barrier();
        }
        step(f0, f1, j + 1 < nk, j + 1, j + AHEAD < nk, j + AHEAD);
        if (j + 1 >= nk) break;
        left = nk - j - 3;
        if (j + 2 < nk) {
            wait_slices<COPIES>(left < AHEAD - 2 ? left : AHEAD - 2);
            slice_barrier();
        }
        step(f1, f0, j + 2 < nk, j + 2, j + 1 + AHEAD < nk, j + 1 + AHEAD);
    }

    // K tail (K not a multiple of 64), as in k_h_dma.hip: the range that ends
    // at the last whole slice stages one more slice with ordinary loads into
    // the LDS positions of the copies (lane l's 16 codes of copy i at dst[i] +
    // 16*l: codes 16c .. 16c+15 of its row, c the swizzled chunk), zero codes
    // (+0.0) for k >= K in both operands, then one more step.  Only k < K is
    // read; no copy is in flight after the loop above.
    const int ktail = (int)(p.K - (int64_t)nk_all * BK);
    if (ktail > 0 && split * f.nks + nk == nk_all) {
        const int ts = nk;
        __syncthreads();
        unsigned char* slot = smem + (ts % SLOTS) * SLOT_BYTES;
#pragma unroll
        for (int i = 0; i < COPIES; ++i) {
            const int r = i < A_COPIES ? BM / 4 * wave + 16 * i + (lane >> 2)
                                       : BN / 4 * wave + 16 * (i - A_COPIES) + (lane >> 2);
            const int kfirst = 16 * ((lane & 3) ^ swz(r));
            const uint8_t* s = src[i] + (int64_t)ts * BK;
            i32x4 v = i32x4{0, 0, 0, 0};
            if (kfirst + 16 <= ktail) {
                v = *(const i32x4*)s;
            } else if (kfirst < ktail) {
                uint8_t e[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) e[q] = kfirst + q < ktail ? s[q] : (uint8_t)0;
                v = __builtin_bit_cast(i32x4, e);
            }
            *(i32x4*)(slot + dst[i] + 16 * lane) = v;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < NR; ++r) read(f0, ts, r);
        step(f0, f1, false, 0, false, 0);
    }

    // Epilogue: lane holds C(m, n..n+3), m = row within the 32x32 block.
    if constexpr (PARTIAL) {
        // Chunk c = (tm * TN + tn) * 4 + q holds acc[tm][tn][4q .. 4q+3].
        float* dst = f.part + ((int64_t)(tmi * tiles_n + tni) * f.ksplit + split) *
                                  (int64_t)(NT * TM * TN * 16) + 4 * tid;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16& a = acc[tm][tn];
                    const f32x4 v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                    *(f32x4*)(dst + (int64_t)((tm * TN + tn) * 4 + q) * NT * 4) = v;
                }
        clock_stamp_end(p, stamp0);
        return;
    }
    f8_epilogue<CT, BN, BMT>(acc, p, f.sa, f.sb, p.C, lane, wm, wn, m0, n0, mlim, nlim);
    clock_stamp_end(p, stamp0);
}

// Second split-K phase: one thread per 16-byte chunk of a tile's
// accumulators sums the K ranges in range order, then scales and stores the
// four outputs as the one-phase epilogue would.
template <int CT, int BN, int BMT = 256>
__global__ __launch_bounds__(NT) void k_f8_reduce(Problem p, F8Args f) {
    constexpr int BM = BMT, TM = BMT / 64, TN = BN / 64, CH = TM * TN * 4;
    constexpr int64_t TILE_FLOATS = (int64_t)NT * TM * TN * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
    const int pos = xcd_linear(blockIdx.x, gridDim.x);   // the first phase's tile order
    const int t = pos / CH, c = pos % CH;
    int tmi, tni;
    tile_from_linear(t, tiles_m, tiles_n, SPLIT_GROUP_M, tmi, tni);
    const int tm = c / (TN * 4), tn = (c / 4) % TN, q = c % 4;
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const int mlim = (int)(p.M - m0 < BM ? p.M - m0 : BM);
    const int nlim = (int)(p.N - n0 < BN ? p.N - n0 : BN);
    const int mi = BMT / 2 * wm + 32 * tm + (lane & 31);
    const int ni = BN / 2 * wn + 32 * tn + 8 * q + 4 * (lane >> 5);
    if (mi >= mlim || ni >= nlim) return;
    const float* src = f.part + (int64_t)(tmi * tiles_n + tni) * f.ksplit * TILE_FLOATS + (int64_t)c * NT * 4 + 4 * tid;
    f32x4 a = *(const f32x4*)src;
    int s = 1;
    for (; s + 4 <= f.ksplit; s += 4) {
        const f32x4 b0 = *(const f32x4*)(src + s * TILE_FLOATS);
        const f32x4 b1 = *(const f32x4*)(src + (s + 1) * TILE_FLOATS);
        const f32x4 b2 = *(const f32x4*)(src + (s + 2) * TILE_FLOATS);
        const f32x4 b3 = *(const f32x4*)(src + (s + 3) * TILE_FLOATS);
        a = (((a + b0) + b1) + b2) + b3;
    }
    for (; s < f.ksplit; ++s) a = a + *(const f32x4*)(src + s * TILE_FLOATS);
    const int nn = nlim - ni < 4 ? nlim - ni : 4;
    const float sam = f.sa[m0 + mi];
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = p.alpha * ((a[e] * sam) * (e < nn ? f.sb[n0 + ni + e] : 0.0f));
    const int es = CT == F32 ? 4 : 2;
    const bool vec_ok = (p.ldc % 4 == 0) && (((uintptr_t)p.C & (4 * es - 1)) == 0);
    store4<CT>(p.C, p.ldc, m0 + mi, n0 + ni, nn, vec_ok, p.beta, v);
}

// Any K, alignment and leading dimension: 64x64 output tiles of 256 threads,
// 64 x 16 slices of both code matrices decoded to FP32 in LDS (zeros past the
// edges), a 4x4 register block per thread.  Every output accumulates its
// products with fmaf in K order over k < K only, then alpha and the row and
// column scales are applied as in the MFMA kernels' epilogue.
constexpr int FG_T = 64, FG_BK = 16;

template <int CT>
__global__ __launch_bounds__(256) void k_f8_general(Problem p, F8Args f) {
    __shared__ float As[FG_BK][FG_T + 4];
    __shared__ float Bs[FG_BK][FG_T + 4];
    const int tid = threadIdx.x;
    const int tiles_m = (int)((p.M + FG_T - 1) / FG_T), tiles_n = (int)((p.N + FG_T - 1) / FG_T);
    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tm, tn);
    const int64_t m0 = (int64_t)tm * FG_T, n0 = (int64_t)tn * FG_T;
    const uint8_t* A = (const uint8_t*)p.A;
    const uint8_t* B = (const uint8_t*)p.B;
    float acc[4][4] = {};
    const int ty = tid / 16, tx = tid % 16;
    for (int64_t k0 = 0; k0 < p.K; k0 += FG_BK) {
        // 64 rows x 16 codes of each operand, 4 per thread; consecutive
        // threads walk K (both code matrices are K-contiguous).
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = tid + r * 256, ri = e / FG_BK, ki = e % FG_BK;
            const int64_t k = k0 + ki, m = m0 + ri, n = n0 + ri;
            As[ki][ri] = (m < p.M && k < p.K) ? e4m3_value(A[m * p.lda + k]) : 0.0f;
            Bs[ki][ri] = (n < p.N && k < p.K) ? e4m3_value(B[n * p.ldb + k]) : 0.0f;
        }
        __syncthreads();
        const int kn = p.K - k0 < FG_BK ? (int)(p.K - k0) : FG_BK;
        for (int kk = 0; kk < kn; ++kk) {
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= p.M) continue;
        const float sam = f.sa[m];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n >= p.N) continue;
            float v[4] = {p.alpha * ((acc[i][j] * sam) * f.sb[n]), 0.f, 0.f, 0.f};
            store4<CT>(p.C, p.ldc, m, n, 1, false, p.beta, v);
        }
    }
}

template <int XT>
hipError_t launch_quant_xt(int64_t M, int64_t K, const void* X, int64_t ldx, uint8_t* Q, int64_t ldq,
                           float* scales, hipStream_t s) {
    constexpr int ES = XT == F32 ? 4 : 2, V = 16 / ES;
    const bool vec = K % V == 0 && (ldx * ES) % 16 == 0 && ((uintptr_t)X & 15) == 0 &&
                     ldq % V == 0 && ((uintptr_t)Q & (V - 1)) == 0;
    const int64_t per_thread = (K / V + 255) / 256;       // 16-byte chunks per thread
    if (vec && per_thread <= 8 && M <= 0x7fffffff) {
        const dim3 grid((unsigned)M);
        if (per_thread <= 1)
            hipLaunchKernelGGL((k_quant_rows_reg<XT, 1>), grid, dim3(256), 0, s, M, K, X, ldx, Q, ldq, scales);
        else if (per_thread <= 2)
            hipLaunchKernelGGL((k_quant_rows_reg<XT, 2>), grid, dim3(256), 0, s, M, K, X, ldx, Q, ldq, scales);
        else if (per_thread <= 4)
            hipLaunchKernelGGL((k_quant_rows_reg<XT, 4>), grid, dim3(256), 0, s, M, K, X, ldx, Q, ldq, scales);
        else
            hipLaunchKernelGGL((k_quant_rows_reg<XT, 8>), grid, dim3(256), 0, s, M, K, X, ldx, Q, ldq, scales);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((M + 3) / 4));
    if (vec) hipLaunchKernelGGL((k_quant_rows<XT, true>), grid, dim3(256), 0, s, M, K, X, ldx, Q, ldq, scales);
    else hipLaunchKernelGGL((k_quant_rows<XT, false>), grid, dim3(256), 0, s, M, K, X, ldx, Q, ldq, scales);
    return hipGetLastError();
}

template <int CT, int BN, bool PARTIAL, int BMT = 256>
hipError_t launch_f8_dma(const Problem& p, const F8Args& f, hipStream_t s) {
    constexpr int BM = BMT;
    auto kern = k_f8_dma<CT, BN, PARTIAL, BMT>;
    const size_t lds = (size_t)SLOTS * F8Cfg<BN, BMT>::SLOT_BYTES;
    static bool attr_set[MAX_DEVICES] = {};
    if (hipError_t e = set_lds_limit_once((const void*)kern, (int)lds, attr_set); e != hipSuccess)
        return e;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3((unsigned)(tiles * f.ksplit)), dim3(NT), lds, s, p, f);
    if constexpr (PARTIAL) {
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        constexpr int CH = F8Cfg<BN, BMT>::TM * (BN / 64) * 4;
        hipLaunchKernelGGL((k_f8_reduce<CT, BN, BMT>), dim3((unsigned)(tiles * CH)), dim3(NT), 0, s, p, f);
    }
    return hipGetLastError();
}

// bn: 256 or 192 for the MFMA kernel, 0 for the scalar kernel; bm: 256, or
// 128 with bn = 192.
template <int CT>
hipError_t launch_f8_ct(const Problem& p, const F8Args& f, int bn, int bm, hipStream_t s) {
    if (bm == 128 && bn == 192)
        return f.ksplit > 1 ? launch_f8_dma<CT, 192, true, 128>(p, f, s)
                            : launch_f8_dma<CT, 192, false, 128>(p, f, s);
    if (bn == 256)
        return f.ksplit > 1 ? launch_f8_dma<CT, 256, true>(p, f, s) : launch_f8_dma<CT, 256, false>(p, f, s);
    if (bn == 192)
        return f.ksplit > 1 ? launch_f8_dma<CT, 192, true>(p, f, s) : launch_f8_dma<CT, 192, false>(p, f, s);
    const int64_t tiles = ((p.M + FG_T - 1) / FG_T) * ((p.N + FG_T - 1) / FG_T);
    hipLaunchKernelGGL(k_f8_general<CT>, dim3((unsigned)tiles), dim3(256), 0, s, p, f);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fp8(int64_t M, int64_t K, const void* X, int64_t ldx, int xtype, void* Q,
                               int64_t ldq, float* scales, hipStream_t s) {
    if (xtype == F32) return launch_quant_xt<F32>(M, K, X, ldx, (uint8_t*)Q, ldq, scales, s);
    if (xtype == F16) return launch_quant_xt<F16>(M, K, X, ldx, (uint8_t*)Q, ldq, scales, s);
    return launch_quant_xt<BF16>(M, K, X, ldx, (uint8_t*)Q, ldq, scales, s);
}

bool f8_mfma_supports_bm(const Problem& p, int bn, int bm) {
    if (bn != 256 && bn != 192) return false;
    if (bm != 256 && (bm != 128 || bn != 192)) return false;
    const int BM = bm;
    // K >= 64; a last partial slice (K not a multiple of 64) is staged by
    // ordinary loads with zero codes past K.
    if (p.K < BK || p.lda % 16 != 0 || p.ldb % 16 != 0) return false;
    if (((uintptr_t)p.A & 15) != 0 || ((uintptr_t)p.B & 15) != 0) return false;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + bn - 1) / bn);
    return tiles > 0 && tiles <= 0x7fffffff;
}

bool f8_mfma_supports(const Problem& p, int bn) { return f8_mfma_supports_bm(p, bn, 256); }

bool f8_general_supports(const Problem& p) {
    return ((p.M + FG_T - 1) / FG_T) * ((p.N + FG_T - 1) / FG_T) <= 0x7fffffff;
}

int f8_splits_bm(const Problem& p, int bn, int bm, int requested, const Workspace& ws) {
    const int BM = bm;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + bn - 1) / bn);
    const int64_t nk = p.K / BK;
    if (requested <= 1 || nk < 2) return 1;
    int64_t ks = requested < nk ? requested : nk;
    const int64_t nks = (nk + ks - 1) / ks;                 // whole 64-slices per range
    ks = (nk + nks - 1) / nks;
    if (ws.part == nullptr || tiles * ks * (int64_t)BM * bn * 4 > ws.part_bytes) return 0;
    return (int)ks;
}

int f8_splits(const Problem& p, int bn, int requested, const Workspace& ws) {
    return f8_splits_bm(p, bn, 256, requested, ws);
}

hipError_t launch_f8_gemm_bm(const Problem& p, const float* sa, const float* sb, int bn, int bm,
                             int ksplit, const Workspace& ws, hipStream_t s) {
    F8Args f{sa, sb, (float*)ws.part, 1, (int)(p.K / BK)};
    if (bn != 0 && ksplit > 1) {
        const int nk = (int)(p.K / BK);
        f.nks = (nk + ksplit - 1) / ksplit;
        f.ksplit = (nk + f.nks - 1) / f.nks;
    }
    if (p.dtype == F32) return launch_f8_ct<F32>(p, f, bn, bm, s);
    if (p.dtype == F16) return launch_f8_ct<F16>(p, f, bn, bm, s);
    return launch_f8_ct<BF16>(p, f, bn, bm, s);
}

hipError_t launch_f8_gemm(const Problem& p, const float* sa, const float* sb, int bn, int ksplit,
                          const Workspace& ws, hipStream_t s) {
    return launch_f8_gemm_bm(p, sa, sb, bn, 256, ksplit, ws, s);
}

}  // namespace mgemm
