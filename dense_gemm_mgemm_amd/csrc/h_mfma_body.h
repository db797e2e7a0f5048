// Register-staged FP16/BF16 GEMM kernel template, shared by k_h_mfma.hip
// (16-byte loads) and k_h_mfma_u.hip (narrow loads for operands that are
// not 16-byte aligned).  Design notes in k_h_mfma.hip.
#pragma once
#include "common.h"

#include <type_traits>

namespace mgemm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BK = 64;              // K elements per LDS slot
constexpr int LDS_ROW = BK + 8;     // padded row, in 16-bit elements (144 B)
constexpr int NT = 256;

template <int DT>
__device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Buffer resource over a K slice of an operand for the narrow loads (AW <
// 16; the 16-byte path addresses memory directly and the unused resource is
// dropped).  Offsets stay below 2^31 bytes (the host limits the leading
// dimensions).
template <int AW>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t narrow_rsrc(const uint16_t* P) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)P, 0, 0x7fffffff, 0x00020000);
}

// Eight consecutive 16-bit elements at element offset `off` of P.  AW = 16:
// one 16-byte load (P + off 16-byte aligned).  AW = 4 (dword-aligned
// operands): one 16-byte buffer load; multi-dword loads need only dword
// alignment outside the strict alignment mode, and 8-byte-aligned ones are
// what the compiler itself makes of two 8-byte loads.  AW = 2: eight 2-byte
// buffer loads, each naturally aligned (through the buffer resource `rs` over
// P: plain 2-byte loads would be merged back into one unaligned 16-byte load).
template <int AW>
__device__ __forceinline__ i32x4 load_run(const uint16_t* P, __amdgpu_buffer_rsrc_t rs, int64_t off) {
    if constexpr (AW == 16) {
        return *(const i32x4*)(P + off);
    } else if constexpr (AW == 4) {
        return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)(off * 2), 0, 0));
    } else {
        static_assert(AW == 2, "load width");
        const unsigned b = (unsigned)(off * 2);
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = __builtin_amdgcn_raw_buffer_load_b16(rs, b + 2 * q, 0, 0);
        return __builtin_bit_cast(i32x4, e);
    }
}

// One operand tile of R rows (M or N index) by BK (K index).
//   KC: the global operand is K-contiguous: element (r, k) at P[r*ld + k].
//   else MN-contiguous: element (r, k) at P[k*ld + r].
// `rlim` / `klim` are the valid extents from the tile origin.
template <int R, bool KC, int AW>
struct TileLoader {
    static constexpr int CHUNKS = R * (BK / 8);                    // 16-byte K-runs (KC)
    static constexpr int PER_T = KC ? CHUNKS / NT : (R / 8 * (BK / 8) + NT - 1) / NT;
    static constexpr int NREG = KC ? PER_T : PER_T * 8;             // i32x4 registers held
    static_assert(!KC || CHUNKS % NT == 0, "K-contiguous tile must split evenly");
    i32x4 v[NREG];

    // FULL: the slice lies entirely inside the matrix (interior tile, whole K
    // slice), so every load is an unconditional 16-byte load.  Keeping the
    // edge masks out of this path matters: per-element conditional loads make
    // the compiler wait for all outstanding loads after each of them.
    template <bool FULL>
    __device__ __forceinline__ void fetch(const uint16_t* __restrict__ P, int64_t ld, int rlim,
                                          int klim, int tid) {
        const __amdgpu_buffer_rsrc_t rs = narrow_rsrc<AW>(P);
        if constexpr (FULL) {
            if constexpr (KC) {
#pragma unroll
                for (int i = 0; i < PER_T; ++i) {
                    const int c = tid + i * NT;
                    const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
                    v[i] = load_run<AW>(P, rs, (int64_t)r * ld + kc);
                }
            } else {
#pragma unroll
                for (int i = 0; i < PER_T; ++i) {
                    const int b = tid + i * NT;
                    const int kb = (b % (BK / 8)) * 8, rb = (b / (BK / 8)) * 8;
                    if (b < R / 8 * (BK / 8)) {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            v[i * 8 + j] = load_run<AW>(P, rs, (int64_t)(kb + j) * ld + rb);
                    }
                }
            }
        } else if constexpr (KC) {
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const int c = tid + i * NT;
                const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
                const uint16_t* src = P + (int64_t)r * ld + kc;
                if (r < rlim && kc + 8 <= klim) {
                    v[i] = load_run<AW>(P, rs, (int64_t)r * ld + kc);
                } else {
                    uint16_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (r < rlim && kc + j < klim) ? src[j] : 0;
                    v[i] = __builtin_bit_cast(i32x4, e);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const int b = tid + i * NT;
                const int kb = (b % (BK / 8)) * 8, rb = (b / (BK / 8)) * 8;
                // Raw rows only: the transpose waits until stash(), after the
                // matrix cores have consumed the current slice, so these loads
                // stay in flight during the MFMAs.
                if (b < R / 8 * (BK / 8)) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint16_t* src = P + (int64_t)(kb + j) * ld + rb;
                        if (kb + j < klim && rb + 8 <= rlim) {
                            v[i * 8 + j] = load_run<AW>(P, rs, (int64_t)(kb + j) * ld + rb);
                        } else {
                            uint16_t e[8];
#pragma unroll
                            for (int q = 0; q < 8; ++q)
                                e[q] = (kb + j < klim && rb + q < rlim) ? src[q] : 0;
                            v[i * 8 + j] = __builtin_bit_cast(i32x4, e);
                        }
                    }
                }
            }
        }
    }

    __device__ __forceinline__ void stash(uint16_t* __restrict__ S, int tid) const {
        if constexpr (KC) {
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const int c = tid + i * NT;
                const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
                *(i32x4*)(S + r * LDS_ROW + kc) = v[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const int b = tid + i * NT;
                if (b < R / 8 * (BK / 8)) {
                    const int kb = (b % (BK / 8)) * 8, rb = (b / (BK / 8)) * 8;
                    // 8x8 transpose of 16-bit elements: K-run c is
                    // (row0[c], row1[c], ..., row7[c]).
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        i32x4 o;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t lo = (uint32_t)v[i * 8 + 2 * q][c / 2];
                            const uint32_t hi = (uint32_t)v[i * 8 + 2 * q + 1][c / 2];
                            o[q] = (int)((c & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                                 : ((lo & 0xffffu) | (hi << 16)));
                        }
                        *(i32x4*)(S + (rb + c) * LDS_ROW + kb) = o;
                    }
                }
            }
        }
    }
};

template <int DT, int BM, int BN, bool AKC, bool BKC, int AW>
__global__ __launch_bounds__(NT, (BM * BN <= 128 * 128) ? 2 : 1) void k_h_mfma(Problem p) {
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    extern __shared__ __align__(16) uint16_t smem[];
    uint16_t* As = smem;                              // [2][BM][LDS_ROW]
    uint16_t* Bs = smem + 2 * BM * LDS_ROW;           // [2][BN][LDS_ROW]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
    int tmi, tni;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tmi, tni);
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const int mlim = (int)(p.M - m0 < BM ? p.M - m0 : BM);
    const int nlim = (int)(p.N - n0 < BN ? p.N - n0 : BN);

    const uint16_t* __restrict__ A = (const uint16_t*)p.A;
    const uint16_t* __restrict__ B = (const uint16_t*)p.B;
    // Tile origins; per K slice the pointers advance along K.
    const uint16_t* a_base = AKC ? A + m0 * p.lda : A + m0;
    const uint16_t* b_base = BKC ? B + n0 * p.ldb : B + n0;
    const int64_t a_kstep = AKC ? BK : (int64_t)BK * p.lda;
    const int64_t b_kstep = BKC ? BK : (int64_t)BK * p.ldb;

    TileLoader<BM, AKC, AW> la;
    TileLoader<BN, BKC, AW> lb;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    const int64_t nk = (p.K + BK - 1) / BK;
    auto klim_of = [&](int64_t kt) { return (int)(p.K - kt * BK < BK ? p.K - kt * BK : BK); };
    const int fr = lane & 31;            // fragment row within a 32-row block
    const int fk = (lane >> 5) * 8;      // this lane's 8 K elements within a 16-K step

    // The whole K loop is instantiated twice: FULL for interior tiles whose
    // every K slice is complete (unconditional 16-byte loads only), and a
    // masked copy for edge tiles and ragged K.  Choosing once per tile keeps
    // the two load paths from merging inside the loop, where the compiler
    // would have to wait for the loads before the contraction.
    auto main_loop = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        auto fetch = [&](int64_t kt) {
            const int kl = klim_of(kt);
            la.template fetch<FULL>(a_base + kt * a_kstep, p.lda, mlim, kl, tid);
            lb.template fetch<FULL>(b_base + kt * b_kstep, p.ldb, nlim, kl, tid);
        };
        fetch(0);
        la.stash(As, tid);
        lb.stash(Bs, tid);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int cur = (int)(kt & 1);
            if (kt + 1 < nk) fetch(kt + 1);
            const uint16_t* as = As + cur * BM * LDS_ROW + (wm * WTM + fr) * LDS_ROW + fk;
            const uint16_t* bs = Bs + cur * BN * LDS_ROW + (wn * WTN + fr) * LDS_ROW + fk;
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                i32x4 af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) af[i] = *(const i32x4*)(as + i * 32 * LDS_ROW + ks * 16);
#pragma unroll
                for (int j = 0; j < TN; ++j) bf[j] = *(const i32x4*)(bs + j * 32 * LDS_ROW + ks * 16);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma<DT>(bf[j], af[i], acc[i][j]);
            }
            if (kt + 1 < nk) {
                la.stash(As + (cur ^ 1) * BM * LDS_ROW, tid);
                lb.stash(Bs + (cur ^ 1) * BN * LDS_ROW, tid);
            }
            __syncthreads();
        }
    };
    if (mlim == BM && nlim == BN && p.K % BK == 0) main_loop(std::true_type{});
    else main_loop(std::false_type{});

    // Epilogue: lane holds C(m, n..n+3) for m = fr, n = 8q + 4*(lane/32).
    uint16_t* C = (uint16_t*)p.C;
    const bool vec_ok = (p.ldc % 4 == 0) && (((uintptr_t)p.C & 7) == 0);
    const int nq = 4 * (lane >> 5);
    with_epilogue(p.epilogue, [&](auto E) {
        constexpr int EPI = decltype(E)::value;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int mi = wm * WTM + i * 32 + fr;
            if (mi >= mlim) continue;
            uint16_t* crow = C + (m0 + mi) * p.ldc + n0;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ni = wn * WTN + j * 32 + 8 * q + nq;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = p.alpha * acc[i][j][4 * q + e];
                    store_out4<DT, EPI>(crow, ni, nlim, vec_ok, p.beta, v);
                }
            }
        }
    });
}

template <int DT, int BM, int BN, bool AKC, bool BKC, int AW>
hipError_t launch_one(const Problem& p, hipStream_t s) {
    auto kern = k_h_mfma<DT, BM, BN, AKC, BKC, AW>;
    const size_t lds = (size_t)2 * (BM + BN) * LDS_ROW * sizeof(uint16_t);
    static bool attr_set[MAX_DEVICES] = {};
    if (hipError_t e = set_lds_limit_once((const void*)kern, (int)lds, attr_set); e != hipSuccess)
        return e;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(NT), lds, s, p);
    return hipGetLastError();
}

template <int BM, int BN, int AW>
hipError_t dispatch_layout(const Problem& p, hipStream_t s) {
    const int k = (p.a_kc ? 2 : 0) | (p.b_kc ? 1 : 0);
    if (p.dtype == F16) {
        switch (k) {
        case 0: return launch_one<F16, BM, BN, false, false, AW>(p, s);
        case 1: return launch_one<F16, BM, BN, false, true, AW>(p, s);
        case 2: return launch_one<F16, BM, BN, true, false, AW>(p, s);
        default: return launch_one<F16, BM, BN, true, true, AW>(p, s);
        }
    }
    switch (k) {
    case 0: return launch_one<BF16, BM, BN, false, false, AW>(p, s);
    case 1: return launch_one<BF16, BM, BN, false, true, AW>(p, s);
    case 2: return launch_one<BF16, BM, BN, true, false, AW>(p, s);
    default: return launch_one<BF16, BM, BN, true, true, AW>(p, s);
    }
}

}  // namespace

// The forms with buffer loads (k_h_mfma_u.hip) for operands that are not
// 16-byte aligned; aw is their common alignment in bytes (2, 4 or 8).
hipError_t launch_h_mfma_narrow(const Problem& p, int variant, int aw, hipStream_t s);

}  // namespace mgemm
