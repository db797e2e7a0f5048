// Skinny-M FP16/BF16 GEMM (M <= 64): C[M x N] = X[M x K] * W[K x N], the
// decode-like projection of the SGEMM report's "decode b1/b32" measurements and
// of the FFN example of "Chapter 5: Operators and Runtime" (section 5.2.1) at
// small M.  The arithmetic intensity is about M flop per byte of W, so the
// kernel is bound by streaming W from HBM once; everything else is arranged
// around keeping enough bytes of W in flight.
//
// Work split.  One 256-thread workgroup per 64-column block of W (128-byte
// row segments: whole L2 lines, so no line is fetched by two workgroups).  Its four waves split K: wave w takes the 32-deep K
// steps w, w+4, w+8, ...  Each wave owns a private 4-slot LDS ring and copies
// its next steps straight from global memory into LDS (global_load_lds_dwordx4,
// lane l's 16 bytes land at base + 16*l), three steps ahead of the one it
// multiplies.  Because every wave only ever reads what it copied itself, the
// main loop needs no workgroup barrier: a wave waits for its own copies with
// vmcnt and proceeds.  At the end the four partial tiles are summed through
// LDS in a fixed order (deterministic) and the epilogue applies alpha/beta and
// rounds once.
//
// Operands.  X rows (K-contiguous) are copied as 64-byte rows; their 16-byte
// chunks are swizzled by ((r>>1) ^ (r>>2)) & 3 so that 16 lanes reading one
// chunk column hit distinct banks.  W rows (N-contiguous) are copied as
// BN*2-byte rows, chunk c of row k in slot c ^ f(k); fragments of W^T come
// out of ds_read_b64_tr_b16 (the transpose happens in the LDS read).  The
// contraction is v_mfma_f32_16x16x32 with W^T as the first operand, so the
// accumulator holds C^T blocks: lane l has C(m = l%16, n = 4(l/16)+0..3).
// Rows of X past M are read from row M-1 (their results are never stored).
#include "common.h"

namespace mgemm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#ifndef MGEMM_SKINNY_SLOTS
#define MGEMM_SKINNY_SLOTS 4
#endif
#ifndef MGEMM_SKINNY_BN
#define MGEMM_SKINNY_BN 64
#endif
constexpr int NW = 4, NT = 256, KS = 32;
constexpr int SLOTS = MGEMM_SKINNY_SLOTS, AHEAD = SLOTS - 1;   // steps in flight per wave

template <int DT>
__device__ __forceinline__ f32x4 mfma16(i32x4 a, i32x4 b, f32x4 c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Wait until at most n (<= K) steps of L copies each are still in flight.
template <int L, int K>
__device__ __forceinline__ void wait_steps(int n) {
    if constexpr (K == 0) {
        wait_vm<0>();
    } else {
        if (n >= K) wait_vm<K * L>();
        else wait_steps<L, K - 1>(n);
    }
}

__device__ __forceinline__ int x_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
template <int BN>
__device__ __forceinline__ int w_swz(int k) {
    if constexpr (BN == 64) return 2 * ((k & 3) ^ ((k >> 3) & 1));
    else return 2 * (((k >> 1) & 1) ^ ((k >> 3) & 1));
}

template <int DT, int MT, int BN>
__global__ __launch_bounds__(NT, (BN == 32 ? 2 : 1)) void k_skinny(Problem p) {
    constexpr int W_ROW = BN * 2;                 // bytes per K row of the W slot
    constexpr int W_BYTES = KS * W_ROW;
    constexpr int X_BYTES = MT * KS * 2;
    constexpr int SLOT = W_BYTES + X_BYTES;
    constexpr int RING = SLOTS * SLOT;            // per wave
    constexpr int W_RPI = 1024 / W_ROW;           // W rows per 1 KiB copy
    constexpr int W_CPR = W_ROW / 16;             // 16-byte chunks per W row
    constexpr int W_COPIES = KS / W_RPI;
    constexpr int X_COPIES = MT / 16;
    constexpr int LOADS = W_COPIES + X_COPIES;    // copies per step per wave
    constexpr int MB = MT / 16, NB = BN / 16;
    static_assert(NW * MT * BN * 4 <= NW * RING, "reduction buffer must fit in the rings");

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Column blocks in XCD-major order: blocks that split one 128-byte line
    // of W run on the same XCD and share its L2.
    int tmi, tni;
    tile_of_block(blockIdx.x, gridDim.x, 1, gridDim.x, 1, tmi, tni);
    const int64_t n0 = (int64_t)tni * BN;
    const int nlim = (int)(p.N - n0 < BN ? p.N - n0 : BN);
    const int M = (int)p.M;
    const uint16_t* __restrict__ X = (const uint16_t*)p.A;   // K-contiguous
    const uint16_t* __restrict__ Wt = (const uint16_t*)p.B;  // N-contiguous

    // Per-lane copy sources (K offset added per step).
    const uint16_t* w_src[W_COPIES];
#pragma unroll
    for (int i = 0; i < W_COPIES; ++i) {
        const int k = i * W_RPI + lane / W_CPR;
        int c = (lane % W_CPR) ^ w_swz<BN>(k);
        const int cmax = (nlim >> 3) - 1;
        c = c <= cmax ? c : cmax;
        w_src[i] = Wt + (int64_t)k * p.ldb + n0 + 8 * c;
    }
    const uint16_t* x_src[X_COPIES];
#pragma unroll
    for (int i = 0; i < X_COPIES; ++i) {
        const int r = 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ x_swz(r);
        const int rr = r < M ? r : M - 1;
        x_src[i] = X + (int64_t)rr * p.lda + 8 * c;
    }
    const int64_t w_kstep = (int64_t)KS * p.ldb;

    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    const unsigned ring = lds0 + (unsigned)w * RING;
    auto issue = [&](int64_t s, int slot) {
        const unsigned base = ring + (unsigned)slot * SLOT;
#pragma unroll
        for (int i = 0; i < W_COPIES; ++i) copy_to_lds(w_src[i] + s * w_kstep, base + i * 1024);
#pragma unroll
        for (int i = 0; i < X_COPIES; ++i) copy_to_lds(x_src[i] + s * KS, base + W_BYTES + i * 1024);
    };

    // Per-lane LDS read offsets within a slot.
    int x_off[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = 16 * mb + (lane & 15), c = lane >> 4;
        x_off[mb] = W_BYTES + r * 64 + ((c ^ x_swz(r)) << 4);
    }
    int w_off[NB][2];
    {
        const int q = lane >> 4, t = lane & 15;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = 8 * q + 4 * h + (t >> 2);
                const int n = 16 * nb + 4 * (t & 3);
                w_off[nb][h] = k * W_ROW + (((n >> 3) ^ w_swz<BN>(k)) << 4) + ((n & 7) << 1);
            }
    }

    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t nk = p.K / KS;
    const int64_t mine = nk > w ? (nk - w + NW - 1) / NW : 0;   // steps w, w+NW, ...
    for (int64_t i = 0; i < mine && i < AHEAD; ++i) issue(w + i * NW, (int)i);

    const unsigned char* lring = smem + w * RING;
    for (int64_t i = 0; i < mine; ++i) {
        // Own copies of step i complete (newer ones may stay in flight).
        const int64_t newer = (i + AHEAD - 1 < mine - 1 ? i + AHEAD - 1 : mine - 1) - i;
        wait_steps<LOADS, AHEAD - 1>((int)newer);
        asm volatile("" ::: "memory");
        const unsigned char* base = lring + (int)(i % SLOTS) * SLOT;
        i32x4 xf[MB], wf[NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[mb] = *(const i32x4*)(base + x_off[mb]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(base + w_off[nb][0]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(base + w_off[nb][1]));
            const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
            wf[nb] = i32x4{l2.x, l2.y, h2.x, h2.y};
        }
        // The next copy reuses the slot read one step ago; that step's LDS
        // reads have completed (its MFMAs consumed them).
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this step's reads done
        asm volatile("" ::: "memory");
        if (i + AHEAD < mine) issue(w + (i + AHEAD) * NW, (int)((i + AHEAD) % SLOTS));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma16<DT>(wf[nb], xf[mb], acc[mb][nb]);
    }

    // ---- cross-wave reduction in a fixed order, then the epilogue ----------
    wait_vm<0>();
    __syncthreads();
    float* red = (float*)smem;                         // [NW][MT][BN]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int m = 16 * mb + (lane & 15), n = 16 * nb + 4 * (lane >> 4);
            *(f32x4*)(red + (w * MT + m) * BN + n) = acc[mb][nb];
        }
    __syncthreads();
    uint16_t* C = (uint16_t*)p.C;
    with_epilogue(p.epilogue, [&](auto E) {
        constexpr int EPI = decltype(E)::value;
        for (int e = tid * 4; e < MT * BN; e += NT * 4) {
            const int m = e / BN, n = e % BN;
            if (m >= M) continue;
            f32x4 s = *(const f32x4*)(red + m * BN + n);
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) {
                const f32x4 t = *(const f32x4*)(red + (ww * MT + m) * BN + n);
                s = s + t;
            }
            uint16_t* crow = C + (int64_t)m * p.ldc + n0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (n + q >= nlim) break;
                float v = p.alpha * s[q];
                if (p.beta != 0.f) v = fmaf(p.beta, from_bits<DT>(crow[n + q]), v);
                crow[n + q] = to_bits<DT>(epilogue_op<DT, EPI>(v));
            }
        }
    });
}

template <int DT, int MT, int BN>
hipError_t launch_cfg(const Problem& p, hipStream_t s) {
    auto kern = k_skinny<DT, MT, BN>;
    constexpr int SLOT = KS * BN * 2 + MT * KS * 2;
    const size_t lds = (size_t)NW * SLOTS * SLOT;
    static bool attr_set[MAX_DEVICES] = {};
    if (hipError_t e = set_lds_limit_once((const void*)kern, (int)lds, attr_set); e != hipSuccess)
        return e;
    const int64_t blocks = (p.N + BN - 1) / BN;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NT), lds, s, p);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const Problem& p, hipStream_t s) {
    if (p.M <= 16) return launch_cfg<DT, 16, MGEMM_SKINNY_BN>(p, s);
    if (p.M <= 32) return launch_cfg<DT, 32, MGEMM_SKINNY_BN>(p, s);
    return launch_cfg<DT, 64, MGEMM_SKINNY_BN>(p, s);
}

}  // namespace

bool skinny_supports(const Problem& p) {
    if (p.dtype != F16 && p.dtype != BF16) return false;
    if (!p.a_kc || p.b_kc) return false;
    if (p.M < 1 || p.M > 64 || p.K <= 0 || p.K % KS != 0 || p.N % 8 != 0) return false;
    if (p.lda % 8 != 0 || p.ldb % 8 != 0) return false;
    if (((uintptr_t)p.A & 15) != 0 || ((uintptr_t)p.B & 15) != 0) return false;
    return (p.N + 31) / 32 <= 0x7fffffff;
}

hipError_t launch_skinny(const Problem& p, hipStream_t s) {
    return p.dtype == F16 ? launch_dt<F16>(p, s) : launch_dt<BF16>(p, s);
}

}  // namespace mgemm
