// FP16/BF16 GEMM for gfx950, "ping-pong" schedule: the fast path for the
// canonical NN problem (A' K-contiguous, B' N-contiguous) on large shapes.
//
// Why a second kernel.  With one wave per SIMD (the register-staged kernel in
// k_h_mfma.hip) every SIMD stalls on its own memory phase -- waiting for the
// global loads, writing them to LDS, the workgroup barrier, the first LDS
// reads of the next slice -- and the matrix core idles meanwhile.  Here a
// 512-thread workgroup runs two groups of four waves, one wave of each group
// per SIMD.  The groups are offset by one phase: while group 0 issues its
// MFMAs, group 1 issues loads and reads its next fragments from LDS, and then
// they swap, separated by workgroup barriers.  The matrix core of each SIMD
// is fed by one of its two waves at all times.
//
// Prior art on the pages, as before: large output tiles (MTT S4000 write-up,
// sections 1 and 15), overlapped data movement and compute in a multi-slot
// buffer (Chapter 5 "Operators and Runtime", section 5.3.2: with more slots
// the mover can start n-1 blocks early), bank-spreading layouts (Chapter 5,
// section 5.2.3, here an XOR swizzle since the copy engine cannot pad),
// XCD-aware M-grouped tile order (common.h).
//
// Data movement.  Global memory is copied straight into LDS with
// global_load_lds_dwordx4: each lane moves 16 bytes and lane l lands at
// base + 16*l, so the LDS layout is chosen by which global chunk each lane
// fetches.  Four LDS slots of one K=32 slice each (16 KiB of A, 16 KiB of B)
// form a ring; slice j+3 is requested while slice j is read.
//   A slice (256 rows x 32 K, K-contiguous rows of 64 B): the 16-byte chunk c
//   of row r sits in slot c ^ (((r>>1) ^ (r>>2)) & 3) of its row.
//   B slice (32 K rows x 256 N, N-contiguous rows of 512 B): chunk c of row k
//   sits in slot c ^ {0,6,10,12}[k&3].
// Both swizzles keep every operand read free of bank conflicts whether the LDS
// serves 128 or 256 bytes per clock.
//
// Operand fetch.  An A fragment (32 rows x 16 K) is one ds_read_b128 per lane.
// A B fragment (16 K x 32 N) comes from the N-contiguous slice through two
// ds_read_b64_tr_b16: within each 16-lane group, lane t reads 4 consecutive N
// of row k0 + t/4 and the instruction hands lane i the 4 K values of column
// i, i.e. the transpose, so B is never transposed in memory or registers.
//
// Restrictions (the host checks them, else the general-purpose kernels run):
// A' K-contiguous, B' N-contiguous, K % 32 == 0, N % 8 == 0, lda and ldb
// multiples of 8 and 16-byte aligned bases.  Rows past M and columns past N
// of an edge tile are read from the last valid row/chunk (their results are
// discarded by the masked store).
#include "common.h"

namespace mgemm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 32, NT = 512, SLOTS = 4, AHEAD = 3;
constexpr int A_ROW = BK * 2;                       // bytes per A row in LDS
constexpr int B_ROW = BN * 2;                       // bytes per B row in LDS
constexpr int A_BYTES = BM * A_ROW;                 // 16 KiB
constexpr int B_BYTES = BK * B_ROW;                 // 16 KiB
constexpr int SLOT_BYTES = A_BYTES + B_BYTES;       // 32 KiB
constexpr int LOADS_PER_SLICE = 4;                  // direct loads per wave per slice
constexpr int TM = 2, TN = 4;                       // 32x32 blocks per wave (64 x 128)

__device__ __forceinline__ int a_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int b_swz(int k) { return (0xCA60 >> ((k & 3) * 4)) & 15; }

template <int DT>
__device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <int DT>
__device__ __forceinline__ uint16_t to_bits(float v) {
    if constexpr (DT == F16) return f32_to_f16_bits(v);
    else return f32_to_bf16_bits(v);
}
template <int DT>
__device__ __forceinline__ float from_bits(uint16_t b) {
    if constexpr (DT == F16) return f16_bits_to_f32(b);
    else return bf16_bits_to_f32(b);
}

// s_waitcnt with only the vector-memory counter constrained (vmcnt <= n).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vm_dyn(int n) {
    // n is wave-uniform and small; pick the immediate.
    if (n <= 0) wait_vm<0>();
    else if (n <= LOADS_PER_SLICE) wait_vm<LOADS_PER_SLICE>();
    else wait_vm<2 * LOADS_PER_SLICE>();
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }  // lgkmcnt(0)

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane l's
// 16 bytes from `src` land at LDS byte address lds + 16*l.  Issued through
// inline asm so the compiler does not treat the LDS reads that follow as
// dependent on it: completion is tracked by hand with the vmcnt waits of the
// schedule below.
__device__ __forceinline__ void copy_to_lds(const void* src, unsigned lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(lds) : "memory", "m0");
}

// Workgroup barrier that neither the compiler nor the scheduler may move
// memory accesses or instructions across.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int DT>
__global__ __launch_bounds__(NT, 1) void k_h_pp(Problem p) {
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave >> 2;            // phase group
    const int wi = wave & 3;            // wave within group
    const int wm = wi >> 1, wn = wi & 1;

    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
    int tmi, tni;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, 8, tmi, tni);
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const int mlim = (int)(p.M - m0 < BM ? p.M - m0 : BM);
    const int nlim = (int)(p.N - n0 < BN ? p.N - n0 : BN);

    const uint16_t* __restrict__ A = (const uint16_t*)p.A;
    const uint16_t* __restrict__ B = (const uint16_t*)p.B;

    // ---- per-lane global sources for this wave's share of a slice --------
    // A: group g covers rows [128g, 128g+128): 8 copies of 16 rows; this wave
    // does copies 2wi and 2wi+1.  Lane l: row 16*copy + l/4, slot l%4.
    const uint16_t* a_src[2];
    int a_dst[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int copy = 2 * wi + i;
        const int r = 128 * g + 16 * copy + (lane >> 2);
        const int c = (lane & 3) ^ a_swz(r);
        const int rr = r < mlim ? r : mlim - 1;
        a_src[i] = A + (m0 + rr) * p.lda + 8 * c;
        a_dst[i] = (128 * g + 16 * copy) * A_ROW;               // wave-uniform
    }
    // B: group g covers K rows [16g, 16g+16): 8 copies of 2 rows.  Lane l:
    // row 2*copy + l/32, slot l%32.
    const uint16_t* b_src[2];
    int b_dst[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int copy = 2 * wi + i;
        const int k = 16 * g + 2 * copy + (lane >> 5);
        int c = (lane & 31) ^ b_swz(k);
        const int cmax = (nlim >> 3) - 1;
        c = c <= cmax ? c : cmax;
        b_src[i] = B + (int64_t)k * p.ldb + n0 + 8 * c;
        b_dst[i] = A_BYTES + (16 * g + 2 * copy) * B_ROW;
    }
    const int64_t b_kstep = (int64_t)BK * p.ldb;

    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    auto issue = [&](int64_t s) {
        const unsigned base = lds0 + (unsigned)(s % SLOTS) * SLOT_BYTES;
#pragma unroll
        for (int i = 0; i < 2; ++i) copy_to_lds(a_src[i] + s * BK, base + a_dst[i]);
#pragma unroll
        for (int i = 0; i < 2; ++i) copy_to_lds(b_src[i] + s * b_kstep, base + b_dst[i]);
    };

    // ---- per-lane LDS read offsets (relative to a slot) -------------------
    int a_off[TM][2];                   // [tm][ks]
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int r = 128 * g + 64 * wm + 32 * tm + (lane & 31);
            const int c = 2 * ks + (lane >> 5);
            a_off[tm][ks] = r * A_ROW + ((c ^ a_swz(r)) << 4);
        }
    int b_off[TN][2][2];                // [tn][ks][half]
    {
        const int q = lane >> 4, t = lane & 15;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = ks * 16 + 8 * (q >> 1) + 4 * h + (t >> 2);
                    const int n = 128 * wn + 32 * tn + 16 * (q & 1) + 4 * (t & 3);
                    const int c = n >> 3;
                    b_off[tn][ks][h] = A_BYTES + k * B_ROW + ((c ^ b_swz(k)) << 4) + ((n & 7) << 1);
                }
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    const int64_t nk = p.K / BK;

    // ---- prologue: slices 0..2 requested, slice 0 complete everywhere ----
    const int64_t npro = nk < AHEAD ? nk : AHEAD;
    for (int64_t s = 0; s < npro; ++s) issue(s);
    wait_vm_dyn((int)(npro - 1) * LOADS_PER_SLICE);
    phase_barrier();
    if (g == 1) phase_barrier();        // group 1 runs one phase behind

    i32x4 af[TM][2];
    i32x4 bf[TN][2];
    for (int64_t j = 0; j < nk; ++j) {
        // ---- memory phase: request slice j+3, finish own part of j+1, read slice j
        if (j + AHEAD < nk) issue(j + AHEAD);
        {
            const int64_t last = (j + AHEAD < nk ? j + AHEAD : nk - 1);
            const int64_t inflight_after_next = last - (j + 1);   // slices newer than j+1
            wait_vm_dyn((int)(inflight_after_next > 0 ? inflight_after_next : 0) * LOADS_PER_SLICE);
        }
        const unsigned char* base = smem + (int)(j % SLOTS) * SLOT_BYTES;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) af[tm][ks] = *(const i32x4*)(base + a_off[tm][ks]);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4*)(base + b_off[tn][ks][0]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4*)(base + b_off[tn][ks][1]));
                const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
                bf[tn][ks] = i32x4{l2.x, l2.y, h2.x, h2.y};
            }
        }
        wait_lds();
        phase_barrier();
        // ---- compute phase
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = mfma<DT>(bf[tn][ks], af[tm][ks], acc[tm][tn]);
        __builtin_amdgcn_s_setprio(0);
        phase_barrier();
    }
    if (g == 0) phase_barrier();        // balance the offset barrier

    // ---- epilogue: lane holds C(m, n..n+3), m = row of the 32x32 block -------
    uint16_t* C = (uint16_t*)p.C;
    const bool vec_ok = (p.ldc % 4 == 0) && (((uintptr_t)p.C & 7) == 0);
    const int fr = lane & 31, nq = 4 * (lane >> 5);
    with_epilogue(p.epilogue, [&](auto E) {
        constexpr int EPI = decltype(E)::value;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int mi = 128 * g + 64 * wm + 32 * tm + fr;
            if (mi >= mlim) continue;
            uint16_t* crow = C + (m0 + mi) * p.ldc + n0;
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ni = 128 * wn + 32 * tn + 8 * q + nq;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = p.alpha * acc[tm][tn][4 * q + e];
                    store_out4<DT, EPI>(crow, ni, nlim, vec_ok, p.beta, v);
                }
            }
        }
    });
}

template <int DT>
hipError_t launch_dt(const Problem& p, hipStream_t s) {
    auto kern = k_h_pp<DT>;
    const size_t lds = (size_t)SLOTS * SLOT_BYTES;
    static bool attr_set[MAX_DEVICES] = {};
    if (hipError_t e = set_lds_limit_once((const void*)kern, (int)lds, attr_set); e != hipSuccess)
        return e;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(NT), lds, s, p);
    return hipGetLastError();
}

}  // namespace

bool h_pp_supports(const Problem& p) {
    if (p.dtype != F16 && p.dtype != BF16) return false;
    if (!p.a_kc || p.b_kc) return false;
    if (p.K <= 0 || p.K % BK != 0 || p.N % 8 != 0) return false;
    if (p.lda % 8 != 0 || p.ldb % 8 != 0) return false;
    if (((uintptr_t)p.A & 15) != 0 || ((uintptr_t)p.B & 15) != 0) return false;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    return tiles > 0 && tiles <= 0x7fffffff;
}

hipError_t launch_h_pp(const Problem& p, hipStream_t s) {
    return p.dtype == F16 ? launch_dt<F16>(p, s) : launch_dt<BF16>(p, s);
}

}  // namespace mgemm
