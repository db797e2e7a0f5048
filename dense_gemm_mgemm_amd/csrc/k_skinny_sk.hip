// Skinny-M FP16/BF16 GEMM (M <= 64) with K split across workgroups:
// C[M x N] = X[M x K] * W[K x N], W N-contiguous (or, in the BKC form below,
// K-contiguous: weights stored out x in), read once from HBM.
//
// Why a second skinny kernel.  Streaming W as 128-byte row segments (one
// 64-column block per workgroup over the whole K range) reaches only about
// 4.2 TB/s on MI355X even with no arithmetic at all; 512-byte segments with
// the K range split over four workgroups reach about 5.1 TB/s (measured with
// copy-only kernels of both shapes).  So each workgroup here owns 256 columns
// (512-byte segments) and one of `ksplit` contiguous K ranges, which also
// cuts the re-reads of X by four against 64-column blocks.
//
// Work split.  256 threads; wave w computes columns [64w, 64w+64) of the
// block for all M rows, so the waves need no reduction among themselves.  K
// is walked in 32-row steps through a four-slot LDS ring shared by the
// workgroup: the waves copy each step straight from global memory into LDS
// (global_load_lds_dwordx4, lane l's 16 bytes land at base + 16*l; W: sixteen
// 1 KiB copies of two 512-byte rows, four per wave; X: one 1 KiB copy of 16
// rows per 16 rows of M, by waves 0..M/16-1).  Step i+4 is requested into
// slot i%4 once every wave has read step i (one barrier per step), so four
// steps are in flight per workgroup.
//
// Split-K reduction (deterministic, no atomics on data).  With ksplit > 1
// every workgroup stores its FP32 partial block (rows < M) to a workspace
// owned by the handle with device-coherent stores, waits for them to
// complete, and bumps the block's arrival counter with a device-scope atomic.
// The workgroup that arrives last reads the other partials with
// device-coherent loads and adds them in split order 0, 1, ..., ksplit-1,
// whatever the arrival order, so the result does not depend on timing; it
// then applies alpha and beta, rounds once, stores C and resets the counter
// to zero for the next call.  Nobody waits for anybody: a workgroup that is
// not last simply exits.  (Release/acquire fences would do the same job but
// write back and invalidate whole L2s; measured, they doubled the run time.)
// This is the fixed-order split-K reduction that "Chapter 5: Operators and
// Runtime" (section 5.2.4) asks for in place of atomically accumulated
// outputs.
//
// Operands and fragments as in k_skinny.hip: v_mfma_f32_16x16x32 with W^T
// as the first operand (fragments from ds_read_b64_tr_b16), X rows as the
// second (ds_read_b128); lane l ends up holding C(m = l%16, n = 4(l/16)+0..3)
// of each 16x16 block.  W rows are 512 bytes; chunk c of row k sits at chunk
// position c ^ f(k), f(k) = {0,6,10,12}[k&3] ^ 8*((k>>3)&1), which keeps every
// transposed read free of bank conflicts.  Rows of X past M are read from row
// M-1 and columns of W past N from the last valid chunk; neither is stored.
#include "common.h"

namespace mgemm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256, BNS = 256, KS = 32, SLOTS = 4;
constexpr int W_ROW = BNS * 2, W_BYTES = KS * W_ROW;   // 512 B rows, 16 KiB per step

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
__device__ __forceinline__ void fence_sched() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ int x_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int w_swz(int k) {
    return ((0xCA60 >> ((k & 3) * 4)) & 15) ^ (8 * ((k >> 3) & 1));
}

struct SplitArgs {
    float* part;        // [blocks][ksplit][MT][256] FP32 partials (ksplit > 1)
    int part_bytes;     // workspace size (bounds the buffer accesses)
    unsigned* cnt;      // [blocks] arrival counters, zero between calls
    int ksplit;         // K ranges per column block
    int per;            // K steps per range (the last range may be shorter)
};

// BKC: W' K-contiguous (weights stored out x in, C = X W^T).  The W slot then
// holds the block's 256 columns as rows of 64 bytes (32 K-values each), copied
// 16 rows per 1 KiB copy with the XOR swizzle ((r>>1) ^ (r>>2)) & 3 on the
// four 16-byte chunks of row r, and each fragment is one ds_read_b128 (lane l:
// column 16nb + l%16 of the wave's 64, chunk l/16), which that swizzle keeps
// free of bank conflicts.
__device__ __forceinline__ int kc_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

template <int DT, int MT, bool BKC = false>
__global__ __launch_bounds__(NT, 1) void k_skinny_sk(Problem p, SplitArgs sa) {
    constexpr int MB = MT / 16;
    constexpr int X_BYTES = MT * KS * 2;
    constexpr int SLOT = W_BYTES + X_BYTES;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int last_flag;
    const ClockStamp stamp0 = clock_stamp_begin();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool has_x = w < MB;           // waves 0..MB-1 also copy X

    // Workgroup -> (column block, K range): the K ranges of one column block
    // take consecutive positions, which the workgroup numbering places on one
    // XCD, so each XCD streams whole column blocks of W over all of K (with
    // weights stored out x in: whole 8 KiB rows of W', 25.0 against 26.5 us
    // at M = 16 when the ranges of a block were spread over the XCDs).
    int tz, t;
    tile_of_block(blockIdx.x, gridDim.x, 1, gridDim.x, 1, tz, t);
    const int blk = t / sa.ksplit, split = t % sa.ksplit;
    const int64_t nk = p.K / KS;
    const int64_t s_begin = (int64_t)split * sa.per;
    const int64_t s_end = s_begin + sa.per < nk ? s_begin + sa.per : nk;
    const int nsteps = s_end > s_begin ? (int)(s_end - s_begin) : 0;

    const int64_t n0 = (int64_t)blk * BNS;
    const int nlim = (int)(p.N - n0 < BNS ? p.N - n0 : BNS);
    const int M = (int)p.M;
    const uint16_t* __restrict__ X = (const uint16_t*)p.A;    // K-contiguous
    const uint16_t* __restrict__ Wt = (const uint16_t*)p.B;   // N-contiguous

    // Copy sources at the first step of the range; step s adds s*KS rows.
    const uint16_t* w_src[4];
    int w_dst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * w + i;
        if constexpr (BKC) {                         // copy j: columns 16j .. 16j+15
            const int r = 16 * j + (lane >> 2);
            const int c = (lane & 3) ^ kc_swz(r);
            const int rr = r < nlim ? r : nlim - 1;  // columns past N: the last valid one
            w_src[i] = Wt + (n0 + rr) * p.ldb + s_begin * KS + 8 * c;
        } else {                                     // copy j: rows 2j, 2j+1 of the step
            const int k = 2 * j + (lane >> 5);
            int c = (lane & 31) ^ w_swz(k);
            const int cmax = (nlim >> 3) - 1;
            c = c <= cmax ? c : cmax;
            w_src[i] = Wt + (s_begin * KS + k) * p.ldb + n0 + 8 * c;
        }
        w_dst[i] = j * 1024;
    }
    const uint16_t* x_src;
    {
        const int r = 16 * (has_x ? w : 0) + (lane >> 2);
        const int c = (lane & 3) ^ x_swz(r);
        const int rr = r < M ? r : M - 1;
        x_src = X + (int64_t)rr * p.lda + s_begin * KS + 8 * c;
    }
    const int x_dst = W_BYTES + (has_x ? w : 0) * 1024;
    const int64_t w_step = BKC ? (int64_t)KS : (int64_t)KS * p.ldb;

    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    auto issue = [&](int s) {
        const unsigned base = lds0 + (unsigned)(s % SLOTS) * SLOT;
#pragma unroll
        for (int i = 0; i < 4; ++i) copy_to_lds(w_src[i] + (int64_t)s * w_step, base + w_dst[i]);
        if (has_x) copy_to_lds(x_src + (int64_t)s * KS, base + x_dst);
    };
    auto wait_own = [&](int n) {        // at most n of this wave's steps in flight
        if (has_x) wait_steps<5, SLOTS - 1>(n);
        else wait_steps<4, SLOTS - 1>(n);
    };

    // Fragment read offsets within a slot.
    int x_off[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = 16 * mb + (lane & 15), c = lane >> 4;
        x_off[mb] = W_BYTES + r * 64 + ((c ^ x_swz(r)) << 4);
    }
    int w_off[4][2];
    if constexpr (BKC) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int r = 64 * w + 16 * nb + (lane & 15), c = lane >> 4;
            w_off[nb][0] = r * 64 + ((c ^ kc_swz(r)) << 4);
            w_off[nb][1] = 0;
        }
    } else {
        const int q = lane >> 4, tt = lane & 15;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = 8 * q + 4 * h + (tt >> 2);
                const int n = 64 * w + 16 * nb + 4 * (tt & 3);
                w_off[nb][h] = k * W_ROW + (((n >> 3) ^ w_swz(k)) << 4) + ((n & 7) << 1);
            }
    }

    f32x4 acc[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int npro = nsteps < SLOTS ? nsteps : SLOTS;
    for (int s = 0; s < npro; ++s) issue(s);
    if (nsteps > 0) {
        wait_own(npro - 1);
        fence_sched();
        __syncthreads();
        fence_sched();
    }
    for (int i = 0; i < nsteps; ++i) {
        const unsigned char* base = smem + (i % SLOTS) * SLOT;
        i32x4 xf[MB], wf[4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[mb] = *(const i32x4*)(base + x_off[mb]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            if constexpr (BKC) {
                wf[nb] = *(const i32x4*)(base + w_off[nb][0]);
                continue;
            }
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(base + w_off[nb][0]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(base + w_off[nb][1]));
            const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
            wf[nb] = i32x4{l2.x, l2.y, h2.x, h2.y};
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this step's reads are done
        if (i + 1 < nsteps) {
            // Own copies of step i+1 landed (later ones may stay in flight),
            // then every wave's: step i+1 is visible and slot i is free.
            const int last_issued = i + SLOTS - 1 < nsteps - 1 ? i + SLOTS - 1 : nsteps - 1;
            wait_own(last_issued - (i + 1));
            fence_sched();
            __syncthreads();
            fence_sched();
            if (i + SLOTS < nsteps) issue(i + SLOTS);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma16<DT>(wf[nb], xf[mb], acc[mb][nb]);
    }

    // ---- regroup the block through LDS, row by row ---------------------------
    // red[m][n] holds row m of the block (RED_LD pads the rows against bank
    // conflicts).  From here on wave w owns rows w, w+4, ... < M, which move
    // as whole rows: 1 KiB of FP32 per row, 16 bytes per lane.  The row loops
    // stay rolled: this code runs once per workgroup, and unrolled copies of
    // it would mostly cost instruction-cache misses.
    constexpr int RED_LD = BNS + 4;
    static_assert(MT * RED_LD * 4 <= SLOT * SLOTS, "regroup buffer must fit in the ring");
    float* red = (float*)smem;
    __syncthreads();                         // every wave is done with the ring
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int m = 16 * mb + (lane & 15), n = 64 * w + 16 * nb + 4 * (lane >> 4);
            *(f32x4*)(red + m * RED_LD + n) = acc[mb][nb];
        }
    __syncthreads();
    const int n = 4 * lane;

    // ---- split-K reduction -------------------------------------------------
    if (sa.ksplit > 1) {
        // Publish this range's partial rows with device-coherent stores, wait
        // for them to complete, then count the arrival.
        const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(sa.part, 0, sa.part_bytes, 0x00020000);
        const unsigned blk_off = (unsigned)blk * (unsigned)sa.ksplit * (MT * BNS * 4);
        auto part_off = [&](int sp, int m) {
            return blk_off + (unsigned)(sp * (MT * BNS) + m * BNS + n) * 4;
        };
        for (int m = w; m < M; m += 4)
            store_coherent(ws, part_off(split, m), *(const f32x4*)(red + m * RED_LD + n));
        wait_vm<0>();
        __syncthreads();
        if (tid == 0) {
            const unsigned old = __hip_atomic_fetch_add(sa.cnt + blk, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            last_flag = old == (unsigned)(sa.ksplit - 1);
        }
        __syncthreads();
        if (!last_flag) {
            clock_stamp_end(p, stamp0);
            return;
        }
        if (tid == 0) sa.cnt[blk] = 0u;
        // Last arrival: every partial of the block is complete.  Each row is
        // summed over ranges 0, 1, ..., ksplit-1 in that order (own range from
        // LDS) and the sum replaces the row in LDS.
        if (sa.ksplit <= 4) {
            // One round: the (up to three) other ranges of all this wave's
            // rows are in flight together; the own range is slotted in at
            // position `split` of the sum.
            constexpr int RW = MT / 4;
            f32x4 v[RW][3];
#pragma unroll
            for (int g = 0; g < RW; ++g)
#pragma unroll
                for (int c = 0; c < 3; ++c) {
                    const int m = w + 4 * g, sp = c < split ? c : c + 1;
                    v[g][c] = (m < M && sp < sa.ksplit) ? load_coherent(ws, part_off(sp, m))
                                                        : f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int g = 0; g < RW; ++g) {
                const int m = w + 4 * g;
                if (m >= M) break;
                f32x4* row = (f32x4*)(red + m * RED_LD + n);
                const f32x4 mine = *row;
                f32x4 tot = split == 0 ? mine : v[g][0];
#pragma unroll
                for (int pos = 1; pos < 4; ++pos) {
                    if (pos >= sa.ksplit) break;
                    tot = tot + (pos == split ? mine
                                 : (pos < split ? v[g][pos < 3 ? pos : 2] : v[g][pos - 1]));
                }
                *row = tot;
            }
        } else {
            // More ranges: groups of RG rows, rounds of SPC ranges; the
            // RG*SPC loads of a round are in flight together, and each row
            // keeps its sum in range order.
            constexpr int SPC = 4, RG = 4;
            for (int m0r = w; m0r < M; m0r += 4 * RG) {
                f32x4 mine[RG], tot[RG];
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const int m = m0r + 4 * g;
                    mine[g] = m < M ? *(const f32x4*)(red + m * RED_LD + n) : f32x4{0.f, 0.f, 0.f, 0.f};
                    tot[g] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                for (int sp0 = 0; sp0 < sa.ksplit; sp0 += SPC) {
                    f32x4 v[RG][SPC];
#pragma unroll
                    for (int g = 0; g < RG; ++g)
#pragma unroll
                        for (int c = 0; c < SPC; ++c) {
                            const int m = m0r + 4 * g, sp = sp0 + c;
                            v[g][c] = (m < M && sp < sa.ksplit && sp != split)
                                          ? load_coherent(ws, part_off(sp, m)) : mine[g];
                        }
#pragma unroll
                    for (int g = 0; g < RG; ++g)
#pragma unroll
                        for (int c = 0; c < SPC; ++c) {
                            const int sp = sp0 + c;
                            if (sp == 0) tot[g] = v[g][c];
                            else if (sp < sa.ksplit) tot[g] = tot[g] + v[g][c];
                        }
                }
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    const int m = m0r + 4 * g;
                    if (m < M) *(f32x4*)(red + m * RED_LD + n) = tot[g];
                }
            }
        }
    }

    // ---- epilogue: alpha, beta, one rounding, row-contiguous stores ----------
    uint16_t* C = (uint16_t*)p.C;
    const bool vec_ok = (p.ldc % 4 == 0) && (((uintptr_t)p.C & 7) == 0);
    if (n >= nlim) return;              // never thread 0: n = 0 < nlim
    with_epilogue(p.epilogue, [&](auto E) {
        constexpr int EPI = decltype(E)::value;
        for (int m = w; m < M; m += 4) {
            const f32x4 tot = *(const f32x4*)(red + m * RED_LD + n);
            uint16_t* crow = C + (int64_t)m * p.ldc + n0;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = p.alpha * tot[e];
            store_out4<DT, EPI>(crow, n, nlim, vec_ok, p.beta, v);
        }
    });
    clock_stamp_end(p, stamp0);
}

template <int DT, int MT, bool BKC>
hipError_t launch_cfg(const Problem& p, const SplitArgs& sa, int64_t grid, hipStream_t s) {
    auto kern = k_skinny_sk<DT, MT, BKC>;
    const size_t lds = (size_t)SLOTS * (W_BYTES + MT * KS * 2);
    static bool attr_set[MAX_DEVICES] = {};
    if (hipError_t e = set_lds_limit_once((const void*)kern, (int)lds, attr_set); e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, s, p, sa);
    return hipGetLastError();
}

template <int DT, bool BKC>
hipError_t launch_mt(const Problem& p, const SplitArgs& sa, int64_t grid, hipStream_t s) {
    if (p.M <= 16) return launch_cfg<DT, 16, BKC>(p, sa, grid, s);
    if (p.M <= 32) return launch_cfg<DT, 32, BKC>(p, sa, grid, s);
    return launch_cfg<DT, 64, BKC>(p, sa, grid, s);
}
template <int DT>
hipError_t launch_dt(const Problem& p, const SplitArgs& sa, int64_t grid, hipStream_t s) {
    return p.b_kc ? launch_mt<DT, true>(p, sa, grid, s) : launch_mt<DT, false>(p, sa, grid, s);
}

int mt_of(int64_t M) { return M <= 16 ? 16 : (M <= 32 ? 32 : 64); }

}  // namespace

bool skinny_sk_supports(const Problem& p) {
    if (p.dtype != F16 && p.dtype != BF16) return false;
    if (!p.a_kc) return false;
    // N-contiguous W rows are read as 8-element chunks; K-contiguous W'
    // columns (b_kc) as 32-element K slices.
    if (p.M < 1 || p.M > 64 || p.K <= 0 || p.K % KS != 0 || (!p.b_kc && p.N % 8 != 0)) return false;
    if (p.lda % 8 != 0 || p.ldb % 8 != 0) return false;
    if (((uintptr_t)p.A & 15) != 0 || ((uintptr_t)p.B & 15) != 0) return false;
    return (p.N + BNS - 1) / BNS <= 0x7fffffff / 64;
}

int skinny_sk_splits(const Problem& p, const Workspace& ws, int requested) {
    const int64_t blocks = (p.N + BNS - 1) / BNS;
    const int64_t nk = p.K / KS;
    const int64_t slots = p.num_cu > 0 ? p.num_cu : 256;
    const int64_t per_range = blocks * mt_of(p.M) * BNS * (int64_t)sizeof(float);
    const bool room = ws.part != nullptr && blocks <= ws.ncounters;
    int64_t ks;
    if (requested <= 0) {
        // About three workgroups for every four CUs (the copy-only
        // measurements peak there), at most 16 ranges, each of at least 8
        // steps (K = 256; shorter ranges spend more on the partial exchange
        // than they save: 64x6144x1024 took 27 us at 8 ranges of 4 steps).
        ks = (3 * slots / 4 + blocks - 1) / blocks;
        if (ks > 16) ks = 16;
        if (ks > nk / 8) ks = nk / 8;
        if (ks < 1) ks = 1;
        if (ks > 1 && (!room || ks * per_range > ws.part_bytes)) ks = 1;
    } else {
        ks = requested < nk ? requested : nk;
        if (ks > 1 && (!room || ks * per_range > ws.part_bytes)) return 0;
    }
    const int64_t per = (nk + ks - 1) / ks;
    return (int)((nk + per - 1) / per);
}

hipError_t launch_skinny_sk(const Problem& p, const Workspace& ws, int ksplit, hipStream_t s) {
    const int64_t blocks = (p.N + BNS - 1) / BNS;
    const int64_t nk = p.K / KS;
    SplitArgs sa;
    sa.ksplit = ksplit < 1 ? 1 : ksplit;
    sa.per = (int)((nk + sa.ksplit - 1) / sa.ksplit);
    sa.ksplit = (int)((nk + sa.per - 1) / sa.per);
    sa.part = (float*)ws.part;
    sa.part_bytes = (int)(ws.part_bytes < 0x7fffffff ? ws.part_bytes : 0x7fffffff);
    sa.cnt = ws.counters;
    const int64_t grid = blocks * sa.ksplit;
    return p.dtype == F16 ? launch_dt<F16>(p, sa, grid, s) : launch_dt<BF16>(p, sa, grid, s);
}

}  // namespace mgemm
