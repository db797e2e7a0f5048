// FP16/BF16 GEMM for gfx950: 256xBN output tiles (BN = 256 or 192), four
// waves of 128x(BN/2), operands copied straight into a four-slot LDS ring, one
// workgroup barrier per K slice.  The fast path for the canonical NN problem
// (A' K-contiguous, B' N-contiguous).  BN = 192 exists for grids that a
// 256-wide tile fills badly: the 1024x12288 FFN projection is 192 tiles of
// 256x256 on 256 CUs but exactly 256 tiles of 256x192.
//
// Budget that shaped it (measured on MI355X): a CU pulls about 40 B/clk from
// L2 when every CU does, and a 256x256 tile needs 32 B/clk at the matrix-core
// peak, so the tile is as large as the registers allow (each wave holds a
// 128x128 accumulator, 256 AGPRs).  ds_read_b128 reads deliver about twice the
// bytes per clock of ds_read_b64_tr_b16, and a 128x128 wave tile reads 64 B/clk
// of fragments at peak, half of what a 64x128 tile would.
//
// Schedule of slice j (K = 32 per slice, 2 MFMA K-steps "ks"):
//   1. wait until this wave's copies of slice j+1 have landed, workgroup
//      barrier: slice j+1 is now visible to every wave, and every wave is done
//      reading slice j-1, so its slot can be refilled;
//   2. request slice j+3 into that slot (1 KiB copies: four of A and BN/64
//      of B per wave);
//   3. MFMAs of (j, ks=0) while reading the (j, ks=1) fragments;
//   4. MFMAs of (j, ks=1) while reading the (j+1, ks=0) fragments.
// Fragments are read one K-step ahead of the MFMAs that use them, so the
// matrix core never waits for LDS at a slice boundary.  Within a K-step one
// instruction group follows each MFMA (the copies spread evenly, one
// fragment read after each of the first few), and the order is pinned with
// scheduling barriers: with one wave per SIMD every stall of the issuing wave
// is a stall of the matrix core, and bursts of copies or reads back up the
// memory and LDS queues (measured: 58 -> 40 cycles per 32-cycle MFMA).
// This is the two-slot pipeline of "Chapter 5: Operators and Runtime"
// (section 5.3.2) stretched to four slots, with the next slot requested n-1
// blocks ahead.
//
// Under this load the chip is power-limited: the shader clock falls from
// 2.4 GHz to about 1.5-1.9 GHz when all 256 CUs issue MFMAs, so the
// published peak is out of reach and fewer stalls partly turn into a lower
// clock.
//
// LDS layouts: A rows of 64 bytes, chunk c of row r at chunk position
// c ^ a_swz(r) with a_swz(r) = ((r >> 1) ^ (r >> 2)) & 3; B rows
// of 2*BN bytes, chunk c of K-row k at chunk position pos(c, k): for BN = 256
// c ^ {0,6,10,12}[k&3], for BN = 192 the 16-byte chunks are permuted inside
// each 128-byte group by a 16-row XOR table.  Both are free of bank conflicts
// for the transposed reads (checked exhaustively over every read of a slice).
// A 1 KiB B copy covers 64 consecutive chunk positions of the slot (two rows
// for BN = 256, 2 2/3 rows for BN = 192).  B fragments come from
// ds_read_b64_tr_b16; rows past M and columns past N of an edge tile are read
// from the last valid row/chunk and never stored.
// Split K: when a grid of tiles fills the CUs badly (the 1024x1536 share of
// the FFN projection is 32 tiles on 256 CUs), each tile's K slices are cut
// into ksplit ranges of whole slices, one workgroup per (tile, range).  Each
// workgroup stores its FP32 accumulators in the handle's workspace, in
// register order (16-byte chunks, thread-contiguous, so every store and load
// of the exchange is fully coalesced), and a second kernel on the same stream
// sums the ranges of every output in range order and applies the epilogue.
// The sum order is fixed, so results do not depend on timing; the kernel
// boundary orders the two phases, so no atomics or fences are needed.
//
// Restrictions (host-checked): A' K-contiguous, or M-contiguous with M % 8 ==
// 0 (the AMC form, with an N-contiguous B'); B' N-contiguous (N % 8 == 0) or
// K-contiguous (the BKC form); K >= 32 (a last partial slice is staged by
// ordinary loads with zeros past K), lda and ldb multiples of 8, 16-byte
// aligned bases.
#include "common.h"

namespace mgemm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Epilogue of the first split-K phase: FP32 accumulators to the workspace.
constexpr int EPI_PARTIAL = 2;
// alpha times the FP32 accumulators, stored as FP32 in C's place with C's
// leading dimension (mgemm_run_acc32): the same sums the 16-bit epilogue
// rounds once.
constexpr int EPI_ACC32 = 3;

// K-range arguments.  Without a split: ksplit = 1, nks = K / 32, part unused.
struct HSplit {
    float* part;    // [tile][range][chunk][thread] f32x4, tile = tm * tiles_n + tn
    int ksplit;     // number of K ranges
    int nks;        // 32-slices per range (the last range may hold fewer)
};
// Tile order of split launches: groups two M-tiles deep.  Each XCD holds all
// K ranges of its tiles, and a deeper group would make it stream more of A
// over the whole K (FFN share 1024x1536x4096: 24.8 us at 2, 26.2 at 8, the
// unsplit order of 8 tiles kept per range 26.0).
constexpr int SPLIT_GROUP_M = 2;
// Tile order of unsplit launches: groups four M-tiles deep (each XCD's 32
// resident tiles a 4 x 8 block).  Against groups of 8 (8 x 4 blocks), BF16
// 4096x16384x4096 483 against 604 us, 4096^3 123 against 129, the FP16
// 8192x8192x16384 problem 1.756 against 1.779 ms at a higher clock; never
// slower on the square and tall shapes tried (groups of 2: as 8; 16: 30%
// slower on the 8k problem).
constexpr int UNSPLIT_GROUP_M = 4;

#ifndef MGEMM_DMA_SLOTS
#define MGEMM_DMA_SLOTS 4
#endif
constexpr int BK = 32, NT = 256;
constexpr int SLOTS = MGEMM_DMA_SLOTS, AHEAD = SLOTS - 1;   // slices in flight
constexpr int A_ROW = BK * 2;                               // bytes per A row of a slice

// BN is the width of the B slot.  The plain GEMM lays its four waves out 2x2
// (128 rows x BN/2 columns each).  The gated pair (DUAL) fills the 192-wide
// slot with 96 columns of each of two B matrices and lays the waves out 4x1
// (64 rows x all 192 columns each), so that every wave holds the G and U
// blocks of the same outputs in matching registers.
// BMT = 128 halves the tile height for short M (the four waves then hold
// 64 x BN/2 each): a 128-row problem no longer pays for 256 rows of MFMA work.
// BMT = 64 (four waves of 32 x BN/2) is for 32 < M <= 64, where the product
// streams B from HBM and half of a 128-row tile's rows would be padding.
template <int BN, bool DUAL, int BMT = 256>
struct Cfg {
    static_assert(BN == 256 || BN == 192, "tile width");
    static_assert(!DUAL || BN == 192, "the gated pair uses the 192-wide slot");
    static_assert(BMT == 256 || BMT == 128 || BMT == 64, "tile height");
    static constexpr int BM = BMT;
    static constexpr int A_BYTES = BM * A_ROW;              // 16 or 8 KiB
    static constexpr int A_COPIES = BM / 64;                // 1 KiB A copies per wave per slice
    static constexpr int B_ROW = BN * 2, B_CHUNKS = BN / 8;
    static constexpr int B_BYTES = BK * B_ROW;
    static constexpr int B_COPIES = B_BYTES / 1024 / 4;     // per wave per slice
    static constexpr int COPIES = A_COPIES + B_COPIES;
    static constexpr int SLOT_BYTES = A_BYTES + B_BYTES;
    static constexpr int WROWS = DUAL ? BM / 4 : BM / 2;    // rows per wave
    static constexpr int TM = WROWS / 32;                   // 32-row blocks per wave
    static constexpr int TN = DUAL ? BN / 32 : BN / 64;     // 32-column blocks per wave
    static constexpr int WN = DUAL ? 0 : BN / 2;            // column offset of wave column 1
    static constexpr int OUT = DUAL ? BN / 2 : BN;          // output columns per tile
};

__device__ __forceinline__ int a_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
// Chunk position of chunk c in K-row k of the B slot (an involution for each k).
template <int BN>
__device__ __forceinline__ int b_pos(int c, int k) {
    if constexpr (BN == 256) return c ^ ((0xCA60 >> ((k & 3) * 4)) & 15);
    else return (c & ~7) | ((c & 7) ^ (int)((0x6204035651271642ull >> ((k & 15) * 4)) & 7));
}

template <int DT>
__device__ __forceinline__ f32x16 mfma(i32x4 a, i32x4 b, f32x16 c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Wait until at most n slices of L copies each are still in flight (copies
// complete in issue order).
template <int L>
__device__ __forceinline__ void wait_slices(int n) {
    static_assert(L * 3 < 64, "vmcnt range");
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
    i32x4 a[TM];
    i32x4 b[TN];
};

// BKC: B' K-contiguous (a row-major A times a column-major B, the x W^T
// layout of weights stored out x in).  The B slot then holds BN rows of 64
// bytes, one column of B' each, staged and read exactly like A's rows
// (ds_read_b128 fragments, no transposed reads).
// AMC: A' M-contiguous (a column-major A times a row-major B, after the
// transpose identity).  The A slot then holds 32 K-rows of 512 bytes staged
// and read exactly like the 256-wide B slot (chunk swizzle, transposed reads).
template <int DT, int BN, bool DUAL, int EPI, bool BKC = false, bool AMC = false, int BMT = 256>
__global__ __launch_bounds__(NT, 1) void k_h_dma(Problem p, HSplit sp) {
    using G = Cfg<BN, DUAL, BMT>;
    static_assert(!(BKC && DUAL) && !(AMC && DUAL) && !(AMC && BKC), "operand forms");
    static_assert(!AMC || BMT == 256, "the M-contiguous A slot is 256 wide");
    constexpr int BM = G::BM, A_BYTES = G::A_BYTES, A_COPIES = G::A_COPIES;
    constexpr int TM = G::TM, TN = G::TN, COPIES = G::COPIES, SLOT_BYTES = G::SLOT_BYTES;
    constexpr int B_ROW = G::B_ROW, OUT = G::OUT;
    using Fr = Frags<TM, TN>;
    extern __shared__ __align__(16) unsigned char smem[];
    const ClockStamp stamp0 = clock_stamp_begin();
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = DUAL ? wave : wave >> 1, wn = DUAL ? 0 : wave & 1;

    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + OUT - 1) / OUT);
    // Workgroups of one XCD take consecutive positions; a position is
    // tile * ksplit + range, so all K ranges of a tile run on one XCD and the
    // second phase, which places each tile on the same XCD, reads their
    // partials from that XCD's L2.  Split launches group tiles two M-tiles
    // deep (an XCD's tiles then share A and B panels over the whole K),
    // unsplit ones four deep.
    const int pos = xcd_linear(blockIdx.x, gridDim.x);
    const int split = pos % sp.ksplit;
    int tmi, tni;
    tile_from_linear(pos / sp.ksplit, tiles_m, tiles_n, sp.ksplit > 1 ? SPLIT_GROUP_M : UNSPLIT_GROUP_M,
                     tmi, tni);
    const int j0 = split * sp.nks;                        // first 32-slice of this range
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * OUT;
    const int mlim = (int)(p.M - m0 < BM ? p.M - m0 : BM);
    const int nlim = (int)(p.N - n0 < OUT ? p.N - n0 : OUT);
    const uint16_t* __restrict__ A = (const uint16_t*)p.A;
    const uint16_t* __restrict__ B = (const uint16_t*)p.B;
    const uint16_t* __restrict__ B2 = (const uint16_t*)p.B2;   // gated pair: U's matrix

    // Copies of this wave: A rows [64w, 64w+64) (four copies of 16 rows); B
    // copies j = w*B_COPIES + i, each the 64 chunk positions [64j, 64j+64) of
    // the B slot (lane l: position 64j+l of the row-major slot).
    const uint16_t* src[COPIES];
    int dst[COPIES];
    if constexpr (AMC) {
        // Copy j covers the 64 chunk positions [64j, 64j+64) of the A slot
        // (32 K-rows of 32 chunks); rows past M read the last valid chunk.
#pragma unroll
        for (int i = 0; i < A_COPIES; ++i) {
            const int j = wave * A_COPIES + i;
            const int f = 64 * j + lane;
            const int k = f / 32, pos = f % 32;
            int c = b_pos<256>(pos, k);
            const int cmax = (mlim >> 3) - 1;
            c = c <= cmax ? c : cmax;
            src[i] = A + ((int64_t)j0 * BK + k) * p.lda + m0 + 8 * c;
            dst[i] = j * 1024;
        }
    } else {
#pragma unroll
    for (int i = 0; i < A_COPIES; ++i) {
        const int r = (BM / 4) * wave + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ a_swz(r);
        const int rr = r < mlim ? r : mlim - 1;
        src[i] = A + (m0 + rr) * p.lda + (int64_t)j0 * BK + 8 * c;
        dst[i] = ((BM / 4) * wave + 16 * i) * A_ROW;
    }
    }
    if constexpr (BKC) {
        constexpr int BR = BN / 4;                        // B' columns copied per wave
        static_assert(BR == 16 * G::B_COPIES, "B copies must cover the slot");
#pragma unroll
        for (int i = 0; i < G::B_COPIES; ++i) {
            const int r = BR * wave + 16 * i + (lane >> 2);
            const int c = (lane & 3) ^ a_swz(r);
            const int rr = r < nlim ? r : nlim - 1;      // columns past N: the last valid one
            src[A_COPIES + i] = B + (n0 + rr) * p.ldb + (int64_t)j0 * BK + 8 * c;
            dst[A_COPIES + i] = A_BYTES + (BR * wave + 16 * i) * A_ROW;
        }
    } else {
#pragma unroll
    for (int i = 0; i < G::B_COPIES; ++i) {
        const int j = wave * G::B_COPIES + i;
        const int f = 64 * j + lane;
        const int k = f / G::B_CHUNKS, pos = f % G::B_CHUNKS;
        int c = b_pos<BN>(pos, k);
        const int cmax = (nlim >> 3) - 1;
        if constexpr (DUAL) {
            // Chunks 0..11 of a slot row come from B (G), 12..23 from B2 (U).
            const bool second = c >= G::B_CHUNKS / 2;
            int cc = second ? c - G::B_CHUNKS / 2 : c;
            cc = cc <= cmax ? cc : cmax;
            src[A_COPIES + i] = (second ? B2 : B) + ((int64_t)j0 * BK + k) * p.ldb + n0 + 8 * cc;
        } else {
            c = c <= cmax ? c : cmax;
            src[A_COPIES + i] = B + ((int64_t)j0 * BK + k) * p.ldb + n0 + 8 * c;
        }
        dst[A_COPIES + i] = A_BYTES + j * 1024;
    }
    }
    // (The gated pair's two B matrices share ldb: host-checked.)
    const int64_t a_kstep = AMC ? (int64_t)BK * p.lda : (int64_t)BK;
    const int64_t b_kstep = BKC ? (int64_t)BK : (int64_t)BK * p.ldb;
    const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    auto copy = [&](int s, int i) {
        const unsigned base = lds0 + (unsigned)(s % SLOTS) * SLOT_BYTES;
        copy_to_lds(src[i] + (int64_t)s * (i < A_COPIES ? a_kstep : b_kstep), base + dst[i]);
    };

    // Fragment read offsets within a slot.
    int a_off[TM][2][AMC ? 2 : 1];
    if constexpr (AMC) {
        const int q = lane >> 4, t = lane & 15;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = ks * 16 + 8 * (q >> 1) + 4 * h + (t >> 2);
                    const int m = G::WROWS * wm + 32 * tm + 16 * (q & 1) + 4 * (t & 3);
                    a_off[tm][ks][h] = k * 512 + (b_pos<256>(m >> 3, k) << 4) + ((m & 7) << 1);
                }
    } else {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int r = G::WROWS * wm + 32 * tm + (lane & 31);
                const int c = 2 * ks + (lane >> 5);
                a_off[tm][ks][0] = r * A_ROW + ((c ^ a_swz(r)) << 4);
            }
    }
    int b_off[TN][2][2];
    if constexpr (BKC) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int r = G::WN * wn + 32 * tn + (lane & 31);
                const int c = 2 * ks + (lane >> 5);
                b_off[tn][ks][0] = A_BYTES + r * A_ROW + ((c ^ a_swz(r)) << 4);
                b_off[tn][ks][1] = 0;
            }
    } else {
        const int q = lane >> 4, t = lane & 15;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = ks * 16 + 8 * (q >> 1) + 4 * h + (t >> 2);
                    const int n = G::WN * wn + 32 * tn + 16 * (q & 1) + 4 * (t & 3);
                    b_off[tn][ks][h] = A_BYTES + k * B_ROW + (b_pos<BN>(n >> 3, k) << 4) + ((n & 7) << 1);
                }
    }
    auto read_a = [&](Fr& f, int s, int ks, int tm) {
        const unsigned char* base = smem + (s % SLOTS) * SLOT_BYTES;
        if constexpr (AMC) {
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(base + a_off[tm][ks][0]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(base + a_off[tm][ks][AMC ? 1 : 0]));
            const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
            f.a[tm] = i32x4{l2.x, l2.y, h2.x, h2.y};
        } else {
            f.a[tm] = *(const i32x4*)(base + a_off[tm][ks][0]);
        }
    };
    auto read_b = [&](Fr& f, int s, int ks, int tn) {
        const unsigned char* base = smem + (s % SLOTS) * SLOT_BYTES;
        if constexpr (BKC) {
            f.b[tn] = *(const i32x4*)(base + b_off[tn][ks][0]);
            return;
        }
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(base + b_off[tn][ks][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(base + b_off[tn][ks][1]));
        const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
        f.b[tn] = i32x4{l2.x, l2.y, h2.x, h2.y};
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    // One K-step: the TM*TN MFMAs on `use`, with the fragment reads that fill
    // `nxt` (slice rs, k-step rks) and copies c0..c1-1 of slice cs spread
    // evenly between them, one instruction group after each MFMA.  Reads come
    // in the order the next K-step first needs them (A0, B0.., A1..A3), so
    // its first MFMAs wait on the oldest reads only.
    constexpr int NM = TM * TN;
    auto kstep = [&](const Fr& use, Fr& nxt, bool do_read, int rs, int rks,
                     bool do_copy, int cs, int c0, int c1) {
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            // Row-wise snake: consecutive MFMAs share an operand also across
            // a row change, so the matrix core's inputs switch less (the
            // chip runs at its power limit here: 0.4-0.8% faster, measured).
            const int tm = i / TN, tn = (tm & 1) ? TN - 1 - i % TN : i % TN;
            acc[tm][tn] = mfma<DT>(use.b[tn], use.a[tm], acc[tm][tn]);
            if (do_copy) {
#pragma unroll
                for (int c = c0; c < c1; ++c)
                    if (i == (c - c0) * NM / (c1 - c0)) copy(cs, c);
            }
            if (do_read) {
                if (i == 1) read_a(nxt, rs, rks, 0);
                if (i >= 2 && i < 2 + TN) read_b(nxt, rs, rks, i - 2);
                if (i >= 2 + TN && i < 1 + TN + TM) read_a(nxt, rs, rks, i - 1 - TN);
            }
            fence_sched();
        }
        // Tiles with fewer MFMAs per K-step than fragments to read (the
        // 128-row gated pair: 1 x 6 blocks) issue the remaining reads here.
        if constexpr (NM < TM + TN + 1) {
            if (do_read) {
                if (NM <= 1) read_a(nxt, rs, rks, 0);
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    if (2 + t >= NM) read_b(nxt, rs, rks, t);
#pragma unroll
                for (int m = 1; m < TM; ++m)
                    if (1 + TN + m >= NM) read_a(nxt, rs, rks, m);
            }
            fence_sched();
        }
    };

    const int nk_all = (int)(p.K / BK);
    const int nk = nk_all - j0 < sp.nks ? nk_all - j0 : sp.nks;
    // Prologue: request slices 0..AHEAD-1, make slice 0 visible, read (0, ks=0).
    const int npro = nk < AHEAD ? nk : AHEAD;
    for (int s = 0; s < npro; ++s)
        for (int i = 0; i < COPIES; ++i) copy(s, i);
    wait_slices<COPIES>(npro - 1);
    slice_barrier();
    Fr f0, f1;
    read_a(f0, 0, 0, 0);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) read_b(f0, 0, 0, tn);
#pragma unroll
    for (int tm = 1; tm < TM; ++tm) read_a(f0, 0, 0, tm);

    // Slice j: wait for this wave's copies of slice j+1 (later slices may
    // stay in flight), barrier (slice j+1 visible to all waves, slot of slice
    // j-1 free), then K-step 0 reading (j, ks=1) with the A copies of slice
    // j+AHEAD and K-step 1 reading (j+1, ks=0) with its B copies.
    int j = 0;
    for (; j + AHEAD < nk; ++j) {
        wait_slices<COPIES>(AHEAD - 2);
        slice_barrier();
        kstep(f0, f1, true, j, 1, true, j + AHEAD, 0, A_COPIES);
        kstep(f1, f0, true, j + 1, 0, true, j + AHEAD, A_COPIES, COPIES);
    }
    for (; j < nk; ++j) {       // last (up to) AHEAD slices: no more copies
        const bool next = j + 1 < nk;
        if (next) wait_slices<COPIES>(nk - j - 2);
        if (next) slice_barrier();
        kstep(f0, f1, true, j, 1, false, 0, 0, 1);
        kstep(f1, f0, next, j + 1, 0, false, 0, 0, 1);
    }

    // K tail (K not a multiple of 32): the range that ends at the last whole
    // slice adds one more slice holding k in [32*nk_all, K).  It is staged by
    // ordinary loads into the LDS positions the copies would fill (lane l's
    // 16 bytes of copy i at dst[i] + 16*l, so the swizzled layout is the
    // copies' own), with zeros for k >= K in both operands, so the two usual
    // K-steps add exact zeros there.  Only k < K is ever read.  No copy is in
    // flight any more (the loop above waited for the last slice), so a
    // barrier frees the ring; a second one, after the LDS writes have
    // completed, publishes the slice.
    const int ktail = (int)(p.K - (int64_t)nk_all * BK);
    if (ktail > 0 && j0 + nk == nk_all) {
        const int ts = nk;                          // slice index after the range's last
        __syncthreads();
        unsigned char* slot = smem + (ts % SLOTS) * SLOT_BYTES;
#pragma unroll
        for (int i = 0; i < COPIES; ++i) {
            const bool is_a = i < A_COPIES;
            const uint16_t* s = src[i] + (int64_t)ts * (is_a ? a_kstep : b_kstep);
            // K-contiguous copies (A rows, or B' columns in the BKC form)
            // hold 8 consecutive k from 8c; the others one K-row of 8
            // consecutive m or n.
            const bool k_runs = is_a ? !AMC : BKC;
            int kfirst;
            if (k_runs) {
                const int r = is_a ? (BM / 4) * wave + 16 * i + (lane >> 2)
                                   : (BN / 4) * wave + 16 * (i - A_COPIES) + (lane >> 2);
                kfirst = 8 * ((lane & 3) ^ a_swz(r));
            } else {
                const int jj = is_a ? wave * A_COPIES + i : wave * G::B_COPIES + (i - A_COPIES);
                kfirst = (64 * jj + lane) / (is_a ? 32 : G::B_CHUNKS);
            }
            i32x4 v = i32x4{0, 0, 0, 0};
            if (!k_runs) {
                if (kfirst < ktail) v = *(const i32x4*)s;
            } else if (kfirst + 8 <= ktail) {
                v = *(const i32x4*)s;
            } else if (kfirst < ktail) {
                uint16_t e[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) e[q] = kfirst + q < ktail ? s[q] : (uint16_t)0;
                v = __builtin_bit_cast(i32x4, e);
            }
            *(i32x4*)(slot + dst[i] + 16 * lane) = v;
        }
        __syncthreads();
        read_a(f0, ts, 0, 0);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) read_b(f0, ts, 0, tn);
#pragma unroll
        for (int tm = 1; tm < TM; ++tm) read_a(f0, ts, 0, tm);
        kstep(f0, f1, true, ts, 1, false, 0, 0, 1);
        kstep(f1, f0, false, 0, 0, false, 0, 0, 1);
    }

    if constexpr (EPI == EPI_PARTIAL) {
        // Chunk c = (tm * TN + tn) * 4 + q holds acc[tm][tn][4q .. 4q+3], all of
        // one output row (lane & 31 of block tm); rows past M are not stored
        // (the second phase reads only rows below M).
        float* dst = sp.part + ((int64_t)(tmi * tiles_n + tni) * sp.ksplit + split) *
                                   (int64_t)(NT * TM * TN * 16) + 4 * tid;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            if (G::WROWS * wm + 32 * tm + (lane & 31) >= mlim) continue;
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x16& a = acc[tm][tn];
                    const f32x4 v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                    *(f32x4*)(dst + (int64_t)((tm * TN + tn) * 4 + q) * NT * 4) = v;
                }
        }
        clock_stamp_end(p, stamp0);
        return;
    }

    if constexpr (EPI == EPI_ACC32) {
        static_assert(!DUAL, "plain products only");
        float* C32 = (float*)p.C;
        const bool vec4 = (p.ldc % 4 == 0) && (((uintptr_t)p.C & 15) == 0);
        const int fr = lane & 31, nq = 4 * (lane >> 5);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int mi = G::WROWS * wm + 32 * tm + fr;
            if (mi >= mlim) continue;
            float* crow = C32 + (m0 + mi) * p.ldc + n0;
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ni = G::WN * wn + 32 * tn + 8 * q + nq;
                    const f32x4 v = {p.alpha * acc[tm][tn][4 * q], p.alpha * acc[tm][tn][4 * q + 1],
                                     p.alpha * acc[tm][tn][4 * q + 2], p.alpha * acc[tm][tn][4 * q + 3]};
                    if (vec4 && ni + 4 <= nlim) {
                        *(f32x4*)(crow + ni) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (ni + e < nlim) crow[ni + e] = v[e];
                    }
                }
        }
        clock_stamp_end(p, stamp0);
        return;
    }

    // Epilogue: lane holds C(m, n..n+3), m = row within the 32x32 block.
    uint16_t* C = (uint16_t*)p.C;
    const bool vec_ok = (p.ldc % 4 == 0) && (((uintptr_t)p.C & 7) == 0);
    const int fr = lane & 31, nq = 4 * (lane >> 5);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int mi = G::WROWS * wm + 32 * tm + fr;
        if (mi >= mlim) continue;
        uint16_t* crow = C + (m0 + mi) * p.ldc + n0;
        if constexpr (DUAL) {
            // Gated pair: block tn holds G and block tn + TN/2 holds U of the
            // same outputs (same lane layout); Z = round(T * round(U)),
            // T = round(SiLU(round(G))).
#pragma unroll
            for (int tn = 0; tn < TN / 2; ++tn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ni = 32 * tn + 8 * q + nq;
                    float z[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        z[e] = swiglu_out<DT>(acc[tm][tn][4 * q + e], acc[tm][tn + TN / 2][4 * q + e]);
                    store_out4<DT, EPI_NONE>(crow, ni, nlim, vec_ok, 0.f, z);
                }
            continue;
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ni = G::WN * wn + 32 * tn + 8 * q + nq;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = p.alpha * acc[tm][tn][4 * q + e];
                store_out4<DT, EPI>(crow, ni, nlim, vec_ok, p.beta, v);
            }
        }
    }
    clock_stamp_end(p, stamp0);
}

// Second split-K phase: one thread per 16-byte chunk of one tile's
// accumulators (the chunk and thread of the first phase), sums the K ranges in
// range order and stores four outputs as the one-phase epilogue would.  The
// gated pair's threads take a G chunk and the U chunk of the same outputs.
template <int DT, int BN, bool DUAL, int EPI, int BMT = 256>
__global__ __launch_bounds__(NT) void k_h_dma_reduce(Problem p, HSplit sp) {
    using G = Cfg<BN, DUAL, BMT>;
    constexpr int BM = G::BM;
    constexpr int TM = G::TM, TN = G::TN, OUT = G::OUT;
    constexpr int TNO = DUAL ? TN / 2 : TN;                 // blocks that hold outputs
    constexpr int CH = TM * TNO * 4;                        // chunks walked per tile
    constexpr int64_t TILE_FLOATS = (int64_t)NT * TM * TN * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = DUAL ? wave : wave >> 1, wn = DUAL ? 0 : wave & 1;
    const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + OUT - 1) / OUT);
    // CH consecutive positions per tile, in the first phase's tile order: a
    // tile's sum runs on the XCD that computed its partials.
    const int pos = xcd_linear(blockIdx.x, gridDim.x);
    const int t = pos / CH, c = pos % CH;
    int tmi, tni;
    tile_from_linear(t, tiles_m, tiles_n, SPLIT_GROUP_M, tmi, tni);
    const int tm = c / (TNO * 4), tn = (c / 4) % TNO, q = c % 4;
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * OUT;
    const int mlim = (int)(p.M - m0 < BM ? p.M - m0 : BM);
    const int nlim = (int)(p.N - n0 < OUT ? p.N - n0 : OUT);
    const int mi = G::WROWS * wm + 32 * tm + (lane & 31);
    const int ni = G::WN * wn + 32 * tn + 8 * q + 4 * (lane >> 5);
    if (mi >= mlim || ni >= nlim) return;
    const float* tile = sp.part + (int64_t)(tmi * tiles_n + tni) * sp.ksplit * TILE_FLOATS + 4 * tid;
    auto sum = [&](int chunk) {
        const float* src = tile + (int64_t)chunk * NT * 4;
        f32x4 a = *(const f32x4*)src;
        int s = 1;
        for (; s + 4 <= sp.ksplit; s += 4) {
            const f32x4 b0 = *(const f32x4*)(src + s * TILE_FLOATS);
            const f32x4 b1 = *(const f32x4*)(src + (s + 1) * TILE_FLOATS);
            const f32x4 b2 = *(const f32x4*)(src + (s + 2) * TILE_FLOATS);
            const f32x4 b3 = *(const f32x4*)(src + (s + 3) * TILE_FLOATS);
            a = (((a + b0) + b1) + b2) + b3;
        }
        for (; s < sp.ksplit; ++s) a = a + *(const f32x4*)(src + s * TILE_FLOATS);
        return a;
    };
    uint16_t* crow = (uint16_t*)p.C + (m0 + mi) * p.ldc + n0;
    const bool vec_ok = (p.ldc % 4 == 0) && (((uintptr_t)p.C & 7) == 0);
    const f32x4 g = sum((tm * TN + tn) * 4 + q);
    float v[4];
    if constexpr (DUAL) {
        const f32x4 u = sum((tm * TN + tn + TN / 2) * 4 + q);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = swiglu_out<DT>(g[e], u[e]);
        store_out4<DT, EPI_NONE>(crow, ni, nlim, vec_ok, 0.f, v);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = p.alpha * g[e];
        store_out4<DT, EPI>(crow, ni, nlim, vec_ok, p.beta, v);
    }
}

template <int BN, bool DUAL, int BMT = 256>
constexpr int64_t tile_part_bytes() {
    using G = Cfg<BN, DUAL, BMT>;
    return (int64_t)NT * G::TM * G::TN * 16 * (int64_t)sizeof(float);
}

template <int DT, int BN, bool DUAL, int EPI, bool BKC, bool AMC, int BMT>
hipError_t launch_epi(const Problem& p, const HSplit& sp, hipStream_t s) {
    using G = Cfg<BN, DUAL, BMT>;
    auto kern = k_h_dma<DT, BN, DUAL, EPI, BKC, AMC, BMT>;
    const size_t lds = (size_t)SLOTS * G::SLOT_BYTES;
    static bool attr_set[MAX_DEVICES] = {};
    if (hipError_t e = set_lds_limit_once((const void*)kern, (int)lds, attr_set); e != hipSuccess)
        return e;
    constexpr int OUT = G::OUT, BM = G::BM;
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + OUT - 1) / OUT);
    hipLaunchKernelGGL(kern, dim3((unsigned)(tiles * sp.ksplit)), dim3(NT), lds, s, p, sp);
    return hipGetLastError();
}

template <int DT, int BN, bool DUAL, int EPI, int BMT>
hipError_t launch_reduce(const Problem& p, const HSplit& sp, hipStream_t s) {
    using G = Cfg<BN, DUAL, BMT>;
    constexpr int CH = G::TM * (DUAL ? G::TN / 2 : G::TN) * 4;
    const int64_t tiles = ((p.M + G::BM - 1) / G::BM) * ((p.N + G::OUT - 1) / G::OUT);
    hipLaunchKernelGGL((k_h_dma_reduce<DT, BN, DUAL, EPI, BMT>), dim3((unsigned)(tiles * CH)), dim3(NT), 0,
                       s, p, sp);
    return hipGetLastError();
}

// One kernel per epilogue: the store loop is unrolled over every output of
// the tile, so a runtime choice would put the activation's code between the
// plain stores (and the 256-wide tile has no registers to spare for it).
template <int DT, int BN, bool DUAL, bool BKC = false, bool AMC = false, int BMT = 256>
hipError_t launch_dt(const Problem& p, int ksplit, const Workspace& ws, hipStream_t s) {
    const int nk = (int)(p.K / BK);
    HSplit sp{(float*)ws.part, 1, nk};
    const bool silu = !DUAL && p.epilogue == EPI_SILU;
    if (ksplit <= 1) {
        if constexpr (!DUAL)
            if (silu) return launch_epi<DT, BN, false, EPI_SILU, BKC, AMC, BMT>(p, sp, s);
        return launch_epi<DT, BN, DUAL, EPI_NONE, BKC, AMC, BMT>(p, sp, s);
    }
    sp.nks = (nk + ksplit - 1) / ksplit;
    sp.ksplit = (nk + sp.nks - 1) / sp.nks;
    hipError_t e = launch_epi<DT, BN, DUAL, EPI_PARTIAL, BKC, AMC, BMT>(p, sp, s);
    if (e != hipSuccess) return e;
    if constexpr (!DUAL)
        if (silu) return launch_reduce<DT, BN, false, EPI_SILU, BMT>(p, sp, s);
    return launch_reduce<DT, BN, DUAL, EPI_NONE, BMT>(p, sp, s);
}

}  // namespace

bool h_dma_supports(const Problem& p, int bn, int bm) {
    if (bn != 256 && bn != 192) return false;
    // 128 or 64 rows: BN = 192 with A' K-contiguous only.
    if (bm != 256 && ((bm != 128 && bm != 64) || bn != 192 || !p.a_kc)) return false;
    if (p.dtype != F16 && p.dtype != BF16) return false;
    if (!p.a_kc && p.b_kc) return false;
    // N-contiguous B' rows (M-contiguous A' columns) are read as 8-element
    // chunks; K-contiguous operands as 32-element K slices, the last one
    // (K not a multiple of 32) staged by ordinary loads.
    if (p.K < BK || p.K / BK > 0x7fffffff || (!p.b_kc && p.N % 8 != 0)) return false;
    if (!p.a_kc && p.M % 8 != 0) return false;
    if (p.lda % 8 != 0 || p.ldb % 8 != 0) return false;
    if (((uintptr_t)p.A & 15) != 0 || ((uintptr_t)p.B & 15) != 0) return false;
    const int64_t tiles = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    return tiles > 0 && tiles <= 0x7fffffff / 64;
}

int h_dma_splits(const Problem& p, int bn, bool dual, int requested, const Workspace& ws, int bm) {
    const int out = dual ? 96 : bn;
    const int64_t tiles = ((p.M + bm - 1) / bm) * ((p.N + out - 1) / out);
    const int64_t nk = p.K / BK;
    const int64_t tile_bytes = bm == 64    ? tile_part_bytes<192, false, 64>()
                               : bm == 128 ? tile_part_bytes<192, false, 128>()
                               : (bn == 256 ? tile_part_bytes<256, false>() : tile_part_bytes<192, false>());
    if (requested <= 1 || nk < 2) return 1;
    int64_t ks = requested < nk ? requested : nk;
    const int64_t nks = (nk + ks - 1) / ks;                 // whole slices per range
    ks = (nk + nks - 1) / nks;
    if (ws.part == nullptr || tiles * ks * tile_bytes > ws.part_bytes) return 0;
    return (int)ks;
}

hipError_t launch_h_dma(const Problem& p, int bn, int ksplit, const Workspace& ws, hipStream_t s,
                        int bm) {
    if (bm == 64) {
        if (p.b_kc)
            return p.dtype == F16 ? launch_dt<F16, 192, false, true, false, 64>(p, ksplit, ws, s)
                                  : launch_dt<BF16, 192, false, true, false, 64>(p, ksplit, ws, s);
        return p.dtype == F16 ? launch_dt<F16, 192, false, false, false, 64>(p, ksplit, ws, s)
                              : launch_dt<BF16, 192, false, false, false, 64>(p, ksplit, ws, s);
    }
    if (bm == 128) {
        if (p.b_kc)
            return p.dtype == F16 ? launch_dt<F16, 192, false, true, false, 128>(p, ksplit, ws, s)
                                  : launch_dt<BF16, 192, false, true, false, 128>(p, ksplit, ws, s);
        return p.dtype == F16 ? launch_dt<F16, 192, false, false, false, 128>(p, ksplit, ws, s)
                              : launch_dt<BF16, 192, false, false, false, 128>(p, ksplit, ws, s);
    }
    if (!p.a_kc) {
        if (bn == 192)
            return p.dtype == F16 ? launch_dt<F16, 192, false, false, true>(p, ksplit, ws, s)
                                  : launch_dt<BF16, 192, false, false, true>(p, ksplit, ws, s);
        return p.dtype == F16 ? launch_dt<F16, 256, false, false, true>(p, ksplit, ws, s)
                              : launch_dt<BF16, 256, false, false, true>(p, ksplit, ws, s);
    }
    if (p.b_kc) {
        if (bn == 192)
            return p.dtype == F16 ? launch_dt<F16, 192, false, true>(p, ksplit, ws, s)
                                  : launch_dt<BF16, 192, false, true>(p, ksplit, ws, s);
        return p.dtype == F16 ? launch_dt<F16, 256, false, true>(p, ksplit, ws, s)
                              : launch_dt<BF16, 256, false, true>(p, ksplit, ws, s);
    }
    if (bn == 192)
        return p.dtype == F16 ? launch_dt<F16, 192, false>(p, ksplit, ws, s)
                              : launch_dt<BF16, 192, false>(p, ksplit, ws, s);
    return p.dtype == F16 ? launch_dt<F16, 256, false>(p, ksplit, ws, s)
                          : launch_dt<BF16, 256, false>(p, ksplit, ws, s);
}

hipError_t launch_h_dma_acc32(const Problem& p, int bn, hipStream_t s) {
    const HSplit sp{nullptr, 1, (int)(p.K / BK)};
    if (!p.a_kc) {
        if (bn == 192)
            return p.dtype == F16 ? launch_epi<F16, 192, false, EPI_ACC32, false, true, 256>(p, sp, s)
                                  : launch_epi<BF16, 192, false, EPI_ACC32, false, true, 256>(p, sp, s);
        return p.dtype == F16 ? launch_epi<F16, 256, false, EPI_ACC32, false, true, 256>(p, sp, s)
                              : launch_epi<BF16, 256, false, EPI_ACC32, false, true, 256>(p, sp, s);
    }
    if (p.b_kc) {
        if (bn == 192)
            return p.dtype == F16 ? launch_epi<F16, 192, false, EPI_ACC32, true, false, 256>(p, sp, s)
                                  : launch_epi<BF16, 192, false, EPI_ACC32, true, false, 256>(p, sp, s);
        return p.dtype == F16 ? launch_epi<F16, 256, false, EPI_ACC32, true, false, 256>(p, sp, s)
                              : launch_epi<BF16, 256, false, EPI_ACC32, true, false, 256>(p, sp, s);
    }
    if (bn == 192)
        return p.dtype == F16 ? launch_epi<F16, 192, false, EPI_ACC32, false, false, 256>(p, sp, s)
                              : launch_epi<BF16, 192, false, EPI_ACC32, false, false, 256>(p, sp, s);
    return p.dtype == F16 ? launch_epi<F16, 256, false, EPI_ACC32, false, false, 256>(p, sp, s)
                          : launch_epi<BF16, 256, false, EPI_ACC32, false, false, 256>(p, sp, s);
}

bool h_gated_supports(const Problem& p) {
    if (p.b_kc || !p.a_kc || !h_dma_supports(p, 192) || p.B2 == nullptr || p.ldb2 != p.ldb)
        return false;
    return ((uintptr_t)p.B2 & 15) == 0;
}

hipError_t launch_h_gated(const Problem& p, int ksplit, const Workspace& ws, hipStream_t s, int bm) {
    if (bm == 128)
        return p.dtype == F16 ? launch_dt<F16, 192, true, false, false, 128>(p, ksplit, ws, s)
                              : launch_dt<BF16, 192, true, false, false, 128>(p, ksplit, ws, s);
    return p.dtype == F16 ? launch_dt<F16, 192, true>(p, ksplit, ws, s)
                          : launch_dt<BF16, 192, true>(p, ksplit, ws, s);
}

}  // namespace mgemm
