// libmgemm host side: argument validation, normalisation to one canonical
// row-major problem, kernel selection and launch.  See include/mgemm.h for
// the contract of every entry point.
#include <hip/hip_runtime.h>

#include <new>
#include <string.h>
#include <utility>

#include "f8_tiles.h"
#include "host.h"

namespace mgemm_host {

namespace {
inline bool valid_layout(mgemm_layout_t l) { return l == MGEMM_ROW_MAJOR || l == MGEMM_COL_MAJOR; }
inline bool valid_dtype(mgemm_dtype_t d) { return d == MGEMM_F32 || d == MGEMM_F16 || d == MGEMM_BF16; }
inline int64_t max1(int64_t x) { return x > 1 ? x : 1; }
}  // namespace

// Checks the rules of mgemm_run and builds the canonical problem for a
// device with num_cu compute units.
mgemm_status_t make_problem_on(int num_cu, mgemm_layout_t layoutA, mgemm_layout_t layoutB,
                               int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                               int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                               int64_t ldc, mgemm_dtype_t dtype, Problem* out) {
    if (!valid_layout(layoutA) || !valid_layout(layoutB) || !valid_dtype(dtype))
        return MGEMM_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return MGEMM_ERR_INVALID_ARG;
    const bool rowA = layoutA == MGEMM_ROW_MAJOR, rowB = layoutB == MGEMM_ROW_MAJOR;
    if (lda < max1(rowA ? K : M)) return MGEMM_ERR_INVALID_ARG;
    if (ldb < max1(rowB ? N : K)) return MGEMM_ERR_INVALID_ARG;
    if (ldc < max1(rowA ? N : M)) return MGEMM_ERR_INVALID_ARG;
    // Offsets are formed in 64-bit; keep every addressed element index below 2^62.
    const int64_t lim = (int64_t)1 << 62;
    if (M > lim / max1(ldc) || N > lim / max1(ldc) || K > lim / max1(lda) || K > lim / max1(ldb) ||
        M > lim / max1(lda) || N > lim / max1(ldb))
        return MGEMM_ERR_INVALID_ARG;
    const bool empty = M == 0 || N == 0;
    const bool reads_ab = !empty && K > 0 && alpha != 0.f;
    if (!empty && C == nullptr) return MGEMM_ERR_INVALID_ARG;
    if (reads_ab && (A == nullptr || B == nullptr)) return MGEMM_ERR_INVALID_ARG;

    Problem p;
    p.K = K;
    p.alpha = alpha;
    p.beta = beta;
    p.C = C;
    p.ldc = ldc;
    p.dtype = (int)dtype;
    p.num_cu = num_cu;
    p.epilogue = mgemm::EPI_NONE;
    p.B2 = nullptr;
    p.ldb2 = 0;
    if (rowA) {
        // Row-major C = A B.  A row-major is K-contiguous; B row-major is
        // N-contiguous, column-major is K-contiguous.
        p.M = M; p.N = N;
        p.A = A; p.lda = lda; p.a_kc = 1;
        p.B = B; p.ldb = ldb; p.b_kc = rowB ? 0 : 1;
    } else {
        // Column-major C is row-major C^T (N x M) = B^T A^T on the same bytes.
        //   A'' = B^T (N x K): B row-major -> B^T is N-contiguous along its
        //   rows' index, i.e. not K-contiguous; B column-major -> K-contiguous.
        //   B'' = A^T (K x M): A column-major -> M-contiguous.
        p.M = N; p.N = M;
        p.A = B; p.lda = ldb; p.a_kc = rowB ? 0 : 1;
        p.B = A; p.ldb = lda; p.b_kc = 0;
    }
    *out = p;
    return MGEMM_SUCCESS;
}

mgemm_status_t make_problem(mgemm_handle_t h, mgemm_layout_t layoutA, mgemm_layout_t layoutB,
                            int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                            int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                            int64_t ldc, mgemm_dtype_t dtype, Problem* out) {
    if (!h) return MGEMM_ERR_INVALID_ARG;
    return make_problem_on(h->num_cu, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                           ldc, dtype, out);
}

bool variant_supports(const Problem& p, mgemm_kernel_t k) {
    switch (k) {
    case MGEMM_KERNEL_GENERAL: return true;
    case MGEMM_KERNEL_F32_MFMA: return mgemm::f32_mfma_supports(p);
    case MGEMM_KERNEL_H_256x256:
    case MGEMM_KERNEL_H_256x192:
    case MGEMM_KERNEL_H_128x128: return mgemm::h_mfma_supports(p, (int)k);
    case MGEMM_KERNEL_SKINNY: return mgemm::skinny_supports(p);
    case MGEMM_KERNEL_F32_FAST: return mgemm::f32_fast_supports(p, true);
    case MGEMM_KERNEL_F32_FAST_128: return mgemm::f32_fast_supports(p, false);
    case MGEMM_KERNEL_H_DMA_256: return mgemm::h_dma_supports(p, 256);
    case MGEMM_KERNEL_H_DMA_192: return mgemm::h_dma_supports(p, 192);
    case MGEMM_KERNEL_H_DMA_128: return mgemm::h_dma_supports(p, 192, 128);
    case MGEMM_KERNEL_H_DMA_64: return mgemm::h_dma_supports(p, 192, 64);
    case MGEMM_KERNEL_F32_FAST_U: return mgemm::f32_unaligned_supports(p);
    case MGEMM_KERNEL_F32_SK: return mgemm::f32_unaligned_supports(p);
    case MGEMM_KERNEL_SKINNY_SK: return mgemm::skinny_sk_supports(p);
    default: return false;
    }
}

// Predicted time (microseconds) of a 16-bit MFMA kernel on this problem:
// waves of workgroups times the time of one workgroup (per 32-wide K slice of
// a bm x bn tile SLICE_US * bm*bn/256^2 / speed, times the workgroups sharing
// a CU, plus 2 us), and for a split of K the second pass over the FP32
// partials (4 us plus the partial bytes at 2.6 TB/s).  Constants fitted to
// MI355X measurements of 1024x1536x4096, 512x1024x2048, 2048^3 and
// 512x4096x8192 BF16 over every split from 1 to 16; `speed` is a kernel's
// per-CU rate relative to the register-staged kernel (the direct-to-LDS
// kernel runs a full 256x256 tile 1.4x as fast: 1024 NN tiles in 2.12 vs
// 2.58 ms).  A slice never takes less than its operand bytes ((bm + bn) x 32
// 16-bit values) at 60 KB/us per CU: the rate one CU's copies reach (128-
// and 64-row tiles of 1024^3, 512x1024x2048 and 256x1536x4096 spend 0.33 and
// 0.25-0.27 us per slice, above their share of the MFMA time).  `part_rate`
// replaces the partials' 2.6 TB/s where a caller measured its own.
double predict_us(const Problem& p, int bm, int bn, int out_n, double speed, int per_cu, int ks,
                  double part_rate = 0.0) {
    constexpr double SLICE_US = 0.98, WG_US = 2.0, PASS_US = 4.0;
    const double PART_BYTES_PER_US = part_rate > 0.0 ? part_rate : 2.6e6;
    constexpr double CU_BYTES_PER_US = 60e3;
    const int64_t slots = p.num_cu > 0 ? p.num_cu : 256;
    const int64_t tiles = ((p.M + bm - 1) / bm) * ((p.N + out_n - 1) / out_n);
    const int64_t nk = (p.K + 31) / 32;
    const int64_t cap = slots * per_cu;
    const int64_t waves = (tiles * ks + cap - 1) / cap;
    const int64_t nks = (nk + ks - 1) / ks;
    const double mfma = SLICE_US * (double)(bm * bn) / 65536.0 / speed * per_cu;
    const double copy = (double)(bm + bn) * 64.0 * per_cu / CU_BYTES_PER_US;
    const double slice = mfma > copy ? mfma : copy;
    double t = (double)waves * ((double)nks * slice + WG_US);
    if (ks > 1) t += PASS_US + (double)tiles * ks * bm * bn * 4.0 / PART_BYTES_PER_US;
    return t;
}

// True when a split of K into ks ranges (of ceil((K/32)/ks) 32-row slices)
// makes the ranges of a streamed 16-bit B start a multiple of 2 MiB apart
// while B's row pitch is a power of two of at least 8 KiB.  The ranges then
// read addresses that agree in their low 21 bits at every step, and B
// streams from HBM markedly slower (per-workgroup stamps, BF16 M = 32 x
// W[K x 4096]: K = 8192 in 11 ranges, 6 MiB apart, 0.62 us per slice and
// 4.1 TB/s against 0.43 us and 5.2 TB/s in 10 ranges, 6.5 MiB apart; K =
// 4096 in 8 ranges 0.57 against 0.49 us in 10; the split skinny kernel at
// 16 ranges, 2 MiB apart, 1.29 us per slice against 0.54 at 12).  A 24 KiB
// pitch (W[K x 12288]) streams at full rate at 24 MiB apart.  Only M <= 64
// is affected: larger M re-reads B from the caches, and there such splits
// measured fastest (BF16 2048x4096x12288 in 2 ranges 177 us, 240 without).
bool conflicting_split(const Problem& p, int ks) {
    if (ks <= 1 || p.b_kc || p.M > 64 || p.dtype == mgemm::F32) return false;
    const int64_t pitch = p.ldb * 2;
    if (pitch < 8192 || (pitch & (pitch - 1)) != 0) return false;
    const int64_t nk = p.K / 32, nks = (nk + ks - 1) / ks;
    return (nks * 32 * pitch) % ((int64_t)2 << 20) == 0;
}

// The split skinny kernel's own choice of ranges, moved to the nearest count
// (within one round of workgroups) whose ranges do not conflict as above.
int skinny_sk_auto(const Problem& p, const mgemm::Workspace& ws) {
    const int64_t slots = p.num_cu > 0 ? p.num_cu : 256;
    const int64_t blocks = (p.N + 255) / 256;
    const int ks = mgemm::skinny_sk_splits(p, ws, 0);
    if (!conflicting_split(p, ks)) return ks;
    for (int d : {-1, 1, -2, 2, -3, 3}) {
        const int r = ks + d;
        if (r < 2 || blocks * r > slots) continue;
        const int k2 = mgemm::skinny_sk_splits(p, ws, r);
        if (k2 >= 2 && !conflicting_split(p, k2)) return k2;
    }
    return ks;
}

// Split of K with the smallest predicted time for the direct-to-LDS kernel
// (tile width bn; the gated pair's tile holds 96 output columns), among the
// splits that fit the workspace and do not conflict as above.
int auto_split(const Problem& p, int bn, bool dual, const mgemm::Workspace& ws, double* t_out,
               int bm = 256) {
    const double speed = bn == 256 ? 1.4 : 1.3;
    const int out_n = dual ? 96 : bn;
    int best = 1;
    double best_t = predict_us(p, bm, bn, out_n, speed, 1, 1);
    int last = 1;
    for (int req = 2; req <= mgemm::MAX_KSPLIT; ++req) {
        const int ks = mgemm::h_dma_splits(p, bn, dual, req, ws, bm);
        if (ks <= last) continue;          // same number of ranges as a smaller request
        last = ks;
        if (conflicting_split(p, ks)) continue;
        const double t = predict_us(p, bm, bn, out_n, speed, 1, ks);
        if (t < best_t) { best_t = t; best = ks; }
    }
    if (t_out) *t_out = best_t;
    return best;
}

// Kernel choice of the built-in model for a canonical problem.
Choice model_choice(const Problem& p, const mgemm::Workspace& ws) {
    const int64_t slots = p.num_cu > 0 ? p.num_cu : 256;
    // Fraction of the CU-time a grid of bm x bn tiles spends on useful
    // outputs (wave quantisation and ragged-edge padding count as waste).
    auto fill = [&](int bm, int bn, int per_cu) {
        const int64_t tiles = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
        const int64_t cap = slots * per_cu;
        const int64_t waves = (tiles + cap - 1) / cap;
        return (double)p.M * (double)p.N / ((double)waves * cap * bm * bn);
    };
    if (p.dtype == mgemm::F32) {
        // Stream-K whenever whole 256x256 tiles would leave CUs idle in the
        // last wave and every CU gets at least two K slices (measured:
        // 1000x12290x4095 892 against 1063 us, 3000^3 466 against 754 us,
        // 4096x3072x4096 799 against 985 us, 1000^3 78 against 126 us).
        // Aligned shapes whose 128x128 tiles fill whole waves of one per CU
        // take those instead (2048^3 159-162 against 171-172 us on stream-K,
        // 4096x3072x4096 770-771 against 794; 1024x4096x4096 306-307 against
        // 297-307, depending on the box).
        {
            const int64_t pairs = ((p.M + 255) / 256) * ((p.N + 255) / 256) * ((p.K + 31) / 32);
            if (fill(256, 256, 1) < 0.95 && pairs >= 2 * slots && mgemm::f32_unaligned_supports(p) &&
                mgemm::f32_sk_fits(p, ws)) {
                if (fill(128, 128, 1) >= 0.95 && mgemm::f32_fast_supports(p, false))
                    return {MGEMM_KERNEL_F32_FAST_128, 1};
                return {MGEMM_KERNEL_F32_SK, 1};
            }
        }
        const bool big = mgemm::f32_fast_supports(p, true), small = mgemm::f32_fast_supports(p, false);
        if (big && (!small || fill(256, 256, 1) >= fill(128, 128, 2) * 0.9))
            return {MGEMM_KERNEL_F32_FAST, 1};
        if (small) return {MGEMM_KERNEL_F32_FAST_128, 1};
        // NN operands that are not 16-byte aligned or a K that is not a
        // multiple of the slice: the same kernel with narrower loads.  It has
        // only 256x256 tiles; a grid of them that leaves more than half of the
        // CUs idle runs faster on the 128x128 masked kernel (1000^3: 125 vs
        // 260 us).
        if (mgemm::f32_unaligned_supports(p)) {
            const int64_t tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
            if (tiles * 2 <= slots && mgemm::f32_mfma_supports(p)) return {MGEMM_KERNEL_F32_MFMA, 1};
            return {MGEMM_KERNEL_F32_FAST_U, 1};
        }
        return {MGEMM_KERNEL_F32_MFMA, 1};
    }
    // M <= 64 streams B once.  Short K (at most 64 slices) runs whole-K: with
    // few steps per range the exchange of partial rows costs more than a split
    // saves (BF16, K = 2048, M = 1 / 16 / 32 x 1024 columns 6.8 / 6.7 / 8.0 us
    // against 7.2 / 8.7 / 11.5 on the split skinny kernel; M = 64 x 12288
    // columns 14.7 against 15.3 on 64-row tiles in 3 ranges; K = 1024, M = 64
    // x 12288: 10.0 against 11.7).  Above 32 rows and 32 slices the whole-K
    // kernel's 64-column blocks need N >= 8192 (128 workgroups) to keep up
    // (K = 2048, M = 64 x 6144 / 4096 / 1024 columns: 13.7 / 13.1 / 10.5 us
    // against 11.1 / 10.4 / 8.6 on 64-row tiles with a K split).
    // Longer K splits over workgroups.  The split skinny kernel reads B in
    // 512-byte row segments of 256-column blocks; it wins only for M <= 16,
    // only where at most 16 ranges of those blocks still give three quarters
    // of the CUs a workgroup, and above 4 rows only where 6 ranges do (BF16 x
    // W[4096 x 12288], M = 1 / 16: 21.0 / 22.4 us against 22.2 / 22.8 on
    // 64-row tiles).  Narrower B, or more rows (whose cost the skinny
    // kernel's 16-row MFMA blocks pay in full), go to the time model below,
    // which picks the 64- or 128-row tiles of the direct-to-LDS kernel with a
    // K split (M = 1 / 16 / 32 x W[4096 x 1536]: 7.6 / 7.9 / 8.5 us against
    // 8.8 / 11.4 / 16.3 on the skinny kernel; M = 32 x W[4096 x 4096] 15.0
    // against 17.1; M = 64 x W[4096 x 12288] 26.0 against 31.5).
    if (p.M <= 64 && p.K <= 2048 && (p.M <= 32 || p.K <= 1024 || p.N >= 8192) &&
        mgemm::skinny_supports(p))
        return {MGEMM_KERNEL_SKINNY, 1};
    const int64_t sk_blocks = (p.N + 255) / 256;
    // Its last-arriving workgroup per block sums the other ranges' partial
    // rows (M of them, through device-scope memory): cheap for a few rows or
    // ranges, but for 8-16 rows over 8-16 ranges the 64-row tiles' separate
    // sum pass is faster (M = 16 x W[4096 x 4096]: 13.2 us in 12 ranges
    // against 11.5; M = 8: 12.1 against 11.4; M = 16 x W[4096 x 3072] 13.2
    // against 10.2; but M = 16 x W[4096 x 8192] in 6 ranges 16.3 against 16.8,
    // M = 8 x W[8192 x 8192] 27.5 against 29.2, M = 1 x W[4096 x 4096] in 10
    // ranges 10.9 against 11.2).
    if (p.M <= 16 && sk_blocks * 16 * 4 >= slots * 3 && mgemm::skinny_sk_supports(p)) {
        const int ks = skinny_sk_auto(p, ws);
        if (p.M <= 4 || ks <= 6) return {MGEMM_KERNEL_SKINNY_SK, ks};
    }
    if (p.M <= 64 && !mgemm::h_dma_supports(p, 192, 64)) {
        if (mgemm::skinny_sk_supports(p)) return {MGEMM_KERNEL_SKINNY_SK, skinny_sk_auto(p, ws)};
        if (mgemm::skinny_supports(p)) return {MGEMM_KERNEL_SKINNY, 1};
    }
    // 16-bit: the variant (and split of K) with the smallest predicted time.
    Choice best{MGEMM_KERNEL_GENERAL, 1};
    double best_t = 1e300;
    for (int bn : {256, 192}) {
        if (!mgemm::h_dma_supports(p, bn)) continue;
        double t;
        const int ks = auto_split(p, bn, false, ws, &t);
        if (t < best_t) { best_t = t; best = {bn == 256 ? MGEMM_KERNEL_H_DMA_256 : MGEMM_KERNEL_H_DMA_192, ks}; }
    }
    // 128-row tiles: each extra 128-row band streams B once more, so they are
    // considered only for M <= 128 or a B small enough to be shared through
    // the 256 MiB last-level cache (<= 32 MiB).  Measured (BF16): M = 96 / 128
    // x W[4096 x 12288] 33.5 / 36.5 us against 38.3 / 40.8 on 256-row tiles,
    // but M = 192 / 256 45.3 / 52.3 against 44.1 / 47.4 (W is 96 MiB); the
    // FFN share 1024x1536x4096 25.9 against 28.6 us, 512x1024x2048 15.9
    // against 19.4, 256x4096x4096 22.1 against 25.0.  From M = 1024 the
    // 256-row tiles read each B panel four or more times already, and the
    // 128-row grid can fill a last round that 256-row tiles leave half empty
    // (M = 1536 x W[4096 x 12288]: 161.6 us against 182.3; the time model
    // keeps 256-row tiles at M = 1024, 1280, 1792, 2048, 2560 and 3072, where
    // they are the faster).
    const bool b_small = (double)p.K * (double)p.N * 2.0 <= 32.0 * 1024 * 1024;
    if ((p.M <= 128 || b_small || p.M >= 1024) && mgemm::h_dma_supports(p, 192, 128)) {
        double t;
        const int ks = auto_split(p, 192, false, ws, &t, 128);
        if (t < best_t) { best_t = t; best = {MGEMM_KERNEL_H_DMA_128, ks}; }
    }
    // 64-row tiles for 32 < M <= 64: no padding rows, half the partial bytes
    // of a 128-row split (BF16 x W[4096 x N], N = 12288: M = 64 / 48 / 33 in
    // 27.2 / 26.0 / 24.8 us against 27.9 / 26.7 us on 128-row tiles and 25.9
    // on the skinny kernel at M = 33; N = 4096, M = 64: 13.1 against 13.7).
    // Above 64 rows, under the same small-B rule as the 128-row tiles: small
    // grids gain CUs at the per-CU copy rate (BF16 1024^3 11.8 against 15.3
    // us, 512^3 7.9 against 10.3, 512x1024x2048 11.6 against 12.6).
    if ((p.M <= 64 || b_small) && mgemm::h_dma_supports(p, 192, 64)) {
        double t;
        const int ks = auto_split(p, 192, false, ws, &t, 64);
        if (t < best_t) { best_t = t; best = {MGEMM_KERNEL_H_DMA_64, ks}; }
    }
    // Register-staged kernels (any layout); two 128x128 workgroups share a CU
    // and together run at 0.8 of the 256x256 rate (2048^3 BF16: 43.9 us).
    struct Cand { mgemm_kernel_t k; int bm, bn, per_cu; double speed; };
    const Cand regs[3] = {{MGEMM_KERNEL_H_256x256, 256, 256, 1, 1.0},
                          {MGEMM_KERNEL_H_256x192, 256, 192, 1, 1.0},
                          {MGEMM_KERNEL_H_128x128, 128, 128, 2, 0.8}};
    for (const Cand& c : regs) {
        if (!mgemm::h_mfma_supports(p, (int)c.k)) continue;
        const double t = predict_us(p, c.bm, c.bn, c.bn, c.speed, c.per_cu, 1);
        if (t < best_t) { best_t = t; best = {c.k, 1}; }
    }
    return best;
}

bool splittable(mgemm_kernel_t k) {
    return k == MGEMM_KERNEL_H_DMA_256 || k == MGEMM_KERNEL_H_DMA_192 || k == MGEMM_KERNEL_H_DMA_128 ||
           k == MGEMM_KERNEL_H_DMA_64 ||
           k == MGEMM_KERNEL_SKINNY_SK;
}

// Number of K ranges a forced variant runs with (0: it cannot run them).
int forced_splits(const Problem& p, const mgemm::Workspace& ws, mgemm_kernel_t k, int requested) {
    switch (k) {
    case MGEMM_KERNEL_H_DMA_256:
        return requested == 0 ? auto_split(p, 256, false, ws, nullptr)
                              : mgemm::h_dma_splits(p, 256, false, requested, ws);
    case MGEMM_KERNEL_H_DMA_192:
        return requested == 0 ? auto_split(p, 192, false, ws, nullptr)
                              : mgemm::h_dma_splits(p, 192, false, requested, ws);
    case MGEMM_KERNEL_H_DMA_128:
        return requested == 0 ? auto_split(p, 192, false, ws, nullptr, 128)
                              : mgemm::h_dma_splits(p, 192, false, requested, ws, 128);
    case MGEMM_KERNEL_H_DMA_64:
        return requested == 0 ? auto_split(p, 192, false, ws, nullptr, 64)
                              : mgemm::h_dma_splits(p, 192, false, requested, ws, 64);
    case MGEMM_KERNEL_SKINNY_SK:
        return requested == 0 ? skinny_sk_auto(p, ws) : mgemm::skinny_sk_splits(p, ws, requested);
    case MGEMM_KERNEL_F32_SK: return requested <= 1 && mgemm::f32_sk_fits(p, ws) ? 1 : 0;
    default: return requested <= 1 ? 1 : 0;
    }
}

// A table entry for the problem (exact shape first, then its bucket) if its
// variant can run it; otherwise the model.
Choice choose_in(const Table* table, const mgemm::Workspace& ws, const Problem& p) {
    if (table && !table->entries.empty()) {
        const auto& tab = table->entries;
        for (const TableKey& key : {exact_key(p), bucket_key(p)}) {
            auto it = tab.find(key);
            if (it == tab.end()) continue;
            const mgemm_kernel_t k = (mgemm_kernel_t)it->second.kernel;
            if (!variant_supports(p, k)) continue;
            const int ks = forced_splits(p, ws, k, it->second.ksplit);
            if (ks >= 1) return {k, ks};
        }
    }
    return model_choice(p, ws);
}

Choice choose(mgemm_handle_t h, const Problem& p) { return choose_in(&h->table, h->ws, p); }

mgemm_status_t launch(mgemm_handle_t h, const Problem& p, Choice c, hipStream_t s) {
    return launch_ws(h->ws, p, c, s);
}

mgemm_status_t launch_ws(const mgemm::Workspace& ws, const Problem& p, Choice c, hipStream_t s) {
    hipError_t e;
    switch (c.k) {
    case MGEMM_KERNEL_SKINNY_SK: e = mgemm::launch_skinny_sk(p, ws, c.ksplit, s); break;
    case MGEMM_KERNEL_GENERAL: e = mgemm::launch_general(p, s); break;
    case MGEMM_KERNEL_F32_MFMA: e = mgemm::launch_f32_mfma(p, s); break;
    case MGEMM_KERNEL_H_256x256:
    case MGEMM_KERNEL_H_256x192:
    case MGEMM_KERNEL_H_128x128: e = mgemm::launch_h_mfma(p, (int)c.k, s); break;
    case MGEMM_KERNEL_SKINNY: e = mgemm::launch_skinny(p, s); break;
    case MGEMM_KERNEL_F32_FAST: e = mgemm::launch_f32_fast(p, true, s); break;
    case MGEMM_KERNEL_F32_FAST_128: e = mgemm::launch_f32_fast(p, false, s); break;
    case MGEMM_KERNEL_H_DMA_256: e = mgemm::launch_h_dma(p, 256, c.ksplit, ws, s); break;
    case MGEMM_KERNEL_H_DMA_192: e = mgemm::launch_h_dma(p, 192, c.ksplit, ws, s); break;
    case MGEMM_KERNEL_H_DMA_128: e = mgemm::launch_h_dma(p, 192, c.ksplit, ws, s, 128); break;
    case MGEMM_KERNEL_H_DMA_64: e = mgemm::launch_h_dma(p, 192, c.ksplit, ws, s, 64); break;
    case MGEMM_KERNEL_F32_FAST_U: e = mgemm::launch_f32_unaligned(p, s); break;
    case MGEMM_KERNEL_F32_SK: e = mgemm::launch_f32_sk(p, ws, s); break;
    default: return MGEMM_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
}

mgemm_status_t run_core(int num_cu, const mgemm::Workspace& ws, const Table* table,
                        mgemm_kernel_t forced, int ksplit, mgemm_layout_t layoutA,
                        mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                        void* C, int64_t ldc, mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                        hipStream_t stream, mgemm_status_t too_big,
                        unsigned long long* stamps, int64_t stamps_cap) {
    Problem p;
    mgemm_status_t st = make_problem_on(num_cu, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb,
                                        beta, C, ldc, dtype, &p);
    if (st != MGEMM_SUCCESS) return st;
    p.stamps = stamps;
    p.stamps_cap = stamps ? stamps_cap : 0;
    if (forced != MGEMM_KERNEL_AUTO && (forced <= 0 || forced >= MGEMM_KERNEL_COUNT))
        return MGEMM_ERR_INVALID_ARG;
    if (ksplit < 0 || ksplit > MGEMM_MAX_KSPLIT || (forced == MGEMM_KERNEL_AUTO && ksplit != 0))
        return MGEMM_ERR_INVALID_ARG;
    if (epilogue != MGEMM_EPILOGUE_NONE && epilogue != MGEMM_EPILOGUE_SILU)
        return MGEMM_ERR_INVALID_ARG;
    p.epilogue = epilogue == MGEMM_EPILOGUE_SILU ? mgemm::EPI_SILU : mgemm::EPI_NONE;
    if (p.M == 0 || p.N == 0) return MGEMM_SUCCESS;
    if (p.K == 0 || p.alpha == 0.f) {
        hipError_t e = mgemm::launch_scale(p, stream);
        return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
    }
    Choice c;
    if (forced == MGEMM_KERNEL_AUTO) {
        c = choose_in(table, ws, p);
    } else {
        if (!variant_supports(p, forced)) return MGEMM_ERR_UNSUPPORTED;
        c = {forced, forced_splits(p, ws, forced, ksplit)};
        if (c.ksplit < 1) {
            // Tell a split (or stream-K) form that the workspace cannot hold
            // apart from a variant that cannot run the shape at all: ask again
            // with an unbounded workspace (sizes only; nothing is launched).
            const mgemm::Workspace unbounded{(void*)256, (int64_t)1 << 62, (unsigned*)256,
                                             (int64_t)1 << 40};
            return forced_splits(p, unbounded, forced, ksplit) >= 1 ? too_big
                                                                     : MGEMM_ERR_UNSUPPORTED;
        }
    }
    return launch_ws(ws, p, c, stream);
}

namespace {

mgemm_status_t run_impl(mgemm_handle_t h, mgemm_kernel_t forced, int ksplit, mgemm_layout_t layoutA,
                        mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                        void* C, int64_t ldc, mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                        hipStream_t stream) {
    if (!h) return MGEMM_ERR_INVALID_ARG;
    return run_core(h->num_cu, h->ws, &h->table, forced, ksplit, layoutA, layoutB, M, N, K, alpha,
                    A, lda, B, ldb, beta, C, ldc, dtype, epilogue, stream, MGEMM_ERR_UNSUPPORTED,
                    h->stamps, h->stamps_cap);
}

}  // namespace
}  // namespace mgemm_host

using namespace mgemm_host;

extern "C" {

mgemm_status_t mgemm_create(mgemm_handle_t* out) {
    if (!out) return MGEMM_ERR_INVALID_ARG;
    *out = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MGEMM_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MGEMM_ERR_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MGEMM_ERR_UNSUPPORTED;
    mgemm_handle_s* h = new (std::nothrow) mgemm_handle_s;
    if (!h) return MGEMM_ERR_ALLOC;
    h->device = dev;
    h->num_cu = prop.multiProcessorCount;
    h->stamps = nullptr;
    h->stamps_cap = 0;
    h->ws = mgemm::Workspace{nullptr, 0, nullptr, 0};
    const int64_t part_bytes = (int64_t)128 << 20, ncounters = (int64_t)1 << 16;
    void* part = nullptr;
    void* cnt = nullptr;
    if (hipMalloc(&part, (size_t)part_bytes) != hipSuccess ||
        hipMalloc(&cnt, (size_t)ncounters * sizeof(unsigned)) != hipSuccess ||
        hipMemset(cnt, 0, (size_t)ncounters * sizeof(unsigned)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        if (part) (void)hipFree(part);
        if (cnt) (void)hipFree(cnt);
        delete h;
        return MGEMM_ERR_HIP;
    }
    h->ws = mgemm::Workspace{part, part_bytes, (unsigned*)cnt, ncounters};
    *out = h;
    return MGEMM_SUCCESS;
}

mgemm_status_t mgemm_destroy(mgemm_handle_t h) {
    if (!h) return MGEMM_SUCCESS;
    if (h->ws.part) (void)hipFree(h->ws.part);
    if (h->ws.counters) (void)hipFree(h->ws.counters);
    delete h;
    return MGEMM_SUCCESS;
}

mgemm_status_t mgemm_run(mgemm_handle_t h, mgemm_layout_t layoutA, mgemm_layout_t layoutB,
                         int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                         const void* B, int64_t ldb, float beta, void* C, int64_t ldc,
                         mgemm_dtype_t dtype, hipStream_t stream) {
    return run_impl(h, MGEMM_KERNEL_AUTO, 0, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta,
                    C, ldc, dtype, MGEMM_EPILOGUE_NONE, stream);
}

mgemm_status_t mgemm_run_kernel(mgemm_handle_t h, mgemm_kernel_t kernel, mgemm_layout_t layoutA,
                                mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                                float alpha, const void* A, int64_t lda, const void* B,
                                int64_t ldb, float beta, void* C, int64_t ldc,
                                mgemm_dtype_t dtype, hipStream_t stream) {
    if (kernel == MGEMM_KERNEL_AUTO) return MGEMM_ERR_INVALID_ARG;
    return run_impl(h, kernel, 0, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                    dtype, MGEMM_EPILOGUE_NONE, stream);
}

mgemm_status_t mgemm_run_ex(mgemm_handle_t h, mgemm_kernel_t kernel, mgemm_layout_t layoutA,
                            mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K, float alpha,
                            const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                            void* C, int64_t ldc, mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                            hipStream_t stream) {
    return run_impl(h, kernel, 0, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                    dtype, epilogue, stream);
}

mgemm_status_t mgemm_run_variant(mgemm_handle_t h, const mgemm_variant_t* v,
                                 mgemm_layout_t layoutA, mgemm_layout_t layoutB, int64_t M,
                                 int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, float beta, void* C, int64_t ldc,
                                 mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                                 hipStream_t stream) {
    const mgemm_kernel_t k = v ? (mgemm_kernel_t)v->kernel : MGEMM_KERNEL_AUTO;
    const int ks = v ? v->ksplit : 0;
    return run_impl(h, k, ks, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype,
                    epilogue, stream);
}

mgemm_status_t mgemm_run_gated(mgemm_handle_t h, int64_t M, int64_t N, int64_t K, const void* X,
                               int64_t ldx, const void* Wg, const void* Wu, int64_t ldw, void* Z,
                               int64_t ldz, mgemm_dtype_t dtype, hipStream_t stream) {
    return mgemm_run_gated_ex(h, 0, M, N, K, X, ldx, Wg, Wu, ldw, Z, ldz, dtype, stream);
}

mgemm_status_t mgemm_run_gated_ex(mgemm_handle_t h, int32_t ksplit, int64_t M, int64_t N, int64_t K,
                                  const void* X, int64_t ldx, const void* Wg, const void* Wu,
                                  int64_t ldw, void* Z, int64_t ldz, mgemm_dtype_t dtype,
                                  hipStream_t stream) {
    if (ksplit < 0 || ksplit > MGEMM_MAX_KSPLIT) return MGEMM_ERR_INVALID_ARG;
    if (dtype != MGEMM_F16 && dtype != MGEMM_BF16) {
        if (!valid_dtype(dtype)) return MGEMM_ERR_INVALID_ARG;
    }
    Problem p;
    mgemm_status_t st = make_problem(h, MGEMM_ROW_MAJOR, MGEMM_ROW_MAJOR, M, N, K, 1.0f, X, ldx,
                                     Wg, ldw, 0.0f, Z, ldz, dtype, &p);
    if (st != MGEMM_SUCCESS) return st;
    if (M > 0 && N > 0 && K > 0 && Wu == nullptr) return MGEMM_ERR_INVALID_ARG;
    if (dtype != MGEMM_F16 && dtype != MGEMM_BF16) return MGEMM_ERR_UNSUPPORTED;
    if (p.M == 0 || p.N == 0) return MGEMM_SUCCESS;
    p.B2 = Wu;
    p.ldb2 = ldw;
    p.stamps = h->stamps;
    p.stamps_cap = h->stamps ? h->stamps_cap : 0;
    if (p.K == 0) {
        // G = U = 0, so Z = SiLU(0) * 0 = 0.
        p.beta = 0.0f;
        hipError_t e = mgemm::launch_scale(p, stream);
        return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
    }
    if (!mgemm::h_gated_supports(p)) return MGEMM_ERR_UNSUPPORTED;
    // Tile height as for the plain product: 128-row tiles for M <= 128 or
    // weights small enough (both of them) to be shared through the
    // last-level cache, when the model predicts them faster.
    int bm = 256;
    if (p.M <= 128 || 2.0 * (double)p.K * (double)p.N * 2.0 <= 32.0 * 1024 * 1024) {
        double t256, t128;
        auto_split(p, 192, true, h->ws, &t256);
        auto_split(p, 192, true, h->ws, &t128, 128);
        if (t128 < t256) bm = 128;
    }
    const int ks = ksplit == 0 ? auto_split(p, 192, true, h->ws, nullptr, bm)
                               : mgemm::h_dma_splits(p, 192, true, ksplit, h->ws, bm);
    if (ks < 1) return MGEMM_ERR_UNSUPPORTED;
    hipError_t e = mgemm::launch_h_gated(p, ks, h->ws, stream, bm);
    return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
}

mgemm_status_t mgemm_quantize_fp8(mgemm_handle_t h, int64_t M, int64_t K, const void* X,
                                  int64_t ldx, mgemm_dtype_t xtype, void* Q, int64_t ldq,
                                  float* scales, hipStream_t stream) {
    if (!h || M < 0 || K < 0 || !valid_dtype(xtype)) return MGEMM_ERR_INVALID_ARG;
    if (ldx < (K > 1 ? K : 1) || ldq < (K > 1 ? K : 1)) return MGEMM_ERR_INVALID_ARG;
    const int64_t lim = (int64_t)1 << 62;
    if (M > lim / ldx || M > lim / ldq) return MGEMM_ERR_INVALID_ARG;
    if (M == 0) return MGEMM_SUCCESS;
    if (!scales || (K > 0 && (!X || !Q))) return MGEMM_ERR_INVALID_ARG;
    if ((M + 3) / 4 > 0x7fffffff) return MGEMM_ERR_INVALID_ARG;
    hipError_t e = mgemm::launch_quantize_fp8(M, K, X, ldx, (int)xtype, Q, ldq, scales, stream);
    return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
}

mgemm_status_t mgemm_run_fp8(mgemm_handle_t h, mgemm_kernel_t kernel, int32_t ksplit, int64_t M,
                             int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                             const float* sa, const void* B, int64_t ldb, const float* sb,
                             float beta, void* C, int64_t ldc, mgemm_dtype_t ctype,
                             hipStream_t stream) {
    if (!h || M < 0 || N < 0 || K < 0 || !valid_dtype(ctype)) return MGEMM_ERR_INVALID_ARG;
    if (ksplit < 0 || ksplit > MGEMM_MAX_KSPLIT || (kernel == MGEMM_KERNEL_AUTO && ksplit != 0))
        return MGEMM_ERR_INVALID_ARG;
    if (kernel != MGEMM_KERNEL_AUTO && kernel != MGEMM_KERNEL_F8_MFMA &&
        kernel != MGEMM_KERNEL_F8_MFMA_192 && kernel != MGEMM_KERNEL_F8_MFMA_128 &&
        kernel != MGEMM_KERNEL_F8_GENERAL)
        return MGEMM_ERR_INVALID_ARG;
    if (lda < max1(K) || ldb < max1(K) || ldc < max1(N)) return MGEMM_ERR_INVALID_ARG;
    const int64_t lim = (int64_t)1 << 62;
    if (M > lim / lda || N > lim / ldb || M > lim / ldc) return MGEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return MGEMM_SUCCESS;
    if (!C) return MGEMM_ERR_INVALID_ARG;
    Problem p;
    p.M = M; p.N = N; p.K = K;
    p.A = A; p.lda = lda; p.a_kc = 1;
    p.B = B; p.ldb = ldb; p.b_kc = 1;
    p.C = C; p.ldc = ldc;
    p.alpha = alpha; p.beta = beta;
    p.dtype = (int)ctype;
    p.num_cu = h->num_cu;
    p.epilogue = mgemm::EPI_NONE;
    p.B2 = nullptr;
    p.ldb2 = 0;
    p.stamps = h->stamps;
    p.stamps_cap = h->stamps ? h->stamps_cap : 0;
    if (K == 0 || alpha == 0.f) {
        hipError_t e = mgemm::launch_scale(p, stream);
        return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
    }
    if (!A || !B || !sa || !sb) return MGEMM_ERR_INVALID_ARG;
    // The MFMA kernel's time per (tile, split) by the 16-bit time model: a
    // 64-wide FP8 slice moves the bytes of a 32-wide 16-bit slice and measured
    // the same time per slice (0.59 us for 256x192 tiles at 1024x12288).  The
    // partials of a split are priced at 4.5 TB/s: timing every tile at 1-8
    // ranges on ten FP8 shapes, the 16-bit 2.6 TB/s kept 256x12288x4096 and
    // 2048x1536x4096 unsplit on 128x192 tiles (31.0 / 30.4 us) where 2 ranges
    // take 27.2 / 27.6 us; at 4.5 TB/s every pick is within 2.1% of the best.
    Problem q = p;
    q.K = p.K / 2;
    auto best_split = [&](int w, int bm, double* t_out) {
        int best = 1;
        double bt = 1e300;
        for (int req = 1, last = 0; req <= MGEMM_MAX_KSPLIT; ++req) {
            const int ks = mgemm::f8_splits_bm(p, w, bm, req, h->ws);
            if (ks <= last) continue;
            last = ks;
            const double t = predict_us(q, bm, w, w, w == 256 ? 1.4 : 1.3, 1, ks, 4.5e6);
            if (t < bt) { bt = t; best = ks; }
        }
        if (t_out) *t_out = bt;
        return best;
    };
    // MFMA tile width (0 = scalar kernel) and height, K ranges.
    int bn = -1, bm = 256, ks = 1;
    if (kernel == MGEMM_KERNEL_F8_MFMA || kernel == MGEMM_KERNEL_F8_MFMA_192 ||
        kernel == MGEMM_KERNEL_F8_MFMA_128) {
        bn = kernel == MGEMM_KERNEL_F8_MFMA ? 256 : 192;
        bm = kernel == MGEMM_KERNEL_F8_MFMA_128 ? 128 : 256;
        if (!mgemm::f8_mfma_supports_bm(p, bn, bm)) return MGEMM_ERR_UNSUPPORTED;
        ks = ksplit == 0 ? best_split(bn, bm, nullptr)
                         : mgemm::f8_splits_bm(p, bn, bm, ksplit, h->ws);
        if (ks < 1) return MGEMM_ERR_UNSUPPORTED;
    } else if (kernel == MGEMM_KERNEL_F8_GENERAL) {
        if (!mgemm::f8_general_supports(p)) return MGEMM_ERR_UNSUPPORTED;
        if (ksplit > 1) return MGEMM_ERR_UNSUPPORTED;
        bn = 0;
    } else {
        // 128-row tiles (width 192) where a grid of 256-row tiles leaves CUs
        // idle: FP8 4096x1536x4096, 128 tiles of 256x192, against 256 of 128x192.
        double best_t = 1e300;
        for (const auto& [w, tm] : {std::pair<int, int>{256, 256}, {192, 256}, {192, 128}}) {
            if (!mgemm::f8_mfma_supports_bm(p, w, tm)) continue;
            double t;
            const int k2 = best_split(w, tm, &t);
            if (t < best_t) { best_t = t; bn = w; bm = tm; ks = k2; }
        }
        if (bn < 0) {
            if (!mgemm::f8_general_supports(p)) return MGEMM_ERR_UNSUPPORTED;
            bn = 0;
        }
    }
    hipError_t e = mgemm::launch_f8_gemm_bm(p, sa, sb, bn, bm, ks, h->ws, stream);
    return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
}

mgemm_status_t mgemm_select_kernel(mgemm_handle_t h, mgemm_layout_t layoutA,
                                   mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                                   float alpha, const void* A, int64_t lda, const void* B,
                                   int64_t ldb, float beta, void* C, int64_t ldc,
                                   mgemm_dtype_t dtype, mgemm_kernel_t* kernel_out) {
    if (!kernel_out) return MGEMM_ERR_INVALID_ARG;
    Problem p;
    mgemm_status_t st = make_problem(h, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                     ldc, dtype, &p);
    if (st != MGEMM_SUCCESS) return st;
    if (p.M == 0 || p.N == 0 || p.K == 0 || p.alpha == 0.f) *kernel_out = MGEMM_KERNEL_AUTO;
    else *kernel_out = choose(h, p).k;
    return MGEMM_SUCCESS;
}

mgemm_status_t mgemm_run_acc32(mgemm_handle_t h, mgemm_kernel_t kernel, mgemm_layout_t layoutA,
                               mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                               float alpha, const void* A, int64_t lda, const void* B,
                               int64_t ldb, float* C32, int64_t ldc, mgemm_dtype_t dtype,
                               hipStream_t stream) {
    if (kernel != MGEMM_KERNEL_AUTO && kernel != MGEMM_KERNEL_H_DMA_256 &&
        kernel != MGEMM_KERNEL_H_DMA_192)
        return MGEMM_ERR_INVALID_ARG;
    Problem p;
    mgemm_status_t st = make_problem(h, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, 0.0f,
                                     C32, ldc, dtype, &p);
    if (st != MGEMM_SUCCESS) return st;
    if (dtype != MGEMM_F16 && dtype != MGEMM_BF16) return MGEMM_ERR_UNSUPPORTED;
    if (p.M == 0 || p.N == 0) return MGEMM_SUCCESS;
    if (p.K == 0 || alpha == 0.f) return MGEMM_ERR_UNSUPPORTED;
    int bn = kernel == MGEMM_KERNEL_H_DMA_192 ? 192 : 256;
    if (kernel == MGEMM_KERNEL_AUTO) {
        const Choice c = model_choice(p, h->ws);
        bn = c.k == MGEMM_KERNEL_H_DMA_192 ? 192 : 256;
        if (!mgemm::h_dma_supports(p, bn)) bn = bn == 256 ? 192 : 256;
    }
    if (!mgemm::h_dma_supports(p, bn)) return MGEMM_ERR_UNSUPPORTED;
    p.stamps = h->stamps;
    p.stamps_cap = h->stamps ? h->stamps_cap : 0;
    const hipError_t e = mgemm::launch_h_dma_acc32(p, bn, stream);
    return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
}

mgemm_status_t mgemm_select_variant(mgemm_handle_t h, mgemm_layout_t layoutA,
                                    mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                                    float alpha, const void* A, int64_t lda, const void* B,
                                    int64_t ldb, float beta, void* C, int64_t ldc,
                                    mgemm_dtype_t dtype, mgemm_variant_t* out) {
    if (!out) return MGEMM_ERR_INVALID_ARG;
    Problem p;
    mgemm_status_t st = make_problem(h, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                     ldc, dtype, &p);
    if (st != MGEMM_SUCCESS) return st;
    if (p.M == 0 || p.N == 0 || p.K == 0 || p.alpha == 0.f) {
        out->kernel = MGEMM_KERNEL_AUTO;
        out->ksplit = 0;
    } else {
        const Choice c = choose(h, p);
        out->kernel = c.k;
        out->ksplit = c.ksplit;
    }
    return MGEMM_SUCCESS;
}

const char* mgemm_status_string(mgemm_status_t s) {
    switch (s) {
    case MGEMM_SUCCESS: return "success";
    case MGEMM_ERR_INVALID_ARG: return "invalid argument";
    case MGEMM_ERR_UNSUPPORTED: return "unsupported";
    case MGEMM_ERR_HIP: return "HIP error";
    case MGEMM_ERR_ALLOC: return "allocation failed";
    case MGEMM_ERR_SCRATCH: return "needs more scratch memory than the no-allocation entry point holds";
    }
    return "unknown";
}

const char* mgemm_kernel_name(mgemm_kernel_t k) {
    switch (k) {
    case MGEMM_KERNEL_AUTO: return "auto";
    case MGEMM_KERNEL_GENERAL: return "general";
    case MGEMM_KERNEL_F32_MFMA: return "f32_mfma";
    case MGEMM_KERNEL_H_256x256: return "h_mfma_256x256";
    case MGEMM_KERNEL_H_256x192: return "h_mfma_256x192";
    case MGEMM_KERNEL_H_128x128: return "h_mfma_128x128";
    case MGEMM_KERNEL_SKINNY: return "skinny";
    case MGEMM_KERNEL_RESERVED_7: return "reserved_7";
    case MGEMM_KERNEL_F32_FAST: return "f32_fast";
    case MGEMM_KERNEL_F32_FAST_128: return "f32_fast_128";
    case MGEMM_KERNEL_H_DMA_256: return "h_dma_256x256";
    case MGEMM_KERNEL_H_DMA_192: return "h_dma_256x192";
    case MGEMM_KERNEL_F32_FAST_U: return "f32_fast_u";
    case MGEMM_KERNEL_SKINNY_SK: return "skinny_sk";
    case MGEMM_KERNEL_F8_MFMA: return "f8_mfma_256x256";
    case MGEMM_KERNEL_F8_GENERAL: return "f8_general";
    case MGEMM_KERNEL_F8_MFMA_192: return "f8_mfma_256x192";
    case MGEMM_KERNEL_F8_MFMA_128: return "f8_mfma_128x192";
    case MGEMM_KERNEL_F32_SK: return "f32_sk";
    case MGEMM_KERNEL_H_DMA_128: return "h_dma_128x192";
    case MGEMM_KERNEL_H_DMA_64: return "h_dma_64x192";
    default: return "unknown";
    }
}

int mgemm_num_cu(mgemm_handle_t h) { return h ? h->num_cu : 0; }

mgemm_status_t mgemm_set_clock_stamps(mgemm_handle_t h, uint64_t* buf, int64_t nblocks) {
    if (!h || nblocks < 0 || (buf != nullptr && nblocks == 0)) return MGEMM_ERR_INVALID_ARG;
    h->stamps = (unsigned long long*)buf;
    h->stamps_cap = buf ? nblocks : 0;
    return MGEMM_SUCCESS;
}

}  // extern "C"
