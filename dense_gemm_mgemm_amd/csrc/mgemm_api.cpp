// libmgemm host side: argument validation, normalisation to one canonical
// row-major problem, kernel selection and launch.  See include/mgemm.h for
// the contract of every entry point.
#include <hip/hip_runtime.h>

#include <new>
#include <string.h>

#include "../../include/mgemm.h"
#include "common.h"

struct mgemm_handle_s {
    int device;
    int num_cu;
    mgemm::Workspace ws;     // device memory owned by the handle
};

namespace {

using mgemm::Problem;

inline bool valid_layout(mgemm_layout_t l) { return l == MGEMM_ROW_MAJOR || l == MGEMM_COL_MAJOR; }
inline bool valid_dtype(mgemm_dtype_t d) { return d == MGEMM_F32 || d == MGEMM_F16 || d == MGEMM_BF16; }
inline int64_t max1(int64_t x) { return x > 1 ? x : 1; }

// Checks the rules of mgemm_run and builds the canonical problem.
mgemm_status_t make_problem(mgemm_handle_t h, mgemm_layout_t layoutA, mgemm_layout_t layoutB,
                            int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                            int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                            int64_t ldc, mgemm_dtype_t dtype, Problem* out) {
    if (!h || !valid_layout(layoutA) || !valid_layout(layoutB) || !valid_dtype(dtype))
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
    p.num_cu = h->num_cu;
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

bool variant_supports(const Problem& p, mgemm_kernel_t k) {
    switch (k) {
    case MGEMM_KERNEL_GENERAL: return true;
    case MGEMM_KERNEL_F32_MFMA: return mgemm::f32_mfma_supports(p);
    case MGEMM_KERNEL_H_256x256:
    case MGEMM_KERNEL_H_256x192:
    case MGEMM_KERNEL_H_128x128: return mgemm::h_mfma_supports(p, (int)k);
    case MGEMM_KERNEL_SKINNY: return mgemm::skinny_supports(p);
    case MGEMM_KERNEL_H_PP_256: return mgemm::h_pp_supports(p);
    case MGEMM_KERNEL_F32_FAST: return mgemm::f32_fast_supports(p, true);
    case MGEMM_KERNEL_F32_FAST_128: return mgemm::f32_fast_supports(p, false);
    case MGEMM_KERNEL_H_DMA_256: return mgemm::h_dma_supports(p, 256);
    case MGEMM_KERNEL_H_DMA_192: return mgemm::h_dma_supports(p, 192);
    case MGEMM_KERNEL_F32_FAST_U: return mgemm::f32_unaligned_supports(p);
    case MGEMM_KERNEL_SKINNY_SK: return mgemm::skinny_sk_supports(p);
    default: return false;
    }
}

// Kernel choice for a canonical problem.
mgemm_kernel_t choose(const Problem& p) {
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
        const bool big = mgemm::f32_fast_supports(p, true), small = mgemm::f32_fast_supports(p, false);
        if (big && (!small || fill(256, 256, 1) >= fill(128, 128, 2) * 0.9))
            return MGEMM_KERNEL_F32_FAST;
        if (small) return MGEMM_KERNEL_F32_FAST_128;
        // NN operands that are not 16-byte aligned or a K that is not a
        // multiple of the slice: the same kernel with narrower loads.
        if (mgemm::f32_unaligned_supports(p)) return MGEMM_KERNEL_F32_FAST_U;
        return MGEMM_KERNEL_F32_MFMA;
    }
    // M <= 64 streams B once: 256-column blocks with K split over workgroups
    // read B in 512-byte row segments (about 5.1 TB/s in copy-only
    // measurements, against 4.2 TB/s for the 128-byte segments of the
    // whole-K kernel).
    if (p.M <= 64 && mgemm::skinny_sk_supports(p)) return MGEMM_KERNEL_SKINNY_SK;
    if (p.M <= 64 && mgemm::skinny_supports(p)) return MGEMM_KERNEL_SKINNY;
    // 16-bit: score each variant by the fraction of CU-time its grid spends
    // on useful outputs (wave quantisation and the padding of ragged edge
    // tiles count as waste) times its measured per-CU speed relative to the
    // register-staged kernel.  The four-wave direct-to-LDS kernel runs a full
    // 256x256 tile about 1.4x as fast (1024 NN tiles: 2.12 vs 2.58 ms); its
    // 256x192 form moves more bytes per flop and is preferred only where the
    // narrower tile fills the CUs clearly better.
    struct Cand { mgemm_kernel_t k; int bm, bn; double speed; };
    const Cand cands[5] = {{MGEMM_KERNEL_H_DMA_256, 256, 256, 1.4},
                           {MGEMM_KERNEL_H_DMA_192, 256, 192, 1.3},
                           {MGEMM_KERNEL_H_256x256, 256, 256, 1.0},
                           {MGEMM_KERNEL_H_256x192, 256, 192, 1.0},
                           {MGEMM_KERNEL_H_128x128, 128, 128, 1.0}};
    mgemm_kernel_t best = MGEMM_KERNEL_GENERAL;
    double best_score = -1.0;
    for (const Cand& c : cands) {
        const bool ok = c.k == MGEMM_KERNEL_H_DMA_256   ? mgemm::h_dma_supports(p, 256)
                        : c.k == MGEMM_KERNEL_H_DMA_192 ? mgemm::h_dma_supports(p, 192)
                                                        : mgemm::h_mfma_supports(p, (int)c.k);
        if (!ok) continue;
        const double score = fill(c.bm, c.bn, 1) * c.speed;
        if (score > best_score + 1e-9) { best_score = score; best = c.k; }
    }
    return best;
}

mgemm_status_t launch(mgemm_handle_t h, const Problem& p, mgemm_kernel_t k, hipStream_t s) {
    hipError_t e;
    switch (k) {
    case MGEMM_KERNEL_SKINNY_SK: e = mgemm::launch_skinny_sk(p, h->ws, s); break;
    case MGEMM_KERNEL_GENERAL: e = mgemm::launch_general(p, s); break;
    case MGEMM_KERNEL_F32_MFMA: e = mgemm::launch_f32_mfma(p, s); break;
    case MGEMM_KERNEL_H_256x256:
    case MGEMM_KERNEL_H_256x192:
    case MGEMM_KERNEL_H_128x128: e = mgemm::launch_h_mfma(p, (int)k, s); break;
    case MGEMM_KERNEL_SKINNY: e = mgemm::launch_skinny(p, s); break;
    case MGEMM_KERNEL_H_PP_256: e = mgemm::launch_h_pp(p, s); break;
    case MGEMM_KERNEL_F32_FAST: e = mgemm::launch_f32_fast(p, true, s); break;
    case MGEMM_KERNEL_F32_FAST_128: e = mgemm::launch_f32_fast(p, false, s); break;
    case MGEMM_KERNEL_H_DMA_256: e = mgemm::launch_h_dma(p, 256, s); break;
    case MGEMM_KERNEL_H_DMA_192: e = mgemm::launch_h_dma(p, 192, s); break;
    case MGEMM_KERNEL_F32_FAST_U: e = mgemm::launch_f32_unaligned(p, s); break;
    default: return MGEMM_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
}

mgemm_status_t run_impl(mgemm_handle_t h, mgemm_kernel_t forced, mgemm_layout_t layoutA,
                        mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                        void* C, int64_t ldc, mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                        hipStream_t stream) {
    Problem p;
    mgemm_status_t st = make_problem(h, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                     ldc, dtype, &p);
    if (st != MGEMM_SUCCESS) return st;
    if (forced != MGEMM_KERNEL_AUTO && (forced <= 0 || forced >= MGEMM_KERNEL_COUNT))
        return MGEMM_ERR_INVALID_ARG;
    if (epilogue != MGEMM_EPILOGUE_NONE && epilogue != MGEMM_EPILOGUE_SILU)
        return MGEMM_ERR_INVALID_ARG;
    p.epilogue = epilogue == MGEMM_EPILOGUE_SILU ? mgemm::EPI_SILU : mgemm::EPI_NONE;
    if (p.M == 0 || p.N == 0) return MGEMM_SUCCESS;
    if (p.K == 0 || p.alpha == 0.f) {
        hipError_t e = mgemm::launch_scale(p, stream);
        return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
    }
    mgemm_kernel_t k = forced == MGEMM_KERNEL_AUTO ? choose(p) : forced;
    if (!variant_supports(p, k)) return MGEMM_ERR_UNSUPPORTED;
    return launch(h, p, k, stream);
}

}  // namespace

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
    h->ws = mgemm::Workspace{nullptr, 0, nullptr, 0};
    const int64_t part_bytes = (int64_t)32 << 20, ncounters = (int64_t)1 << 16;
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
    return run_impl(h, MGEMM_KERNEL_AUTO, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                    ldc, dtype, MGEMM_EPILOGUE_NONE, stream);
}

mgemm_status_t mgemm_run_kernel(mgemm_handle_t h, mgemm_kernel_t kernel, mgemm_layout_t layoutA,
                                mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                                float alpha, const void* A, int64_t lda, const void* B,
                                int64_t ldb, float beta, void* C, int64_t ldc,
                                mgemm_dtype_t dtype, hipStream_t stream) {
    if (kernel == MGEMM_KERNEL_AUTO) return MGEMM_ERR_INVALID_ARG;
    return run_impl(h, kernel, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                    dtype, MGEMM_EPILOGUE_NONE, stream);
}

mgemm_status_t mgemm_run_ex(mgemm_handle_t h, mgemm_kernel_t kernel, mgemm_layout_t layoutA,
                            mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K, float alpha,
                            const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                            void* C, int64_t ldc, mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                            hipStream_t stream) {
    return run_impl(h, kernel, layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                    dtype, epilogue, stream);
}

mgemm_status_t mgemm_run_gated(mgemm_handle_t h, int64_t M, int64_t N, int64_t K, const void* X,
                               int64_t ldx, const void* Wg, const void* Wu, int64_t ldw, void* Z,
                               int64_t ldz, mgemm_dtype_t dtype, hipStream_t stream) {
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
    if (p.K == 0) {
        // G = U = 0, so Z = SiLU(0) * 0 = 0.
        p.beta = 0.0f;
        hipError_t e = mgemm::launch_scale(p, stream);
        return e == hipSuccess ? MGEMM_SUCCESS : MGEMM_ERR_HIP;
    }
    if (!mgemm::h_gated_supports(p)) return MGEMM_ERR_UNSUPPORTED;
    hipError_t e = mgemm::launch_h_gated(p, stream);
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
    else *kernel_out = choose(p);
    return MGEMM_SUCCESS;
}

const char* mgemm_status_string(mgemm_status_t s) {
    switch (s) {
    case MGEMM_SUCCESS: return "success";
    case MGEMM_ERR_INVALID_ARG: return "invalid argument";
    case MGEMM_ERR_UNSUPPORTED: return "unsupported";
    case MGEMM_ERR_HIP: return "HIP error";
    case MGEMM_ERR_ALLOC: return "allocation failed";
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
    case MGEMM_KERNEL_H_PP_256: return "h_pp_256x256";
    case MGEMM_KERNEL_F32_FAST: return "f32_fast";
    case MGEMM_KERNEL_F32_FAST_128: return "f32_fast_128";
    case MGEMM_KERNEL_H_DMA_256: return "h_dma_256x256";
    case MGEMM_KERNEL_H_DMA_192: return "h_dma_256x192";
    case MGEMM_KERNEL_F32_FAST_U: return "f32_fast_u";
    case MGEMM_KERNEL_SKINNY_SK: return "skinny_sk";
    default: return "unknown";
    }
}

int mgemm_num_cu(mgemm_handle_t h) { return h ? h->num_cu : 0; }

}  // extern "C"
