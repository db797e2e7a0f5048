/*
 * mgemm.h -- C ABI of libmgemm, dense matrix multiplication for AMD Instinct
 * MI355X (gfx950).
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * The operation is the GEMM of the SGEMM report "SGEMM measurements and three
 * ledgers" (daleiyang; the naive kernel K1 stores alpha*acc + beta*C) with the
 * (A, B, C, M, N, K, alpha, beta) signature of the zwxr.cn SGEMM post
 * (section 3.3).  FP16/BF16 inputs accumulate in FP32 and are rounded once to
 * the output format at the end ("Chapter 5: Operators and Runtime",
 * ai-infra-book, sections 5.2.1 and 5.4.2, round_to_bf16(acc); the MTT S4000
 * FP16 GEMM write-up, section 1, FP16 in/out with FP32 accumulation).
 * Row-major and column-major storage are related by the transpose identity of
 * the SGEMM report (section "how the cuBLAS denominator was fixed"): row-major
 * C = A B is the same bytes as column-major C^T = B^T A^T.
 *
 * All entry points are plain C.  Pointers passed as A, B, C are DEVICE
 * pointers (HIP device memory of the handle's GPU).  Sizes and leading
 * dimensions are counted in elements.
 */
#ifndef MGEMM_H_
#define MGEMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream type, declared here so this header needs no HIP include. */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    MGEMM_SUCCESS = 0,
    MGEMM_ERR_INVALID_ARG = 1,   /* bad size, enum, leading dimension or null pointer */
    MGEMM_ERR_UNSUPPORTED = 2,   /* device is not gfx950, or a forced kernel cannot run the problem */
    MGEMM_ERR_HIP = 3,           /* a HIP runtime call or kernel launch failed */
    MGEMM_ERR_ALLOC = 4,         /* host allocation failed */
    MGEMM_ERR_SCRATCH = 5        /* mgemm_run_noalloc: the forced variant needs more scratch
                                    memory than the library's static array holds */
} mgemm_status_t;

typedef enum {
    MGEMM_ROW_MAJOR = 0,         /* element (r, c) at r*ld + c */
    MGEMM_COL_MAJOR = 1          /* element (r, c) at c*ld + r */
} mgemm_layout_t;

typedef enum {
    MGEMM_F32 = 0,               /* A, B, C in IEEE binary32; FP32 products and sums */
    MGEMM_F16 = 1,               /* A, B, C in IEEE binary16; FP32 accumulation */
    MGEMM_BF16 = 2               /* A, B, C in bfloat16; FP32 accumulation */
} mgemm_dtype_t;

/* Kernel variants.  MGEMM_KERNEL_AUTO lets the library choose; the others
 * force one code path (each must produce the same result to the stated
 * tolerance; tests run every one of them). */
typedef enum {
    MGEMM_KERNEL_AUTO = 0,
    MGEMM_KERNEL_GENERAL = 1,    /* any dtype/layout/alignment, VALU FMA, 64x64 tiles */
    MGEMM_KERNEL_F32_MFMA = 2,   /* FP32 on v_mfma_f32_32x32x2_f32, 128x128 tiles, any layout */
    MGEMM_KERNEL_H_256x256 = 3,  /* FP16/BF16 MFMA, 256x256 tiles, any layout; operands
                                    4-byte aligned (16-byte: vector loads, else buffer loads) */
    MGEMM_KERNEL_H_256x192 = 4,  /* FP16/BF16 MFMA, 256x192 tiles, as above */
    MGEMM_KERNEL_H_128x128 = 5,  /* FP16/BF16 MFMA, 128x128 tiles, any layout; operands 2-byte
                                    aligned (2-byte loads where not 4-byte aligned) */
    MGEMM_KERNEL_SKINNY = 6,     /* FP16/BF16, M <= 64, streams B once (memory bound) */
    MGEMM_KERNEL_RESERVED_7 = 7, /* no longer built (an 8-wave variant that no shape chose);
                                    forcing it returns MGEMM_ERR_UNSUPPORTED */
    MGEMM_KERNEL_F32_FAST = 8,   /* FP32 (any layout pair), 16-byte aligned operands, K % 32 == 0,
                                    256x256x32 tiles, 16 waves */
    MGEMM_KERNEL_F32_FAST_128 = 9, /* FP32 NN, 16-byte aligned operands, 128x128x16 tiles */
    MGEMM_KERNEL_H_DMA_256 = 10, /* FP16/BF16 (any layout pair), 256x256 tiles, 4 waves of 128x128,
                                    direct-to-LDS ring */
    MGEMM_KERNEL_SKINNY_SK = 11, /* FP16/BF16, M <= 64, 256-column blocks, K split over workgroups */
    MGEMM_KERNEL_H_DMA_192 = 12, /* FP16/BF16 (any layout pair), 256x192 tiles, 4 waves of 128x96,
                                    direct-to-LDS ring */
    MGEMM_KERNEL_F32_FAST_U = 13, /* FP32 NN, any alignment and K: 256x256x32 tiles, narrower loads */
    MGEMM_KERNEL_F8_MFMA = 14,   /* FP8 codes (mgemm_run_fp8 only): 256x256 tiles, f8f6f4 MFMA */
    MGEMM_KERNEL_F8_GENERAL = 15, /* FP8 codes (mgemm_run_fp8 only): any K/alignment, VALU */
    MGEMM_KERNEL_F8_MFMA_192 = 16, /* FP8 codes (mgemm_run_fp8 only): 256x192 tiles, f8f6f4 MFMA */
    MGEMM_KERNEL_F32_SK = 17,    /* FP32 NN as F32_FAST_U, stream-K: one workgroup per CU, equal
                                    shares of all (tile, K slice) pairs, deterministic fix-up */
    MGEMM_KERNEL_H_DMA_128 = 18, /* FP16/BF16, A' K-contiguous (row-major A), 128x192 tiles, 4 waves
                                    of 64x96, direct-to-LDS ring (short M) */
    MGEMM_KERNEL_H_DMA_64 = 19,  /* FP16/BF16, A' K-contiguous, 64x192 tiles, 4 waves of 32x96,
                                    direct-to-LDS ring (M <= 64 beyond the skinny kernels'
                                    shapes: streams B from HBM with a K split; also small
                                    grids with a small B) */
    MGEMM_KERNEL_F8_MFMA_128 = 20, /* FP8 codes (mgemm_run_fp8 only): 128x192 tiles, 4 waves of
                                      64x96, f8f6f4 MFMA (grids of 256-row tiles that leave CUs
                                      idle) */
    MGEMM_KERNEL_COUNT = 21
} mgemm_kernel_t;

/* Output epilogues (see mgemm_run_ex). */
typedef enum {
    MGEMM_EPILOGUE_NONE = 0,     /* C = round(alpha*op(A)*op(B) + beta*C) */
    MGEMM_EPILOGUE_SILU = 1      /* C = round(SiLU(round(alpha*op(A)*op(B) + beta*C))) */
} mgemm_epilogue_t;

typedef struct mgemm_handle_s* mgemm_handle_t;

/* A kernel variant with its split of K (see mgemm_run_variant). */
#define MGEMM_MAX_KSPLIT 32
typedef struct mgemm_variant {
    int32_t kernel;   /* an mgemm_kernel_t; MGEMM_KERNEL_AUTO = the library's choice */
    int32_t ksplit;   /* K ranges: 0 = the library's choice, 1 = all of K in one
                         workgroup per tile, 2 .. MGEMM_MAX_KSPLIT = at most that many */
} mgemm_variant_t;

/*
 * mgemm_create -- bind a handle to the CURRENT HIP device.
 *   out : receives the handle (owned by the caller, release with mgemm_destroy).
 * Returns MGEMM_ERR_UNSUPPORTED if the device is not gfx950, MGEMM_ERR_HIP if
 * the device cannot be queried or its workspace cannot be allocated,
 * MGEMM_ERR_INVALID_ARG if out is NULL.
 * The handle owns a device workspace (128 MiB of FP32 partial results plus
 * 64 Ki arrival counters, allocated and zeroed here) that the split-K and
 * stream-K forms use: calls that run at the same time on different streams must use
 * different handles; calls on one stream (or otherwise ordered) may share one.
 * The counters return to zero at the end of every call that uses them.
 */
mgemm_status_t mgemm_create(mgemm_handle_t* out);

/* mgemm_destroy -- release a handle and its workspace (NULL is accepted and
 * ignored).  No work enqueued with the handle may still be pending. */
mgemm_status_t mgemm_destroy(mgemm_handle_t h);

/*
 * mgemm_run -- enqueue C = alpha*op(A)*op(B) + beta*C on `stream`.
 *
 *   layoutA, layoutB : storage order of the logical A (M x K) and B (K x N).
 *   C (M x N) is stored in layoutA's order (one order for the call, as in
 *   cblas).  Leading dimensions must satisfy
 *       A: lda >= max(1, layoutA == ROW ? K : M)
 *       B: ldb >= max(1, layoutB == ROW ? N : K)
 *       C: ldc >= max(1, layoutA == ROW ? N : M)
 *   M, N, K >= 0.  M == 0 or N == 0 does nothing.  K == 0 or alpha == 0 gives
 *   C = beta*C and does not read A or B.  beta == 0 never reads C (it may hold
 *   NaN).  A and B must not overlap C.
 *   alpha, beta : FP32 scalars by value.
 *   dtype : element type of A, B and C.
 *   stream : HIP stream of the handle's device (0 = the null stream).
 *
 * Asynchronous: returns once the kernel is enqueued, with no device
 * synchronisation.  The caller owns A, B, C and keeps them alive until the
 * stream's work has completed.  No alignment is required: operands that are
 * not 16-byte aligned (or whose leading dimension breaks the alignment of a
 * row) take a narrower load path (FP16/BF16: the register-staged MFMA kernel
 * with buffer loads while A and B are at least 2-byte aligned and their
 * leading dimensions below 2^22; FP32: narrower loads by alignment).
 * Errors: MGEMM_ERR_INVALID_ARG for a violated rule above (nothing enqueued);
 * MGEMM_ERR_HIP if the launch fails.
 */
mgemm_status_t mgemm_run(mgemm_handle_t h, mgemm_layout_t layoutA, mgemm_layout_t layoutB,
                         int64_t M, int64_t N, int64_t K, float alpha,
                         const void* A, int64_t lda, const void* B, int64_t ldb,
                         float beta, void* C, int64_t ldc, mgemm_dtype_t dtype,
                         hipStream_t stream);

/*
 * mgemm_run_kernel -- as mgemm_run, but force one kernel variant.
 * Returns MGEMM_ERR_UNSUPPORTED (nothing enqueued) when that variant cannot
 * run this problem (wrong dtype, alignment or shape class; for
 * MGEMM_KERNEL_F32_SK also more than 64 Ki tiles or a device with more than
 * 256 CUs, whose two 256 KiB partial tiles per CU exceed the workspace).
 * MGEMM_KERNEL_F32_SK sums the pieces of a split tile in K order, so its
 * results are the same on every run of one problem on one device.  Used to check
 * every dispatch branch against the same reference, so that no branch goes
 * untested (the lesson of the MTT S4000 GEMM write-up, section 8).
 */
mgemm_status_t mgemm_run_kernel(mgemm_handle_t h, mgemm_kernel_t kernel,
                                mgemm_layout_t layoutA, mgemm_layout_t layoutB,
                                int64_t M, int64_t N, int64_t K, float alpha,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                float beta, void* C, int64_t ldc, mgemm_dtype_t dtype,
                                hipStream_t stream);

/*
 * mgemm_run_ex -- as mgemm_run (kernel == MGEMM_KERNEL_AUTO) or
 * mgemm_run_kernel (a forced variant), with an output epilogue.
 *   epilogue == MGEMM_EPILOGUE_SILU: the fused projection Y = SiLU(XW) of
 *   "Chapter 5: Operators and Runtime" (ai-infra-book), sections 5.4.2 and
 *   5.4.3.  Each output v = alpha*acc + beta*C (FP32) is first rounded to the
 *   output type, exactly as mgemm_run would store it; then
 *   SiLU(x) = x / (1 + e^-x) is evaluated in FP32 on that rounded value and
 *   the result is rounded once more and stored.  The activation therefore
 *   always follows the complete K sum.  K == 0 or alpha == 0 gives
 *   SiLU(round(beta*C)).  Every kernel variant supports both epilogues.
 * Errors: as mgemm_run / mgemm_run_kernel; MGEMM_ERR_INVALID_ARG for an
 * unknown epilogue (nothing enqueued).
 */
mgemm_status_t mgemm_run_ex(mgemm_handle_t h, mgemm_kernel_t kernel, mgemm_layout_t layoutA,
                            mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K, float alpha,
                            const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                            void* C, int64_t ldc, mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                            hipStream_t stream);

/*
 * mgemm_run_variant -- as mgemm_run_ex, with the variant given as a kernel and
 * a split of K.
 *   v : NULL or {MGEMM_KERNEL_AUTO, 0} lets the library choose both;
 *       {kernel, 0} forces the kernel and lets the library choose its split;
 *       {kernel, n} forces both.  A forced kernel with AUTO is invalid.
 * Split K: K is cut into ranges of whole 32-element slices, one workgroup
 * per output tile and range, and the ranges' FP32 partial sums are added in
 * range order, never with atomics (the MTT S4000 write-up, section 21, found
 * atomically accumulated split-K unusable; "Chapter 5: Operators and
 * Runtime", section 5.2.4: the order of a floating-point sum changes its last
 * bits), so a given variant gives the same bits on every run; different
 * splits round differently (within the tolerance of the sum).
 * Only MGEMM_KERNEL_H_DMA_256, MGEMM_KERNEL_H_DMA_192, MGEMM_KERNEL_H_DMA_128,
 * MGEMM_KERNEL_H_DMA_64 and MGEMM_KERNEL_SKINNY_SK take ksplit > 1 (MGEMM_KERNEL_F32_SK balances K
 * itself and takes 0 or 1); the number of ranges used is
 * ceil(S / ceil(S / ksplit)) for S = K / 32 slices.  The direct-to-LDS kernels
 * then run in two launches on `stream` (partial products, then the sum and
 * the epilogue); the partials live in the handle's workspace.
 * Errors: as mgemm_run_ex; MGEMM_ERR_INVALID_ARG for ksplit < 0 or
 * > MGEMM_MAX_KSPLIT, or a forced split with MGEMM_KERNEL_AUTO;
 * MGEMM_ERR_UNSUPPORTED for ksplit > 1 on another kernel or partials that
 * do not fit the workspace (nothing enqueued).
 */
mgemm_status_t mgemm_run_variant(mgemm_handle_t h, const mgemm_variant_t* v,
                                 mgemm_layout_t layoutA, mgemm_layout_t layoutB, int64_t M,
                                 int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, float beta, void* C, int64_t ldc,
                                 mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                                 hipStream_t stream);

/*
 * mgemm_run_acc32 -- the FP32 sums behind a 16-bit product, before the output
 * rounding: C32 = alpha * op(A) * op(B) in FP32, from the same direct-to-LDS
 * kernel and tile mgemm_run uses for large 16-bit products, unsplit.  The
 * MTT S4000 FP16 GEMM write-up grades FP16 outputs against an absolute
 * tolerance (0.01 * sqrt(K/512)) that the FP16 spacing itself exceeds for
 * large outputs; these sums let a check hold the accumulation to that bare
 * tolerance apart from the output format's rounding.  mgemm_run_variant with
 * the same kernel, one K range and beta = 0 stores exactly these values
 * rounded once to dtype (round to nearest even).
 *   kernel : MGEMM_KERNEL_AUTO (the tile width mgemm_run would pick for an
 *            unsplit product), MGEMM_KERNEL_H_DMA_256 or MGEMM_KERNEL_H_DMA_192.
 *   A, B   : dtype MGEMM_F16 or MGEMM_BF16, layouts and leading dimensions as
 *            for mgemm_run.
 *   C32    : device FP32 M x N in layoutA's order with leading dimension ldc
 *            (elements), written only; beta is not applied.
 * Errors: MGEMM_ERR_INVALID_ARG as mgemm_run, or for another kernel;
 * MGEMM_ERR_UNSUPPORTED for MGEMM_F32, K = 0 or below 32 (K need not be a
 * multiple of 32), alpha = 0, or operands the kernel cannot read (leading
 * dimensions not multiples of 8, bases not 16-byte aligned).  M or N = 0 is a
 * no-op.
 */
mgemm_status_t mgemm_run_acc32(mgemm_handle_t h, mgemm_kernel_t kernel, mgemm_layout_t layoutA,
                               mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                               float alpha, const void* A, int64_t lda, const void* B,
                               int64_t ldb, float* C32, int64_t ldc, mgemm_dtype_t dtype,
                               hipStream_t stream);

/*
 * mgemm_select_variant -- the variant (kernel and number of K ranges)
 * mgemm_run would launch; validation as mgemm_select_kernel.  out->kernel is
 * MGEMM_KERNEL_AUTO (and out->ksplit 0) when nothing or only a scaling of C
 * would be launched.
 */
mgemm_status_t mgemm_select_variant(mgemm_handle_t h, mgemm_layout_t layoutA,
                                    mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                                    float alpha, const void* A, int64_t lda, const void* B,
                                    int64_t ldb, float beta, void* C, int64_t ldc,
                                    mgemm_dtype_t dtype, mgemm_variant_t* out);

/*
 * mgemm_run_gated -- the gated FFN pair Z = SiLU(X * W_g) (.) (X * W_u) in one
 * kernel ("Chapter 5: Operators and Runtime" (ai-infra-book), section 5.3.1:
 * G = X W_g, U = X W_u, Z = SiLU(G) multiplied elementwise by U; fused, the
 * intermediate results keep their rounding, Figure 5-14).
 *   X   : M x K, row-major, leading dimension ldx >= max(1, K);
 *   W_g, W_u : K x N each, row-major, one shared leading dimension
 *         ldw >= max(1, N);
 *   Z   : M x N, row-major, ldz >= max(1, N); written, never read.
 *   dtype : MGEMM_F16 or MGEMM_BF16 for all four matrices.
 * Per output, with FP32 sums g and u over the whole K range:
 *   Z = round(round(SiLU(round(g))) * round(u))
 * (G, U and T = SiLU(G) rounded as if they were stored tensors).  K == 0
 * gives Z = 0.  Asynchronous on `stream`, like mgemm_run.
 * Errors: MGEMM_ERR_INVALID_ARG for a violated size/leading-dimension rule or
 * a NULL pointer with a nonzero extent; MGEMM_ERR_UNSUPPORTED for MGEMM_F32,
 * 0 < K < 32, N % 8 != 0, leading dimensions that are not multiples of 8
 * or bases that are not 16-byte aligned (nothing enqueued);
 * MGEMM_ERR_HIP if the launch fails.
 */
mgemm_status_t mgemm_run_gated(mgemm_handle_t h, int64_t M, int64_t N, int64_t K, const void* X,
                               int64_t ldx, const void* Wg, const void* Wu, int64_t ldw, void* Z,
                               int64_t ldz, mgemm_dtype_t dtype, hipStream_t stream);

/*
 * mgemm_run_gated_ex -- mgemm_run_gated with a split of K: ksplit 0 lets the
 * library choose, 1 keeps all of K in one workgroup per tile, 2 ..
 * MGEMM_MAX_KSPLIT cuts K into at most that many ranges as mgemm_run_variant
 * describes (G and U are both summed in range order before the epilogue).
 * Errors: as mgemm_run_gated; MGEMM_ERR_INVALID_ARG for ksplit < 0 or
 * > MGEMM_MAX_KSPLIT; MGEMM_ERR_UNSUPPORTED when the partials do not fit the
 * workspace.
 */
mgemm_status_t mgemm_run_gated_ex(mgemm_handle_t h, int32_t ksplit, int64_t M, int64_t N, int64_t K,
                                  const void* X, int64_t ldx, const void* Wg, const void* Wu,
                                  int64_t ldw, void* Z, int64_t ldz, mgemm_dtype_t dtype,
                                  hipStream_t stream);

/*
 * mgemm_select_kernel -- the variant mgemm_run would launch for this problem
 * (validates the arguments exactly as mgemm_run does; pointers are only
 * inspected for alignment and may be any value with the intended alignment).
 *   kernel_out : receives the chosen variant; MGEMM_KERNEL_AUTO means the call
 *   would launch nothing (M == 0 or N == 0) or only scale C (K == 0 or
 *   alpha == 0).
 */
mgemm_status_t mgemm_select_kernel(mgemm_handle_t h, mgemm_layout_t layoutA,
                                   mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                                   float alpha, const void* A, int64_t lda, const void* B,
                                   int64_t ldb, float beta, void* C, int64_t ldc,
                                   mgemm_dtype_t dtype, mgemm_kernel_t* kernel_out);

/*
 * Dispatch table tuned by measurement ("Chapter 5: Operators and Runtime"
 * (ai-infra-book), section 5.4.5: rule out what cannot run, then time the
 * remaining candidates on representative shapes and keep the cheapest;
 * Example 5-9: when one choice must serve several shapes, the cheapest is the
 * one with the smallest total time weighted by each shape's call count;
 * section 5.5.3: similar shapes share a choice through buckets).
 *
 * The handle holds a table consulted by mgemm_run, mgemm_run_ex,
 * mgemm_run_variant with MGEMM_KERNEL_AUTO, and mgemm_select_*:
 *   1. an exact entry for the problem's canonical shape (after the
 *      column-major transpose identity), dtype and operand layouts;
 *   2. else a bucket entry: M, N and K each rounded up to a power of two;
 *   3. else the built-in time model.
 * An entry whose variant cannot run the call (e.g. operands less aligned
 * than when it was tuned) falls through to the next step.  Entries never
 * change results beyond the choice of variant; every variant is
 * parity-tested.  The table must not be changed while another call uses the
 * handle.
 */
typedef struct mgemm_tune_result {
    mgemm_variant_t chosen;   /* fastest measured variant (kernel, ranges requested) */
    float chosen_us;          /* its mean time per call, microseconds */
    mgemm_variant_t model;    /* what the built-in model picks (ranges used) */
    float model_us;           /* its measured mean time per call */
} mgemm_tune_result_t;

/*
 * mgemm_tune -- measure every variant that can run each of the n shapes
 * (M[i] x N[i] x K[i], this dtype and these layouts, alpha = 1, beta = 0) on
 * `stream`, add an exact table entry per shape with the fastest, and one
 * entry per bucket with the variant of smallest sum of calls[i] * time over
 * the bucket's shapes (calls NULL: one call each).  Split-capable kernels
 * are measured at splits 1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 24 and 32.
 * Operands are allocated on the device inside this call (hipMalloc) and
 * filled with small exact values; the call blocks until the measurements are
 * done and releases them.  results: NULL or n entries, filled per shape.
 * Errors: MGEMM_ERR_INVALID_ARG for n < 1, a NULL array, a size < 1 or a
 * negative call count; MGEMM_ERR_UNSUPPORTED if no variant runs a shape;
 * MGEMM_ERR_HIP for an allocation or launch failure.
 */
mgemm_status_t mgemm_tune(mgemm_handle_t h, mgemm_dtype_t dtype, mgemm_layout_t layoutA,
                          mgemm_layout_t layoutB, int32_t n, const int64_t* M, const int64_t* N,
                          const int64_t* K, const double* calls, mgemm_tune_result_t* results,
                          hipStream_t stream);

/*
 * mgemm_table_export -- the handle's table as text, one entry per line:
 *     exact  <dtype> <a_kc> <b_kc> <M> <N> <K> <kernel name> <ksplit> <us>
 *     bucket <dtype> <a_kc> <b_kc> <log2 M> <log2 N> <log2 K> <kernel name> <ksplit> <us>
 * (canonical problem: a_kc/b_kc = 1 when A'/B' rows are K-contiguous; us =
 * measured time, for a bucket the call-weighted total).  Writes at most cap
 * bytes including the terminating NUL; *len receives the full length
 * without the NUL (call with buf NULL, cap 0 to size a buffer).
 * MGEMM_ERR_INVALID_ARG if len is NULL or the text does not fit.
 */
mgemm_status_t mgemm_table_export(mgemm_handle_t h, char* buf, size_t cap, size_t* len);

/*
 * mgemm_table_import -- add the entries of text in mgemm_table_export's
 * format (replacing entries with the same key).  All-or-nothing:
 * MGEMM_ERR_INVALID_ARG for a malformed line or an unknown kernel name, and
 * then the table is unchanged.
 */
mgemm_status_t mgemm_table_import(mgemm_handle_t h, const char* text);

/* mgemm_table_clear -- remove every entry (the model alone decides again). */
mgemm_status_t mgemm_table_clear(mgemm_handle_t h);

/*
 * mgemm_weighted_choice -- index of the variant with the smallest
 * sum over shapes of calls[s] * times[s * n_variants + v] (Example 5-9 of
 * section 5.4.5); a variant with a non-finite or negative time for any shape
 * with calls > 0 is out.  Ties go to the lower index.  calls NULL counts one
 * call per shape.  Returns -1 if no variant qualifies or an argument is
 * invalid.  Host-only; needs no device.
 */
int32_t mgemm_weighted_choice(int32_t n_shapes, int32_t n_variants, const double* times,
                              const double* calls);

/*
 * FP8 E4M3 with per-row scales ("Chapter 5: Operators and Runtime"
 * (ai-infra-book): section 5.4.3, Example 5-7, the E4M3FN format and a scale
 * taken from the largest magnitude of the whole row before quantising;
 * section 5.4.4, Example 5-8, FP8 activations with per-row scales times FP8
 * weights).  E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits, largest
 * finite 448, no infinity, codes 0x7F and 0xFF are NaN.
 *
 * mgemm_quantize_fp8 -- per-row quantisation of X (M x K, row-major, element
 * type xtype = F32, F16 or BF16, leading dimension ldx >= max(1, K)) into
 * codes Q (M x K bytes, row stride ldq >= max(1, K)) and FP32 dequantisation
 * scales (M floats): for each row, amax = largest |x| (NaN if the row holds
 * a NaN), scales[row] = amax / 448 (FP32, one rounding), the row factor
 * r = 448 / amax rounded once to FP32, and
 *     Q[row][k] = E4M3( x * r )
 * with the product x * r rounded to FP32 (round to nearest even), then to the
 * nearest E4M3 value with ties to the even mantissa; magnitudes of 448 and
 * above give 448, NaN gives 0x7F, the sign of zero is kept.  (Two roundings,
 * of r and of x * r, so a code can differ by one step from E4M3(x*448/amax)
 * evaluated exactly.)  A row of zeros gets scale 0 and keeps its signed
 * zeros.  So X ~ decode(Q) * scales.
 * Device pointers; asynchronous on `stream`.
 * Errors: MGEMM_ERR_INVALID_ARG for negative sizes, a leading dimension or
 * row stride below K, an unknown xtype or a NULL pointer with M, K > 0.
 */
mgemm_status_t mgemm_quantize_fp8(mgemm_handle_t h, int64_t M, int64_t K, const void* X,
                                  int64_t ldx, mgemm_dtype_t xtype, void* Q, int64_t ldq,
                                  float* scales, hipStream_t stream);

/*
 * mgemm_run_fp8 -- C = alpha * (diag(sa) A) (diag(sb) B)^T + beta * C on FP8
 * codes, i.e. per output
 *     C[m][n] = round(alpha * sa[m] * sb[n] * sum_k A[m][k] * B[n][k] + beta * C[m][n])
 *   A  : M x K codes, row-major (row stride lda >= max(1, K)), sa: M scales;
 *   B  : N x K codes, one row per output column (the weight matrix as
 *        out_features x in_features; row stride ldb >= max(1, K)), sb: N scales;
 *   C  : M x N, row-major, ldc >= max(1, N), element type ctype (F32, F16,
 *        BF16); beta == 0 never reads C.
 *   kernel : MGEMM_KERNEL_AUTO, MGEMM_KERNEL_F8_MFMA, MGEMM_KERNEL_F8_MFMA_192
 *        or MGEMM_KERNEL_F8_MFMA_128 (K >= 64, lda and ldb multiples of 16,
 *        16-byte aligned A and B; a K that is not a multiple of 64 ends with
 *        a partial slice) or MGEMM_KERNEL_F8_GENERAL (anything).
 *        AUTO takes the MFMA tile (256x256, 256x192 or 128x192) and split
 *        of K with the smallest predicted time.
 *   ksplit : 0 = the library's choice, 1 = no split, 2 .. MGEMM_MAX_KSPLIT =
 *        at most that many K ranges of whole 64-element slices (MFMA kernels
 *        only), summed in range order by a second launch as mgemm_run_variant
 *        describes; a forced split with MGEMM_KERNEL_AUTO is invalid.
 * Products of codes are exact; the K sum accumulates in FP32 and the scales
 * are applied to it once: v = alpha * ((acc * sa[m]) * sb[n]).
 * M == 0 or N == 0 does nothing; K == 0 or alpha == 0 gives C = beta * C.
 * Asynchronous on `stream`.
 * Errors: MGEMM_ERR_INVALID_ARG (sizes, strides, NULL pointers, ctype,
 * kernel not an FP8 kernel, ksplit out of range); MGEMM_ERR_UNSUPPORTED when
 * a forced kernel or split cannot run the problem (partials larger than the
 * workspace); MGEMM_ERR_HIP for a failed launch.
 */
mgemm_status_t mgemm_run_fp8(mgemm_handle_t h, mgemm_kernel_t kernel, int32_t ksplit, int64_t M,
                             int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                             const float* sa, const void* B, int64_t ldb, const float* sb,
                             float beta, void* C, int64_t ldc, mgemm_dtype_t ctype,
                             hipStream_t stream);

/*
 * mgemm_run_noalloc -- mgemm_run_variant without a handle and without any
 * device allocation, for callers that cannot allocate: code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, validation, results and errors are those of mgemm_run_variant
 * on the CURRENT HIP device (no dispatch table: the built-in model chooses
 * when v is NULL or AUTO).  The split-K and stream-K forms take their FP32
 * partial results and arrival counters from a static device array inside the
 * library (MGEMM_NOALLOC_SCRATCH_BYTES of partials plus
 * MGEMM_NOALLOC_COUNTERS counters, held on every GPU the library runs on
 * until the process ends) instead of a handle's workspace; the first call on
 * a device looks the array up and enqueues a small kernel on `stream` that
 * zeroes the counters (every later call leaves them at zero).  With AUTO the
 * model only picks forms that fit the array; a forced variant whose partials
 * do not fit returns MGEMM_ERR_SCRATCH and enqueues nothing.
 * Calls that overlap in time on one GPU (different streams, or different
 * host threads) share the array and race: order them on one stream.
 * Errors: as mgemm_run_variant; MGEMM_ERR_UNSUPPORTED also when the current
 * device is not gfx950; MGEMM_ERR_HIP when the device cannot be queried or
 * the array cannot be looked up.
 */
#define MGEMM_NOALLOC_SCRATCH_BYTES (32u << 20)
#define MGEMM_NOALLOC_COUNTERS 16384u
mgemm_status_t mgemm_run_noalloc(const mgemm_variant_t* v, mgemm_layout_t layoutA,
                                 mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K,
                                 float alpha, const void* A, int64_t lda, const void* B,
                                 int64_t ldb, float beta, void* C, int64_t ldc,
                                 mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                                 hipStream_t stream);

/* Static strings; never NULL (unknown values give "unknown"). */
const char* mgemm_status_string(mgemm_status_t s);
const char* mgemm_kernel_name(mgemm_kernel_t k);

/* Number of compute units of the handle's device (0 if h is NULL). */
int mgemm_num_cu(mgemm_handle_t h);

/*
 * mgemm_set_clock_stamps -- measurement hook: the shader clock a kernel
 * actually ran at.  The MI355X lowers its clock within microseconds under
 * heavy matrix-core load, so the clock that sets a kernel's peak can only be
 * read inside the kernel (the SGEMM report, "how the cuBLAS denominator was
 * fixed": the peak is re-derived at the clock measured while running).
 * With buf non-NULL, every later launch through this handle of the
 * direct-to-LDS FP16/BF16 kernels (MGEMM_KERNEL_H_DMA_256/_192/_128/_64 and the
 * gated pair; for a split of K, its first launch), of MGEMM_KERNEL_SKINNY_SK
 * and of the FP8 MFMA kernels (mgemm_run_fp8) has each
 * workgroup b < nblocks store, from its first wave,
 *     buf[4b]   shader-clock cycles at its start, buf[4b+1] at its end,
 *     buf[4b+2] 100 MHz real-time ticks at its start, buf[4b+3] at its end,
 * so its clock is 100 MHz * (buf[4b+1] - buf[4b]) / (buf[4b+3] - buf[4b+2]).
 * Other kernels leave buf alone.  buf NULL (nblocks 0) turns the hook off.
 *   buf : device buffer of 4 * nblocks uint64 values, owned by the caller,
 *         alive while launches that use it are pending.
 * The setting is read when a call is enqueued, so changing it between calls
 * (for a buffer per call) is fine.  Costs two scalar reads at the start and
 * one store at the end of each workgroup.
 * Errors: MGEMM_ERR_INVALID_ARG for a NULL handle, nblocks < 0, or buf
 * non-NULL with nblocks 0.
 */
mgemm_status_t mgemm_set_clock_stamps(mgemm_handle_t h, uint64_t* buf, int64_t nblocks);

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_H_ */
