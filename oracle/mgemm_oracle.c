/*
 * mgemm_oracle.c -- plain, slow, obviously-correct CPU oracle for dense GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (the definition, written out):
 *
 *     C_out[i,j] = round_out( alpha * sum_{k<K} a(i,k) * b(k,j)  +  beta * c(i,j) )
 *
 *   - the product-sum over k with alpha and beta is the GEMM of the SGEMM
 *     report "SGEMM measurements and three ledgers" (daleiyang, section on the
 *     naive kernel K1, whose store is alpha*acc + beta*C) and the signature of
 *     the zwxr.cn SGEMM post (section 3.3, gemm(A,B,C,M,N,K,alpha,beta));
 *   - the triple loop itself, FP32-or-wider accumulation and the single final
 *     rounding to the output format (round_to_bf16(acc)) follow "Chapter 5:
 *     Operators and Runtime" (ai-infra-book), sections 5.2.1 and 5.4.2;
 *   - row-major versus column-major storage is the transpose identity of the
 *     SGEMM report (section "how the cuBLAS denominator was fixed"): the same
 *     bytes read in the other order are the transpose.
 *
 * Numerics.  Every input element (FP32, FP16 or BF16) is first decoded
 * exactly into an IEEE double.  The products a*b are then exact in double
 * (at most 24+24 significant bits), the sum over k runs in ascending k in
 * double, alpha and beta are applied in double, and only then is the value
 * rounded once, round-to-nearest-even, into the output format.  The double
 * sum's own error (about K * 2^-53 * sum|a*b|) is far below every tolerance
 * the GPU path is held to.  The loop is i, then k, then j (one double
 * accumulator per output of the row, section 5.2.1 of Chapter 5 notes the
 * i-k-j order performs the same work), so each output still sums over k in
 * ascending order exactly as the textbook i-j-k loop would.
 *
 * Conventions where the pages are silent (each listed in the design notes):
 *   - C is stored in the same order as A (one "order" for the call);
 *   - beta == 0 means C is never read (it may hold NaN);
 *   - K == 0 gives C = round(beta * c);  M == 0 or N == 0 does nothing;
 *   - rounding is IEEE round-to-nearest-even, overflow goes to +-inf and FP16
 *     and BF16 subnormal outputs are kept (no flush to zero).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_ROW = 0, ORC_COL = 1 };
enum { ORC_OK = 0, ORC_BAD_ARG = 1, ORC_NO_MEM = 2 };

/* ---------------------------------------------------------------------------
 * Element decoding: storage bits -> exact double (IEEE 754 binary32, binary16,
 * and bfloat16 = the top half of a binary32).
 * ------------------------------------------------------------------------- */

static double decode_f16_bits(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static double decode_f32_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;                              /* exact widening */
}

static double decode_bf16_bits(uint16_t b) {
    return decode_f32_bits((uint32_t)b << 16);
}

double orc_decode(int dtype, const void* p, int64_t idx) {
    switch (dtype) {
    case ORC_F32: return decode_f32_bits(((const uint32_t*)p)[idx]);
    case ORC_F16: return decode_f16_bits(((const uint16_t*)p)[idx]);
    case ORC_BF16: return decode_bf16_bits(((const uint16_t*)p)[idx]);
    }
    return NAN;
}

/* ---------------------------------------------------------------------------
 * Rounding: double -> nearest value of a binary format with `p` significant
 * bits, smallest normal exponent `emin` (values 2^emin .. ) and subnormals
 * down to 2^(emin-p+1), ties to even.  Returns the rounded value as a double
 * (exactly representable in the target), or +-inf past the overflow
 * threshold.  `maxfin` is the largest finite value of the format.
 * ------------------------------------------------------------------------- */
static double round_to_format(double x, int p, int emin, double maxfin) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);                      /* ax = f * 2^e, 0.5 <= f < 1, so ulp = 2^(e-p) */
    int qexp = e - p;
    if (qexp < emin - p + 1) qexp = emin - p + 1;   /* subnormal spacing */
    double n = ldexp(ax, -qexp);        /* exact: a power-of-two rescale */
    double r = rint(n);                 /* default mode: nearest, ties to even */
    double y = ldexp(r, qexp);
    /* Overflow: anything that rounds past maxfin (i.e. at or beyond the
     * midpoint between maxfin and the next power of two, with the tie going to
     * the even neighbour, which is the power of two) becomes infinity. */
    if (y > maxfin) y = INFINITY;
    return x < 0 ? -y : y;
}

static uint16_t encode_f16(double x) {
    double y = round_to_format(x, 11, -14, 65504.0);
    uint16_t sign = (signbit(y) ? 0x8000u : 0u);
    double ay = fabs(y);
    if (isnan(y)) return (uint16_t)(sign | 0x7e00u);
    if (isinf(y)) return (uint16_t)(sign | 0x7c00u);
    if (ay == 0.0) return sign;
    if (ay < ldexp(1.0, -14)) {                      /* subnormal: ay = m * 2^-24 */
        return (uint16_t)(sign | (uint16_t)ldexp(ay, 24));
    }
    int e;
    double f = frexp(ay, &e);                        /* ay = f*2^e, f in [0.5,1) */
    uint16_t biased = (uint16_t)(e - 1 + 15);
    uint16_t mant = (uint16_t)ldexp(f * 2.0 - 1.0, 10);
    return (uint16_t)(sign | (biased << 10) | mant);
}

static uint16_t encode_bf16(double x) {
    /* bfloat16: 8 significant bits, same exponent range as binary32
     * (smallest normal 2^-126), largest finite (2 - 2^-7) * 2^127. */
    double maxfin = ldexp(2.0 - ldexp(1.0, -7), 127);
    double y = round_to_format(x, 8, -126, maxfin);
    if (isnan(y)) return (uint16_t)((signbit(y) ? 0x8000u : 0u) | 0x7fc0u);
    float f = (float)y;                              /* exact: y is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static uint32_t encode_f32(double x) {
    double maxfin = ldexp(2.0 - ldexp(1.0, -23), 127);
    double y = round_to_format(x, 24, -126, maxfin);
    float f = (float)y;                              /* exact: y is a binary32 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(y)) u = (signbit(y) ? 0xffc00000u : 0x7fc00000u);
    return u;
}

void orc_encode(int dtype, double x, void* p, int64_t idx) {
    switch (dtype) {
    case ORC_F32: ((uint32_t*)p)[idx] = encode_f32(x); break;
    case ORC_F16: ((uint16_t*)p)[idx] = encode_f16(x); break;
    case ORC_BF16: ((uint16_t*)p)[idx] = encode_bf16(x); break;
    }
}

/* Round a double to the format and return the rounded value as a double. */
double orc_round(int dtype, double x) {
    switch (dtype) {
    case ORC_F32: return decode_f32_bits(encode_f32(x));
    case ORC_F16: return decode_f16_bits(encode_f16(x));
    case ORC_BF16: return decode_bf16_bits(encode_bf16(x));
    }
    return NAN;
}

/* ---------------------------------------------------------------------------
 * Operand access in logical coordinates.
 *   A is M x K:  row-major a(i,k) = A[i*lda + k];  column-major A[k*lda + i]
 *   B is K x N:  row-major b(k,j) = B[k*ldb + j];  column-major B[j*ldb + k]
 *   C is M x N and stored in A's order.
 * ------------------------------------------------------------------------- */
static int64_t a_index(int layout, int64_t i, int64_t k, int64_t lda) {
    return layout == ORC_ROW ? i * lda + k : k * lda + i;
}
static int64_t b_index(int layout, int64_t k, int64_t j, int64_t ldb) {
    return layout == ORC_ROW ? k * ldb + j : j * ldb + k;
}
static int64_t c_index(int layout, int64_t i, int64_t j, int64_t ldc) {
    return layout == ORC_ROW ? i * ldc + j : j * ldc + i;
}

static int check_args(int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc, int dtype) {
    if (M < 0 || N < 0 || K < 0) return ORC_BAD_ARG;
    if ((layoutA != ORC_ROW && layoutA != ORC_COL) || (layoutB != ORC_ROW && layoutB != ORC_COL))
        return ORC_BAD_ARG;
    if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16) return ORC_BAD_ARG;
    int64_t one = 1;
    int64_t need_a = layoutA == ORC_ROW ? (K > one ? K : one) : (M > one ? M : one);
    int64_t need_b = layoutB == ORC_ROW ? (N > one ? N : one) : (K > one ? K : one);
    int64_t need_c = layoutA == ORC_ROW ? (N > one ? N : one) : (M > one ? M : one);
    if (lda < need_a || ldb < need_b || ldc < need_c) return ORC_BAD_ARG;
    return ORC_OK;
}

/*
 * Full product for the listed rows of C (all rows when rows == NULL).
 *   exact   (optional) receives the unrounded double value of row r, column j
 *           at exact[r*N + j], r indexing the rows list;
 *   C_out   (optional) receives round_out(value) at its storage position;
 *   C_in    is read only when beta != 0.
 * One double accumulator per output; rows are independent, so the OpenMP
 * split over rows does not change any result.
 */
int orc_gemm_rows(int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                  double alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                  double beta, const void* C_in, void* C_out, int64_t ldc, int dtype,
                  int64_t nrows, const int64_t* rows, double* exact, int nthreads) {
    int rc = check_args(layoutA, layoutB, M, N, K, lda, ldb, ldc, dtype);
    if (rc != ORC_OK) return rc;
    if (rows == NULL) nrows = M;
    for (int64_t r = 0; r < nrows && rows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return ORC_BAD_ARG;
    if (nrows == 0 || N == 0) return ORC_OK;
    if (beta != 0.0 && C_in == NULL) return ORC_BAD_ARG;

    /* Decode B once into a dense K x N double array (exact conversion). */
    double* Bd = NULL;
    if (K > 0) {
        Bd = (double*)malloc((size_t)K * (size_t)N * sizeof(double));
        if (!Bd) return ORC_NO_MEM;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            Bd[k * N + j] = orc_decode(dtype, B, b_index(layoutB, k, j, ldb));

    int failed = 0;
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)N * sizeof(double));
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!acc) continue;
            int64_t i = rows ? rows[r] : r;
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = orc_decode(dtype, A, a_index(layoutA, i, k, lda));
                const double* brow = Bd + k * N;
                for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
            }
            for (int64_t j = 0; j < N; ++j) {
                double v = alpha * acc[j];
                if (beta != 0.0) v += beta * orc_decode(dtype, C_in, c_index(layoutA, i, j, ldc));
                if (exact) exact[r * N + j] = v;
                if (C_out) orc_encode(dtype, v, C_out, c_index(layoutA, i, j, ldc));
            }
        }
        free(acc);
    }
    free(Bd);
    return failed ? ORC_NO_MEM : ORC_OK;
}

/* Whole product: every row of C. */
int orc_gemm(int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
             double alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
             double beta, const void* C_in, void* C_out, int64_t ldc, int dtype,
             double* exact, int nthreads) {
    return orc_gemm_rows(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C_in,
                         C_out, ldc, dtype, 0, NULL, exact, nthreads);
}

/*
 * Single outputs, one at a time: value[p] = alpha * sum_k a(i_p,k) b(k,j_p)
 * + beta * c(i_p,j_p), unrounded.  Used to sample very large products.
 */
int orc_gemm_points(int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                    double alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
                    double beta, const void* C_in, int64_t ldc, int dtype,
                    int64_t npts, const int64_t* pi, const int64_t* pj, double* value,
                    int nthreads) {
    int rc = check_args(layoutA, layoutB, M, N, K, lda, ldb, ldc, dtype);
    if (rc != ORC_OK) return rc;
    if (beta != 0.0 && C_in == NULL) return ORC_BAD_ARG;
    for (int64_t p = 0; p < npts; ++p)
        if (pi[p] < 0 || pi[p] >= M || pj[p] < 0 || pj[p] >= N) return ORC_BAD_ARG;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p) {
        int64_t i = pi[p], j = pj[p];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += orc_decode(dtype, A, a_index(layoutA, i, k, lda)) *
                 orc_decode(dtype, B, b_index(layoutB, k, j, ldb));
        double v = alpha * s;
        if (beta != 0.0) v += beta * orc_decode(dtype, C_in, c_index(layoutA, i, j, ldc));
        value[p] = v;
    }
    return ORC_OK;
}

/* Array helpers so tests can round/decode whole buffers without Python loops. */
void orc_decode_array(int dtype, const void* p, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_decode(dtype, p, i);
}
void orc_encode_array(int dtype, const double* x, int64_t n, void* p) {
    for (int64_t i = 0; i < n; ++i) orc_encode(dtype, x[i], p, i);
}
void orc_round_array(int dtype, const double* x, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_round(dtype, x[i]);
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
