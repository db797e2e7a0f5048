"""Pins for the CPU oracle: checks against facts other than the oracle itself.

Each check ties the oracle to something independent of its own code:
  * IEEE 754 closed forms and library conversions (numpy float16/float32 casts,
    torch's float32 -> bfloat16 cast) for the output rounding;
  * matrices whose product has a closed form (identity, permutation, all-ones,
    rank one, alpha = 0, K = 0);
  * the transpose identity of the SGEMM report (row-major C = A B is the same
    bytes as column-major C^T = B^T A^T with the pointers swapped);
  * exact integer arithmetic (numpy int64 matmul, Python fractions) and
    numpy's float64 matmul within the float64 error bound.
The battery ``PIN_CHECKS`` is reused by test_oracle_mutations.py, which plants
mistakes in copies of the oracle and requires every one of them to be caught.
"""
from fractions import Fraction
import itertools

import numpy as np
import pytest
import torch

import oracle
from workloads import cast, storage_view, operand

RNG = np.random.default_rng(12345)


def _bits(t):
    return storage_view(t)


def _dense(dtype, x64):
    """float64 matrix -> flat storage bits (row-major, contiguous)."""
    return _bits(cast(np.ascontiguousarray(x64).reshape(-1), dtype))


def _run(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, dtype, c_size):
    store = np.uint32 if dtype == "f32" else np.uint16
    out = np.zeros(c_size, store)
    exact = oracle.gemm(layoutA, layoutB, M, N, K, alpha, A, lda, B, ldb, beta, C0, out, ldc,
                        dtype)
    return out, exact


def _store(layout, mat, ld, dtype):
    """Lay out a float64 matrix with leading dimension ld (NaN padding) as bits."""
    r, c = mat.shape
    outer, inner = (r, c) if layout == "row" else (c, r)
    buf = np.full((outer, ld), np.nan)
    buf[:, :inner] = mat if layout == "row" else mat.T
    return _dense(dtype, buf)


def _read(layout, bits, M, N, ld, dtype):
    vals = oracle.decode(dtype, bits)
    if layout == "row":
        return vals.reshape(-1, ld)[:M, :N]
    return vals.reshape(-1, ld)[:N, :M].T


# --------------------------------------------------------------------------
# Output rounding
# --------------------------------------------------------------------------

def check_f16_against_numpy():
    # Values across the whole binary16 range: subnormals, normals, near overflow.
    mags = np.concatenate([
        np.ldexp(RNG.uniform(0.5, 1.0, 4000), RNG.integers(-26, 17, 4000)),
        RNG.uniform(0, 70000, 2000),
        np.ldexp(np.arange(0, 2048) + 0.5, -24),          # subnormal ties
        np.arange(2040, 2060) + 0.0, np.arange(2040, 2060) + 0.5,
    ])
    x = np.concatenate([mags, -mags])
    got = oracle.encode("f16", x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def check_f16_closed_forms():
    for e in range(-14, 16):                   # normal powers of two: mantissa 0
        assert int(oracle.encode("f16", [2.0 ** e])[0]) == (e + 15) << 10
    for e in range(-24, -14):                  # subnormal powers of two: m * 2^-24
        assert int(oracle.encode("f16", [2.0 ** e])[0]) == 1 << (e + 24)
    enc = lambda v: int(oracle.encode("f16", [v])[0])
    assert enc(65504.0) == 0x7BFF and enc(65519.0) == 0x7BFF
    assert enc(65520.0) == 0x7C00 and enc(-65520.0) == 0xFC00  # tie goes to even = inf
    assert enc(2049.0) == enc(2048.0)          # tie -> even mantissa
    assert enc(2051.0) == enc(2052.0)
    assert enc(1.0 + 2.0 ** -11) == 0x3C00     # tie between 1 and 1+2^-10 -> 1
    assert enc(2.0 ** -25) == 0                # half of the smallest subnormal -> 0 (even)
    assert enc(3 * 2.0 ** -25) == 2            # 1.5 * 2^-24 -> 2 * 2^-24 (even)
    assert enc(float("inf")) == 0x7C00 and enc(-0.0) == 0x8000


def check_bf16_against_torch():
    x32 = np.concatenate([
        np.ldexp(RNG.uniform(0.5, 1.0, 4000), RNG.integers(-135, 128, 4000)),
        RNG.normal(0, 1, 2000),
    ]).astype(np.float32)
    x32 = np.concatenate([x32, -x32])
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode("bf16", x32.astype(np.float64))
    assert np.array_equal(got, want)
    enc = lambda v: int(oracle.encode("bf16", [v])[0])
    assert enc(1.0 + 2.0 ** -8) == 0x3F80      # tie -> even (1.0)
    assert enc(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie -> even (1 + 2^-6)
    assert enc(2.0 ** -133) == 0x0001          # smallest subnormal


def check_f32_against_numpy():
    x = np.concatenate([RNG.normal(0, 1, 3000) * np.ldexp(1.0, RNG.integers(-140, 120, 3000)),
                        np.array([3.4028235677973366e38, 3.4028235677973366e38 * (1 + 2 ** -25),
                                  1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24])])
    got = oracle.encode("f32", x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


def check_decode_all_patterns():
    allbits = np.arange(65536, dtype=np.uint16)
    d16 = oracle.decode("f16", allbits)
    ref16 = allbits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(d16), np.isnan(ref16))
    m = ~np.isnan(ref16)
    assert np.array_equal(d16[m], ref16[m])
    dbf = oracle.decode("bf16", allbits)
    refbf = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    m = ~np.isnan(refbf)
    assert np.array_equal(np.isnan(dbf), np.isnan(refbf)) and np.array_equal(dbf[m], refbf[m])


# --------------------------------------------------------------------------
# Closed-form products
# --------------------------------------------------------------------------

LAYOUTS = list(itertools.product(["row", "col"], ["row", "col"]))


def check_identity():
    M, K = 13, 9
    for dtype in ("f32", "f16", "bf16"):
        for la, lb in LAYOUTS:
            A = RNG.uniform(-1, 1, (M, K))
            A = oracle.round_to(dtype, A)
            I = np.eye(K)
            lda = (K if la == "row" else M) + 3
            ldb = (K if lb == "row" else K) + 2
            ldc = (K if la == "row" else M) + 1
            csz = (M if la == "row" else K) * ldc
            out, _ = _run(la, lb, M, K, K, 1.0, _store(la, A, lda, dtype), lda,
                          _store(lb, I, ldb, dtype), ldb, 0.0, None, ldc, dtype, csz)
            assert np.array_equal(_read(la, out, M, K, ldc, dtype), A), (dtype, la, lb)


def check_permutation():
    # P @ B permutes the rows of B; B @ P would permute columns instead, so a
    # transposed operand or swapped index fails here.
    M, N = 11, 7
    perm = RNG.permutation(M)
    P = np.zeros((M, M))
    P[np.arange(M), perm] = 1.0
    for dtype in ("f32", "f16", "bf16"):
        for la, lb in LAYOUTS:
            B = oracle.round_to(dtype, RNG.uniform(-4, 4, (M, N)))
            lda = M + 1
            ldb = (N if lb == "row" else M) + 2
            ldc = (N if la == "row" else M) + 3
            csz = (M if la == "row" else N) * ldc
            out, _ = _run(la, lb, M, N, M, 1.0, _store(la, P, lda, dtype), lda,
                          _store(lb, B, ldb, dtype), ldb, 0.0, None, ldc, dtype, csz)
            assert np.array_equal(_read(la, out, M, N, ldc, dtype), B[perm]), (dtype, la, lb)


def check_all_ones_alpha_beta():
    M, N, K = 6, 5, 37
    for dtype in ("f32", "f16", "bf16"):
        for la, lb in LAYOUTS:
            C0 = oracle.round_to(dtype, RNG.uniform(-8, 8, (M, N)))
            alpha, beta = 0.5, -0.75
            ldc = N if la == "row" else M
            csz = (M if la == "row" else N) * ldc
            out, exact = _run(la, lb, M, N, K, alpha,
                              _store(la, np.ones((M, K)), K if la == "row" else M, dtype),
                              K if la == "row" else M,
                              _store(lb, np.ones((K, N)), N if lb == "row" else K, dtype),
                              N if lb == "row" else K, beta, _store(la, C0, ldc, dtype), ldc,
                              dtype, csz)
            want = alpha * K + beta * C0
            assert np.array_equal(exact, want)
            assert np.array_equal(_read(la, out, M, N, ldc, dtype), oracle.round_to(dtype, want))


def check_rank_one():
    # a(i,k) = u_i v_k, b(k,j) = w_k z_j  =>  c(i,j) = u_i z_j (v . w), exact for small ints.
    M, N, K = 9, 10, 23
    u, z = RNG.integers(-3, 4, M), RNG.integers(-3, 4, N)
    v, w = RNG.integers(-2, 3, K), RNG.integers(-2, 3, K)
    A = np.outer(u, v).astype(np.float64)
    B = np.outer(w, z).astype(np.float64)
    dot = float(np.dot(v, w))
    for dtype in ("f32", "f16", "bf16"):
        for la, lb in LAYOUTS:
            lda = K if la == "row" else M
            ldb = N if lb == "row" else K
            ldc = N if la == "row" else M
            csz = (M if la == "row" else N) * ldc
            out, exact = _run(la, lb, M, N, K, 1.0, _store(la, A, lda, dtype), lda,
                              _store(lb, B, ldb, dtype), ldb, 0.0, None, ldc, dtype, csz)
            assert np.array_equal(exact, np.outer(u, z) * dot), (dtype, la, lb)


def check_alpha_zero_and_k_zero():
    M, N, K = 4, 6, 5
    for dtype in ("f32", "f16", "bf16"):
        C0 = oracle.round_to(dtype, RNG.uniform(-3, 3, (M, N)))
        A = _store("row", RNG.uniform(-1, 1, (M, K)), K, dtype)
        B = _store("row", RNG.uniform(-1, 1, (K, N)), N, dtype)
        out, exact = _run("row", "row", M, N, K, 0.0, A, K, B, N, 0.5, _store("row", C0, N, dtype),
                          N, dtype, M * N)
        assert np.array_equal(exact, 0.5 * C0)
        out, exact = _run("row", "row", M, N, 0, 2.0, A, 1, B, N, -1.0,
                          _store("row", C0, N, dtype), N, dtype, M * N)
        assert np.array_equal(exact, -C0)
        assert np.array_equal(_read("row", out, M, N, N, dtype), -C0)


def check_beta_zero_never_reads_c():
    M, N, K = 5, 4, 3
    A = _store("row", RNG.uniform(-1, 1, (M, K)), K, "f32")
    B = _store("row", RNG.uniform(-1, 1, (K, N)), N, "f32")
    nan_c = _store("row", np.full((M, N), np.nan), N, "f32")
    out, exact = _run("row", "row", M, N, K, 1.0, A, K, B, N, 0.0, nan_c, N, "f32", M * N)
    assert np.isfinite(exact).all()


def check_transpose_identity():
    # Row-major C = A B  <=>  column-major C^T = B^T A^T with the pointers
    # swapped and M, N swapped: the same bytes must come out.
    M, N, K = 14, 9, 17
    for dtype in ("f32", "f16", "bf16"):
        A = _store("row", RNG.uniform(-1, 1, (M, K)), K + 2, dtype)
        B = _store("row", RNG.uniform(-1, 1, (K, N)), N + 1, dtype)
        C0 = _store("row", RNG.uniform(-1, 1, (M, N)), N + 3, dtype)
        out_r, _ = _run("row", "row", M, N, K, 0.5, A, K + 2, B, N + 1, 2.0, C0, N + 3, dtype,
                        M * (N + 3))
        out_c, _ = _run("col", "col", N, M, K, 0.5, B, N + 1, A, K + 2, 2.0, C0, N + 3, dtype,
                        M * (N + 3))
        assert np.array_equal(out_r, out_c)


def check_integer_exact():
    # Small integers: every partial sum is an exactly representable integer, so
    # the exact product (numpy int64 matmul) rounded once is the only answer.
    M, N, K = 33, 29, 130
    Ai = RNG.integers(-4, 5, (M, K))
    Bi = RNG.integers(-4, 5, (K, N))
    Ci = RNG.integers(-4, 5, (M, N))
    exact_int = Ai @ Bi + 2 * Ci
    for dtype in ("f32", "f16", "bf16"):
        for la, lb in LAYOUTS:
            lda = (K if la == "row" else M) + 1
            ldb = (N if lb == "row" else K) + 2
            ldc = (N if la == "row" else M) + 1
            csz = (M if la == "row" else N) * ldc
            out, exact = _run(la, lb, M, N, K, 1.0, _store(la, Ai.astype(float), lda, dtype), lda,
                              _store(lb, Bi.astype(float), ldb, dtype), ldb, 2.0,
                              _store(la, Ci.astype(float), ldc, dtype), ldc, dtype, csz)
            assert np.array_equal(exact, exact_int.astype(np.float64))
            got = _read(la, out, M, N, ldc, dtype)
            if dtype == "f32":
                ref = exact_int.astype(np.float32).astype(np.float64)
            elif dtype == "f16":
                ref = exact_int.astype(np.float16).astype(np.float64)
            else:
                ref = torch.from_numpy(exact_int.astype(np.float32)).to(torch.bfloat16).double().numpy()
            assert np.array_equal(got, ref), (dtype, la, lb)


def check_against_numpy_float64():
    M, N, K = 37, 41, 300
    for dtype in ("f32", "f16", "bf16"):
        A = oracle.round_to(dtype, RNG.uniform(-1, 1, (M, K)))
        B = oracle.round_to(dtype, RNG.uniform(-1, 1, (K, N)))
        C0 = oracle.round_to(dtype, RNG.uniform(-1, 1, (M, N)))
        for la, lb in LAYOUTS:
            lda = K if la == "row" else M
            ldb = N if lb == "row" else K
            ldc = N if la == "row" else M
            csz = (M if la == "row" else N) * ldc
            _, exact = _run(la, lb, M, N, K, 1.5, _store(la, A, lda, dtype), lda,
                            _store(lb, B, ldb, dtype), ldb, -0.25, _store(la, C0, ldc, dtype), ldc,
                            dtype, csz)
            ref = 1.5 * (A @ B) - 0.25 * C0
            bound = (K + 4) * 2.0 ** -52 * (1.5 * (np.abs(A) @ np.abs(B)) + 0.25 * np.abs(C0))
            assert (np.abs(exact - ref) <= bound).all(), (dtype, la, lb)


def check_brute_force_fractions():
    # Tiny shapes summed in exact rational arithmetic.
    for (M, N, K) in [(1, 1, 1), (2, 3, 4), (3, 1, 5), (4, 4, 7)]:
        A = oracle.round_to("f16", RNG.uniform(-1, 1, (M, K)))
        B = oracle.round_to("f16", RNG.uniform(-1, 1, (K, N)))
        _, exact = _run("row", "col", M, N, K, 1.0, _store("row", A, K, "f16"), K,
                        _store("col", B, K, "f16"), K, 0.0, None, N, "f16", M * N)
        for i in range(M):
            for j in range(N):
                s = sum(Fraction(A[i, k]) * Fraction(B[k, j]) for k in range(K))
                assert exact[i, j] == float(s)   # f16 products/sums this small are exact in f64


def check_points_closed_forms():
    # gemm_points sums each listed output on its own; it is pinned like the
    # row form, at beta != 0, in every layout pair, with padded leading
    # dimensions: all-ones (C = alpha*K + beta*C0), exact integers against
    # numpy int64 (C = A B + 2 C0), and one-hot A rows that pick single rows
    # of B (C = B[k(i), j] - C0, which also catches a transposed B).
    M, N, K = 13, 11, 29
    pi = np.array([0, 12, 5, 7, 0, 12, 3], np.int64)
    pj = np.array([0, 10, 4, 9, 10, 0, 7], np.int64)
    for dtype in ("f32", "f16", "bf16"):
        for la, lb in LAYOUTS:
            lda = (K if la == "row" else M) + 3
            ldb = (N if lb == "row" else K) + 2
            ldc = (N if la == "row" else M) + 1
            C0 = oracle.round_to(dtype, RNG.uniform(-8, 8, (M, N)))
            c0 = _store(la, C0, ldc, dtype)
            got = oracle.gemm_points(la, lb, M, N, K, 0.5, _store(la, np.ones((M, K)), lda, dtype),
                                     lda, _store(lb, np.ones((K, N)), ldb, dtype), ldb, -0.75, c0,
                                     ldc, dtype, pi, pj)
            assert np.array_equal(got, 0.5 * K - 0.75 * C0[pi, pj]), (dtype, la, lb)
            Ai = RNG.integers(-4, 5, (M, K))
            Bi = RNG.integers(-4, 5, (K, N))
            Ci = RNG.integers(-4, 5, (M, N))
            got = oracle.gemm_points(la, lb, M, N, K, 1.0, _store(la, Ai.astype(float), lda, dtype),
                                     lda, _store(lb, Bi.astype(float), ldb, dtype), ldb, 2.0,
                                     _store(la, Ci.astype(float), ldc, dtype), ldc, dtype, pi, pj)
            assert np.array_equal(got, (Ai @ Bi + 2 * Ci)[pi, pj].astype(np.float64)), (dtype, la, lb)
            pick = RNG.integers(0, K, M)
            H = np.zeros((M, K))
            H[np.arange(M), pick] = 1.0
            Bv = oracle.round_to(dtype, RNG.uniform(-4, 4, (K, N)))
            got = oracle.gemm_points(la, lb, M, N, K, 1.0, _store(la, H, lda, dtype), lda,
                                     _store(lb, Bv, ldb, dtype), ldb, -1.0, c0, ldc, dtype, pi, pj)
            assert np.array_equal(got, Bv[pick[pi], pj] - C0[pi, pj]), (dtype, la, lb)


def check_silu_epilogue():
    """SiLU epilogue: the pages' two-partial-sums example, a library sigmoid,
    rounding before the activation, and the limits."""
    import json, os
    from scipy.special import expit
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
    ex = g["silu_partial_sums"]
    # Section 5.4.3: partial sums 1 and -1; activation after the full sum gives
    # SiLU(0) = 0, activation on each partial sum gives about 0.4621.
    A = _dense("f32", np.array([[1.0, -1.0]]))
    B = _dense("f32", np.array([[1.0], [1.0]]))
    _, exact = _run("row", "row", 1, 1, 2, 1.0, A, 2, B, 1, 0.0, None, 1, "f32", 1)
    assert oracle.silu_epilogue("f32", exact)[0, 0] == 0.0
    parts = oracle.silu_epilogue("f32", np.array([1.0, -1.0]))
    assert abs(parts.sum() - ex["activation_before_sum"]) <= ex["abs_tol"]
    # A library sigmoid on values that every format holds exactly.
    for dt in ("f32", "f16", "bf16"):
        x = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -3.0, 8.0, -8.0, 0.125])
        y = oracle.silu_epilogue(dt, x)
        assert np.allclose(y, x * expit(x), rtol=1e-14, atol=0.0), dt
    # Rounding to the output format comes first: 1 + 2^-9 is 1 in BF16, not in FP32.
    c = np.array([1.0 + 2.0 ** -9])
    assert oracle.silu_epilogue("bf16", c)[0] == 1.0 * expit(1.0)
    assert oracle.silu_epilogue("f32", c)[0] == c[0] * expit(c[0])
    # Limits: SiLU(x) -> x for large x, -> -0 for very negative x (no NaN from e^-x overflow).
    big = oracle.silu_epilogue("f32", np.array([1000.0, -1000.0, 60.0]))
    assert big[0] == 1000.0 and big[1] == 0.0 and np.signbit(big[1]) and big[2] == 60.0


def check_swiglu():
    """Gated pair Z = SiLU(G) * U: closed forms and the rounding of the stored
    intermediates."""
    from scipy.special import expit
    g = np.array([0.0, 1.0, -1.0, 2.0, -4.0, 0.5, 3.0])
    u = np.array([5.0, 1.0, 2.0, -3.0, 1.0, 0.0, -0.25])
    for dt in ("f32", "bf16", "f16"):
        z = oracle.swiglu(dt, g, u)
        t = oracle.round_to(dt, g * expit(g))
        assert np.array_equal(z, t * u), dt          # g and u are exact in every format
    assert oracle.swiglu("bf16", np.array([0.0]), np.array([7.0]))[0] == 0.0
    # U = 1 reduces to the SiLU epilogue rounded once.
    x = np.array([0.3, -1.7, 2.2])
    assert np.array_equal(oracle.swiglu("f16", x, np.ones(3)),
                          oracle.round_to("f16", oracle.silu_epilogue("f16", x)))
    # The stored T is rounded before the product: with T = SiLU(1) in BF16 and
    # U = 3, the unrounded SiLU(1) * 3 differs from round(SiLU(1)) * 3.
    z = oracle.swiglu("bf16", np.array([1.0]), np.array([3.0]))[0]
    assert z == oracle.round_to("bf16", np.array([expit(1.0)]))[0] * 3.0
    assert z != expit(1.0) * 3.0
    # G and U are rounded as stored tensors before use.
    z = oracle.swiglu("bf16", np.array([1.0 + 2.0 ** -10]), np.array([1.0 + 2.0 ** -10]))[0]
    assert z == oracle.round_to("bf16", np.array([expit(1.0)]))[0] * 1.0


PIN_CHECKS = [check_silu_epilogue, check_swiglu, check_f16_against_numpy, check_f16_closed_forms, check_bf16_against_torch,
              check_f32_against_numpy, check_decode_all_patterns, check_identity,
              check_permutation, check_all_ones_alpha_beta, check_rank_one,
              check_alpha_zero_and_k_zero, check_beta_zero_never_reads_c,
              check_transpose_identity, check_integer_exact, check_against_numpy_float64,
              check_brute_force_fractions, check_points_closed_forms]


@pytest.mark.parametrize("check", PIN_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_points_and_row_subsets_agree_with_full_product():
    M, N, K = 20, 18, 50
    A = operand("uniform", 7, M, K, "col", M + 2, "bf16")
    B = operand("uniform", 8, K, N, "row", N + 1, "bf16")
    full = oracle.gemm("col", "row", M, N, K, 1.0, A, M + 2, B, N + 1, 0.0, None, None, M, "bf16")
    rows = [0, 7, 19]
    sub = oracle.gemm("col", "row", M, N, K, 1.0, A, M + 2, B, N + 1, 0.0, None, None, M, "bf16",
                      rows=rows)
    assert np.array_equal(sub, full[rows])
    pi, pj = np.array([0, 5, 19, 3]), np.array([0, 17, 2, 9])
    pts = oracle.gemm_points("col", "row", M, N, K, 1.0, A, M + 2, B, N + 1, 0.0, None, M, "bf16",
                             pi, pj)
    assert np.allclose(pts, full[pi, pj], rtol=0, atol=1e-12)


def test_rejects_bad_arguments():
    A = np.zeros(16, np.uint32)
    with pytest.raises(ValueError):
        oracle.gemm("row", "row", 4, 4, 4, 1.0, A, 3, A, 4, 0.0, None, None, 4, "f32")   # lda < K
    with pytest.raises(ValueError):
        oracle.gemm("col", "row", 4, 4, 4, 1.0, A, 4, A, 4, 0.0, None, None, 3, "f32")   # ldc < M
    with pytest.raises(ValueError):
        oracle.gemm("row", "row", 4, 4, 4, 1.0, A, 4, A, 4, 1.0, None, None, 4, "f32")   # beta, no C
