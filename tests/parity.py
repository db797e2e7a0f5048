"""Helpers for GPU parity tests: run a workload through libmgemm and compare it
with the CPU oracle on the same seeded inputs.

Bars (the tolerance rules come with the workloads):
  * integer-valued inputs: the whole C buffer, bit for bit, equals the
    oracle's (every partial sum is exact in FP32, so one rounding of the exact
    integer is the only answer);
  * FP32: max|C - C_exact| <= 1e-4 * sqrt(K/256) * max|C_exact|;
  * FP16/BF16: per element |C - C_exact| <= max(tol, ulp(C_exact)/2 + tol/8),
    tol = 0.01*sqrt(K/512): the stated absolute bound, relaxed only where the
    output format's own spacing makes it impossible to meet;
  * outside the logical M x N region (the ldc padding) C is never written.
"""
from __future__ import annotations

import numpy as np
import torch

import dense_gemm_mgemm_amd as mg
import oracle
from dense_gemm_mgemm_amd.costmodel import tol_f32_rel, tol_half
from workloads import CANARY, Case, c_initial, storage_view

KERNELS_F32 = ["general", "f32_mfma", "f32_fast", "f32_fast_128", "f32_fast_u", "f32_sk"]
KERNELS_16 = ["general", "h_mfma_256x256", "h_mfma_256x192", "h_mfma_128x128",
              "h_dma_256x256", "h_dma_256x192", "h_dma_128x192", "h_dma_64x192"]


def run_gpu(h, case: Case, kernel: str = "auto", inputs=None, stream=None, epilogue="none",
            ksplit=None):
    """Returns (A, B, C0, C_init, C_out) as CPU tensors.  With `ksplit` the call
    goes through mgemm_run_variant (kernel and split of K forced)."""
    A, B, C0 = inputs if inputs is not None else case.make()
    Cin = c_initial(case, C0)
    dA, dB, dC = A.cuda(), B.cuda(), Cin.cuda()
    args = (case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha, dA, case.lda, dB,
            case.ldb, case.beta, dC, case.ldc, case.dtype)
    if ksplit is not None:
        mg.mgemm_run_variant(h, kernel, ksplit, *args, epilogue=epilogue, stream=stream)
    elif epilogue != "none":
        mg.mgemm_run_ex(h, kernel, *args, epilogue=epilogue, stream=stream)
    elif kernel == "auto":
        mg.mgemm_run(h, *args, stream=stream)
    else:
        mg.mgemm_run_kernel(h, kernel, *args, stream=stream)
    torch.cuda.synchronize()
    return A, B, C0, Cin, dC.cpu()


def logical(case: Case, vals: np.ndarray) -> np.ndarray:
    """Flat C storage -> (M, N) logical view."""
    v = vals.reshape(-1, case.ldc)
    if case.layoutA == "row":
        return v[: case.M, : case.N]
    return v[: case.N, : case.M].T


def padding_mask(case: Case) -> np.ndarray:
    """True on C storage positions outside the logical matrix."""
    m = np.ones(case.c_numel(), bool)
    logical(case, m.reshape(-1))[...] = False      # view write-through
    return m


def check_bit_exact(case: Case, A, B, C0, Cin, Cout):
    """Whole-buffer bit equality with the oracle's output (integer data)."""
    ref = storage_view(Cin).copy()
    oracle.gemm(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha,
                storage_view(A), case.lda, storage_view(B), case.ldb, case.beta,
                None if C0 is None else storage_view(C0), ref, case.ldc, case.dtype,
                want_exact=False)
    got = storage_view(Cout)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "%s: %d elements differ, first at %d: got %#x want %#x" % (
        case.name, bad.size, bad[0], got[bad[0]], ref[bad[0]])


def compare(case: Case, got: np.ndarray, exact: np.ndarray) -> dict:
    """Tolerance check of decoded values against the oracle's unrounded values."""
    err = np.abs(got - exact)
    if case.dtype == "f32":
        scale = float(np.max(np.abs(exact))) if exact.size else 0.0
        tol = tol_f32_rel(case.K) * max(scale, 1e-30)
        ok = bool(np.all(err <= tol)) and not np.isnan(got).any()
        return {"ok": ok, "max_err": float(np.nanmax(err)) if err.size else 0.0, "tol": tol}
    tol = tol_half(case.K)
    bound = half_bound(case.dtype, case.K, exact)
    ok = bool(np.all(err <= bound)) and not np.isnan(got).any()
    return {"ok": ok, "max_err": float(np.nanmax(err)) if err.size else 0.0, "tol": tol,
            "over_bare_tol": int(np.sum(err > tol))}


def half_bound(dtype: str, K: int, exact: np.ndarray) -> np.ndarray:
    """Per-element FP16/BF16 bound: max(tol, ulp/2 + tol/8), tol = 0.01*sqrt(K/512).

    The stated absolute bound holds wherever the output format can meet it.
    Where half the output spacing at the exact value comes within tol/8 of
    tol or exceeds it (FP16 outputs of magnitude >= 64 at K = 2048, >= 128 at
    K = 16384), no rounding of the exact value could meet the bare bound, and
    the bound becomes that half spacing plus tol/8 for the FP32 accumulation
    error (which stays below 1e-3 on every workload here)."""
    tol = tol_half(K)
    ulp = _ulp(dtype, oracle.round_to(dtype, exact))
    return np.maximum(tol, 0.5 * ulp + tol / 8)


def _ulp(dtype: str, x: np.ndarray) -> np.ndarray:
    p, emin = (11, -14) if dtype == "f16" else (8, -126)
    ax = np.abs(x)
    e = np.frexp(np.where(ax > 0, ax, 1.0))[1]
    return np.ldexp(1.0, np.maximum(e - p, emin - p + 1))


def check_tolerance(case: Case, A, B, C0, Cin, Cout, rows=None, cols=None):
    """Compare full C (rows None) or the listed rows and columns with the oracle,
    and check the ldc padding is untouched."""
    got_all = oracle.decode(case.dtype, storage_view(Cout))
    got = logical(case, got_all)
    a, b = storage_view(A), storage_view(B)
    c0 = None if C0 is None else storage_view(C0)
    reports = []
    if rows is None and cols is None:
        exact = oracle.gemm(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha, a,
                            case.lda, b, case.ldb, case.beta, c0, None, case.ldc, case.dtype)
        reports.append(compare(case, got, exact))
    if rows is not None:
        rows = np.asarray(sorted(set(int(r) for r in rows if 0 <= r < case.M)), np.int64)
        exact = oracle.gemm(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha, a,
                            case.lda, b, case.ldb, case.beta, c0, None, case.ldc, case.dtype,
                            rows=rows)
        reports.append(compare(case, got[rows], exact))
    if cols is not None:
        cols = sorted(set(int(c) for c in cols if 0 <= c < case.N))
        pi = np.repeat(np.arange(case.M), len(cols))
        pj = np.tile(np.asarray(cols), case.M)
        exact = oracle.gemm_points(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha,
                                   a, case.lda, b, case.ldb, case.beta, c0, case.ldc, case.dtype,
                                   pi, pj)
        reports.append(compare(case, got[pi, pj], exact))
    pad = padding_mask(case)
    init = storage_view(Cin)
    assert np.array_equal(storage_view(Cout)[pad], init[pad]), "%s: wrote outside C" % case.name
    for r in reports:
        assert r["ok"], "%s: %s" % (case.name, r)
    return reports


def exact_cols(case: Case, A, B, C0, cols) -> np.ndarray:
    """Oracle values of whole logical columns of C, shape (M, len(cols)).

    With one layout for A and B this is the transpose identity the oracle is
    pinned to: the columns of C are the rows of C^T = B^T A^T, where B^T, A^T
    and C^T are the same bytes read in the other storage order.  With mixed
    layouts C^T would be stored in the wrong order, so the columns are summed
    point by point instead."""
    if case.layoutA != case.layoutB:
        pi = np.repeat(np.arange(case.M), len(cols))
        pj = np.tile(np.asarray(cols, np.int64), case.M)
        v = oracle.gemm_points(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha,
                               storage_view(A), case.lda, storage_view(B), case.ldb, case.beta,
                               None if C0 is None else storage_view(C0), case.ldc, case.dtype,
                               pi, pj)
        return v.reshape(case.M, len(cols))
    flip = {"row": "col", "col": "row"}
    t = oracle.gemm(flip[case.layoutB], flip[case.layoutA], case.N, case.M, case.K, case.alpha,
                    storage_view(B), case.ldb, storage_view(A), case.lda, case.beta,
                    None if C0 is None else storage_view(C0), None, case.ldc, case.dtype,
                    rows=np.asarray(cols, np.int64))
    return t.T


def boundary_lines(n: int, step: int = 64) -> list[int]:
    """First and last index of every aligned block of `step` (every tile
    boundary of every kernel here: all tile sizes are multiples of 64)."""
    out = set()
    for b in range(0, n, step):
        out.update({b, min(b + step, n) - 1})
    return sorted(out)


def block_points(M: int, N: int, block: int = 64, per_block: int = 4, seed: int = 0):
    """per_block random points inside every block x block block of an M x N
    matrix (fewer only where a ragged block has fewer elements)."""
    rng = np.random.default_rng(seed)
    pi, pj = [], []
    for b0 in range(0, M, block):
        h = min(block, M - b0)
        for c0 in range(0, N, block):
            w = min(block, N - c0)
            k = min(per_block, h * w)
            flat = rng.choice(h * w, size=k, replace=False)
            pi.append(b0 + flat // w)
            pj.append(c0 + flat % w)
    return np.concatenate(pi).astype(np.int64), np.concatenate(pj).astype(np.int64)


def check_stratified(case: Case, A, B, C0, Cin, Cout, block: int = 64, per_block: int = 4,
                     seed: int = 0) -> dict:
    """Full-size check without the whole oracle product:
      * no canary left anywhere in the logical C (beta == 0: C starts as NaN
        canaries, so an output never written is found wherever it is), and the
        ldc padding untouched;
      * every row and every column on a 64-aligned block boundary (the first
        and last row and column of every output tile of every kernel);
      * per_block random points inside every 64 x 64 block of C.
    Returns counts for the report (points, lines, 256 x 256 tiles reached)."""
    got_bits = storage_view(Cout)
    if C0 is None:
        logical_bits = logical(case, got_bits)
        left = int(np.count_nonzero(logical_bits == CANARY[case.dtype]))
        assert left == 0, "%s: %d outputs were never written" % (case.name, left)
    pad = padding_mask(case)
    assert np.array_equal(got_bits[pad], storage_view(Cin)[pad]), "%s: wrote outside C" % case.name
    got = logical(case, oracle.decode(case.dtype, got_bits))
    a, b = storage_view(A), storage_view(B)
    c0 = None if C0 is None else storage_view(C0)
    rows = boundary_lines(case.M)
    cols = boundary_lines(case.N)
    reports = []
    exact = oracle.gemm(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha, a,
                        case.lda, b, case.ldb, case.beta, c0, None, case.ldc, case.dtype,
                        rows=np.asarray(rows, np.int64))
    reports.append(("rows", compare(case, got[rows], exact)))
    reports.append(("cols", compare(case, got[:, cols], exact_cols(case, A, B, C0, cols))))
    pi, pj = block_points(case.M, case.N, block, per_block, seed)
    exact = oracle.gemm_points(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha,
                               a, case.lda, b, case.ldb, case.beta, c0, case.ldc, case.dtype,
                               pi, pj)
    reports.append(("points", compare(case, got[pi, pj], exact)))
    for what, r in reports:
        assert r["ok"], "%s (%s): %s" % (case.name, what, r)
    tiles = {(int(i) // 256, int(j) // 256) for i, j in zip(pi, pj)}
    return {"points": int(pi.size), "rows": len(rows), "cols": len(cols),
            "tiles_256_reached": len(tiles),
            "tiles_256": ((case.M + 255) // 256) * ((case.N + 255) // 256),
            "max_err": max(r["max_err"] for _, r in reports),
            "over_bare_tol": sum(r.get("over_bare_tol", 0) for _, r in reports)}


def sample_rows(M: int, tile: int = 256, extra: int = 16, seed: int = 0) -> list[int]:
    """Rows covering every tile boundary class plus random ones."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, M - 1, M - 2}
    for b in (16, 31, 32, 33, 63, 64, 127, 128, 129, 191, 192, 255, 256):
        if b < M:
            rows.add(b)
    t = tile
    while t < M:
        rows.update({t - 1, t})
        t += tile * max(1, (M // tile) // 6)
    rows.update(int(x) for x in rng.integers(0, M, extra))
    return sorted(r for r in rows if 0 <= r < M)


# ---------------------------------------------------------------------------
# SiLU epilogue: Y = round(SiLU(round(C))).
#
# Against the oracle's unrounded Y_exact = SiLU(round(C_exact)) (FP64):
#   * exact GEMM (integer data): the kernel's rounded C equals the oracle's,
#     so only the FP32 evaluation of SiLU and the final rounding differ:
#     |Y - Y_exact| <= ulp(Y) (one unit of the output format; FP32: 4 units);
#   * general data: SiLU is 1.1-Lipschitz, so the GEMM bound on C (plus one
#     output ulp for rounding C to the other side of a tie) carries over:
#     |Y - Y_exact| <= 1.1 * (tol_C + ulp(C)) + ulp(Y).
# ---------------------------------------------------------------------------
def silu_reference(case: Case, c_exact, exact_gemm=False):
    """(Y_exact, per-element bound) for the SiLU epilogue given the oracle's
    unrounded GEMM values."""
    y_exact = oracle.silu_epilogue(case.dtype, c_exact)
    y_r = oracle.round_to(case.dtype, y_exact)
    c_r = oracle.round_to(case.dtype, c_exact)
    if case.dtype == "f32":
        uy = np.maximum(np.abs(y_r), 2.0 ** -126) * 2.0 ** -23 * 4
        uc = np.maximum(np.abs(c_r), 2.0 ** -126) * 2.0 ** -23
        scale = float(np.max(np.abs(c_exact))) if np.size(c_exact) else 0.0
        tol_c = tol_f32_rel(case.K) * max(scale, 1e-30)
    else:
        uy, uc = _ulp(case.dtype, y_r), _ulp(case.dtype, c_r)
        tol_c = tol_half(case.K)
    bound = uy if exact_gemm else 1.1 * (tol_c + uc) + uy
    return y_exact, bound


def check_silu(case: Case, A, B, C0, Cin, Cout, rows=None, exact_gemm=False):
    a, b = storage_view(A), storage_view(B)
    c0 = None if C0 is None else storage_view(C0)
    c_exact = oracle.gemm(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha, a,
                          case.lda, b, case.ldb, case.beta, c0, None, case.ldc, case.dtype,
                          rows=None if rows is None else np.asarray(rows, np.int64))
    y_exact, bound = silu_reference(case, c_exact, exact_gemm)
    got_all = logical(case, oracle.decode(case.dtype, storage_view(Cout)))
    got = got_all if rows is None else got_all[np.asarray(rows)]
    err = np.abs(got - y_exact)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, "%s: %d outputs off, first %s: got %r want %r (bound %r)" % (
        case.name, len(bad), tuple(bad[0]), got[tuple(bad[0])], y_exact[tuple(bad[0])],
        bound[tuple(bad[0])] if np.ndim(bound) else bound)
    pad = padding_mask(case)
    assert np.array_equal(storage_view(Cout)[pad], storage_view(Cin)[pad]), "%s: wrote outside C" % case.name
    return float(np.max(err)) if err.size else 0.0


# ---------------------------------------------------------------------------
# Gated pair: Z = round(T * round(U)), T = round(SiLU(round(G))).
#   * exact GEMMs (integer data): G and U round exactly as in the oracle; T
#     may land one unit of the format away (FP32 SiLU), which moves T*U by
#     |U| ulp(T): |Z - Z_exact| <= |U| ulp(T) + ulp(Z);
#   * general data: dT <= 1.1 (tol + ulp(G)) + ulp(T), dU <= tol + ulp(U),
#     |Z - Z_exact| <= |U| dT + |T| dU + dT dU + ulp(Z).
# ---------------------------------------------------------------------------
def check_gated(case: Case, X, Wg, Wu, Zout, rows=None, exact_gemm=False):
    xs, gs, us = storage_view(X), storage_view(Wg), storage_view(Wu)
    r = None if rows is None else np.asarray(rows, np.int64)
    kw = dict(rows=r)
    g = oracle.gemm("row", "row", case.M, case.N, case.K, 1.0, xs, case.lda, gs, case.ldb, 0.0,
                    None, None, case.ldc, case.dtype, **kw)
    u = oracle.gemm("row", "row", case.M, case.N, case.K, 1.0, xs, case.lda, us, case.ldb, 0.0,
                    None, None, case.ldc, case.dtype, **kw)
    z = oracle.swiglu(case.dtype, g, u)
    t_r = oracle.round_to(case.dtype, oracle.silu_epilogue(case.dtype, g))
    u_r = oracle.round_to(case.dtype, u)
    g_r = oracle.round_to(case.dtype, g)
    uz = _ulp(case.dtype, oracle.round_to(case.dtype, z))
    ut = _ulp(case.dtype, t_r)
    if exact_gemm:
        bound = np.abs(u_r) * ut + uz
    else:
        tol = tol_half(case.K)
        dT = 1.1 * (tol + _ulp(case.dtype, g_r)) + ut
        dU = tol + _ulp(case.dtype, u_r)
        bound = np.abs(u_r) * dT + np.abs(t_r) * dU + dT * dU + uz
    got_all = oracle.decode(case.dtype, storage_view(Zout)).reshape(-1, case.ldc)[: case.M, : case.N]
    got = got_all if rows is None else got_all[np.asarray(rows)]
    err = np.abs(got - z)
    # An output that overflows the format is inf on both sides.
    z_r = oracle.round_to(case.dtype, z)
    err = np.where(np.isinf(z_r) & (got == z_r), 0.0, err)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, "%s: %d outputs off, first %s: got %r want %r (bound %r)" % (
        case.name, len(bad), tuple(bad[0]), got[tuple(bad[0])], z[tuple(bad[0])], bound[tuple(bad[0])])
    return float(np.max(err)) if err.size else 0.0
