"""Helpers for GPU parity tests: run a workload through libmgemm and compare it
with the CPU oracle on the same seeded inputs.

Bars (the tolerance rules come with the workloads):
  * integer-valued inputs: the whole C buffer, bit for bit, equals the
    oracle's (every partial sum is exact in FP32, so one rounding of the exact
    integer is the only answer);
  * FP32: max|C - C_exact| <= 1e-4 * sqrt(K/256) * max|C_exact|;
  * FP16/BF16: per element |C - C_exact| <= 0.01*sqrt(K/512) + ulp(C_exact)/2,
    the stated absolute bound plus the output format's own rounding;
  * outside the logical M x N region (the ldc padding) C is never written.
"""
from __future__ import annotations

import numpy as np
import torch

import dense_gemm_mgemm_amd as mg
import oracle
from dense_gemm_mgemm_amd.costmodel import tol_f32_rel, tol_half
from workloads import Case, storage_view

# Canary bit patterns written into C before a call (quiet NaNs).
CANARY = {"f32": 0x7FA5A5A5, "f16": 0x7E5A, "bf16": 0x7FA5}

KERNELS_F32 = ["general", "f32_mfma", "f32_fast", "f32_fast_128", "f32_fast_u", "f32_sk"]
KERNELS_16 = ["general", "h_mfma_256x256", "h_mfma_256x192", "h_mfma_128x128", "h_pp_256x256",
              "h_dma_256x256", "h_dma_256x192", "h_dma_128x192"]


def c_initial(case: Case, C0):
    """Initial C buffer (CPU): C0 when beta != 0, else canary bits everywhere."""
    if C0 is not None:
        return C0.clone()
    n = case.c_numel()
    if case.dtype == "f32":
        return torch.full((n,), CANARY["f32"], dtype=torch.int32).view(torch.float32)
    t = torch.full((n,), CANARY[case.dtype], dtype=torch.int16)   # both patterns < 0x8000
    return t.view(torch.float16 if case.dtype == "f16" else torch.bfloat16)


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
    # Half an ulp of the output format at the exact value: the distance from
    # the exact value to its rounding is at most that, and the bound allows it.
    rounded = oracle.round_to(case.dtype, exact)
    ulp = _ulp(case.dtype, rounded)
    bound = tol + 0.5 * ulp
    ok = bool(np.all(err <= bound)) and not np.isnan(got).any()
    return {"ok": ok, "max_err": float(np.nanmax(err)) if err.size else 0.0, "tol": tol,
            "over_bare_tol": int(np.sum(err > tol))}


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
