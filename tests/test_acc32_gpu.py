"""The FP32 sums behind the 16-bit products (mgemm_run_acc32).

The MTT S4000 FP16 GEMM write-up grades outputs against 0.01 * sqrt(K/512)
absolute, which the FP16 spacing exceeds for outputs of magnitude 128 and
more at K = 16384.  These tests hold the kernel's FP32 accumulation to that
bare bound at full size, and show that the 16-bit outputs are those sums
rounded once (round to nearest even), so every excess over the bare bound in
a 16-bit output is the output format's rounding and nothing else.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_mgemm_amd as mg
import oracle
import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.load()
    handle = mg.mgemm_create()
    yield handle
    mg.mgemm_destroy(handle)


def _acc32(h, case, kernel, dA, dB):
    C32 = torch.full((case.c_numel(),), float("nan"), dtype=torch.float32, device="cuda")
    mg.mgemm_run_acc32(h, kernel, case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha,
                       dA, case.lda, dB, case.ldb, C32, case.ldc, case.dtype)
    return C32


def _rounded_equals_16bit(h, case, kernel, dA, dB, C32):
    """The same kernel's 16-bit output (one K range, beta = 0) equals the sums
    rounded to nearest even, everywhere in the logical C."""
    C16 = W.c_initial(case, None).cuda()
    mg.mgemm_run_variant(h, kernel, 1, case.layoutA, case.layoutB, case.M, case.N, case.K,
                         case.alpha, dA, case.lda, dB, case.ldb, 0.0, C16, case.ldc, case.dtype)
    torch.cuda.synchronize()
    r = C32.to(W.TORCH_DTYPES[case.dtype]).view(torch.int16).cpu().numpy()
    g = C16.view(torch.int16).cpu().numpy()
    mask = ~P.padding_mask(case)
    diff = int(np.count_nonzero(r[mask] != g[mask]))
    assert diff == 0, "%s %s: %d outputs differ from the rounded sums" % (case.name, kernel, diff)


SHAPES = [(296, 200, 640), (256, 192, 1024), (520, 776, 320), (40, 104, 160),
          (296, 200, 648), (40, 104, 168)]          # K tails of 8
LAYOUTS = [("row", "row"), ("row", "col"), ("col", "col"), ("col", "row")]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_acc32_integer_sums_are_exact(h, M, N, K):
    # Integer data: every sum is an exact integer, so the FP32 sums must be the
    # oracle's unrounded values exactly, in every operand form and tile width.
    for la, lb in LAYOUTS:
        for dtype in ("f16", "bf16"):
            case = W.Case("acc32_int", M, N, K, dtype, layoutA=la, layoutB=lb, kindA="int",
                          kindB="int", alpha=0.5, seeds=(M, N + 1, K + 2))
            A, B, C0 = case.make()
            dA, dB = A.cuda(), B.cuda()
            for kernel in ("h_dma_256x256", "h_dma_256x192"):
                say("acc32 int", (M, N, K), la, lb, dtype, kernel)
                C32 = _acc32(h, case, kernel, dA, dB)
                torch.cuda.synchronize()
                got = P.logical(case, C32.cpu().numpy())
                exact = oracle.gemm(la, lb, M, N, K, case.alpha, W.storage_view(A), case.lda,
                                    W.storage_view(B), case.ldb, 0.0, None, None, case.ldc, dtype)
                assert np.array_equal(got.astype(np.float64), exact), (la, lb, dtype, kernel)
                pad = P.padding_mask(case)
                assert np.isnan(C32.cpu().numpy()[pad]).all(), "wrote outside C"
                _rounded_equals_16bit(h, case, kernel, dA, dB, C32)


@pytest.mark.parametrize("make,kernel", [
    (lambda: W.hgemm_colmajor(8192, 8192, 16384), "h_dma_256x256"),
    (lambda: W.ffn_bf16(1024), "h_dma_256x192"),
], ids=["fp16_8192x8192x16384_col", "bf16_ffn_1024x12288x4096"])
def test_acc32_within_the_bare_tolerance_at_full_size(h, make, kernel):
    case = make()
    A, B, C0 = case.make()
    dA, dB = A.cuda(), B.cuda()
    say("acc32 full size", case.name, kernel)
    C32 = _acc32(h, case, kernel, dA, dB)
    torch.cuda.synchronize()
    _rounded_equals_16bit(h, case, kernel, dA, dB, C32)
    got = P.logical(case, C32.cpu().numpy())
    assert not np.isnan(got).any(), "outputs never written"
    pi, pj = P.block_points(case.M, case.N, 64, 4, seed=11)
    exact = oracle.gemm_points(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha,
                               W.storage_view(A), case.lda, W.storage_view(B), case.ldb, 0.0,
                               None, case.ldc, case.dtype, pi, pj)
    err = np.abs(got[pi, pj].astype(np.float64) - exact)
    tol = P.tol_half(case.K)
    # The same points rounded to the 16-bit output, for the report.
    r16 = oracle.round_to(case.dtype, got[pi, pj].astype(np.float64))
    over16 = int(np.sum(np.abs(r16 - exact) > tol))
    say(case.name, "points", pi.size, "FP32 sums max err %.3g (bare tol %.3g);" % (err.max(), tol),
        "rounded to", case.dtype, ":", over16, "points over the bare tol")
    assert err.max() <= tol, (case.name, float(err.max()), tol)


def test_acc32_argument_errors(h):
    dA = torch.zeros(64 * 64, dtype=torch.float16, device="cuda")
    dB = torch.zeros(64 * 64, dtype=torch.float16, device="cuda")
    C32 = torch.full((64 * 64,), 7.0, dtype=torch.float32, device="cuda")

    def call(kernel="auto", M=64, N=64, K=64, alpha=1.0, dtype="f16", lda=64, ldc=64):
        mg.mgemm_run_acc32(h, kernel, "row", "row", M, N, K, alpha, dA, lda, dB, 64, C32, ldc, dtype)

    for kw, status in [({"kernel": "f32_fast"}, mg.MGEMM_ERR_INVALID_ARG),
                       ({"lda": 32}, mg.MGEMM_ERR_INVALID_ARG),
                       ({"ldc": 32}, mg.MGEMM_ERR_INVALID_ARG),
                       ({"M": -1}, mg.MGEMM_ERR_INVALID_ARG),
                       ({"dtype": "f32"}, mg.MGEMM_ERR_UNSUPPORTED),
                       ({"K": 16}, mg.MGEMM_ERR_UNSUPPORTED),      # under one 32-wide slice
                       ({"K": 0}, mg.MGEMM_ERR_UNSUPPORTED),
                       ({"alpha": 0.0}, mg.MGEMM_ERR_UNSUPPORTED)]:
        with pytest.raises(mg.MgemmError) as ei:
            call(**kw)
        assert ei.value.status == status, kw
    call(M=0)                                   # empty: a no-op
    torch.cuda.synchronize()
    assert bool((C32 == 7.0).all())             # nothing written by any of the above
