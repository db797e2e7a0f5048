"""CPU checks of the GPU parity helpers themselves (no GPU needed): the
stratified full-size check must accept the oracle's own rounded output and
reject an output block that was never written or holds wrong values, and the
column form must agree with the full product in every layout pair."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import parity as P


def _oracle_output(case):
    A, B, C0 = case.make()
    Cin = W.c_initial(case, C0)
    out = W.storage_view(Cin).copy()
    oracle.gemm(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha,
                W.storage_view(A), case.lda, W.storage_view(B), case.ldb, case.beta,
                None if C0 is None else W.storage_view(C0), out, case.ldc, case.dtype,
                want_exact=False)
    Cout = torch.from_numpy(out.view(np.int32 if case.dtype == "f32" else np.int16).copy())
    Cout = Cout.view(W.TORCH_DTYPES[case.dtype])
    return A, B, C0, Cin, Cout


@pytest.mark.parametrize("layouts", list(itertools.product(["row", "col"], ["row", "col"])))
def test_exact_cols_match_full_product(layouts):
    la, lb = layouts
    case = W.Case("cols", 70, 45, 33, "bf16", layoutA=la, layoutB=lb, beta=0.5,
                  lda=(33 if la == "row" else 70) + 3, ldb=(45 if lb == "row" else 33) + 1,
                  ldc=(45 if la == "row" else 70) + 2, seeds=(1, 2, 3))
    A, B, C0 = case.make()
    full = oracle.gemm(la, lb, case.M, case.N, case.K, case.alpha, W.storage_view(A), case.lda,
                       W.storage_view(B), case.ldb, case.beta, W.storage_view(C0), None,
                       case.ldc, case.dtype)
    cols = [0, 7, 44]
    assert np.array_equal(P.exact_cols(case, A, B, C0, cols), full[:, cols])


def test_stratified_accepts_oracle_output_and_reaches_every_tile():
    case = W.Case("strat", 300, 520, 96, "f16", layoutA="col", layoutB="col", seeds=(4, 5, 6))
    rep = P.check_stratified(case, *_oracle_output(case))
    assert rep["tiles_256_reached"] == rep["tiles_256"] == 6
    assert rep["points"] >= 4 * (300 // 64) * (520 // 64)


def test_stratified_rejects_unwritten_and_wrong_blocks():
    case = W.Case("strat", 256, 384, 64, "bf16", seeds=(7, 8, 9))
    A, B, C0, Cin, Cout = _oracle_output(case)
    bits = W.storage_view(Cout).reshape(case.M, case.ldc)
    # One 64 x 64 block left unwritten (still the canary).
    holed = bits.copy()
    holed[64:128, 128:192] = W.CANARY["bf16"]
    with pytest.raises(AssertionError, match="never written"):
        P.check_stratified(case, A, B, C0, Cin, torch.from_numpy(holed.view(np.int16).reshape(-1))
                           .view(torch.bfloat16))
    # One interior block with a wrong value (written, but twice as large).
    wrong = bits.copy()
    vals = oracle.decode("bf16", wrong[130:190, 200:250]) * 2 + 1
    wrong[130:190, 200:250] = oracle.encode("bf16", vals)
    with pytest.raises(AssertionError, match="points"):
        P.check_stratified(case, A, B, C0, Cin, torch.from_numpy(wrong.view(np.int16).reshape(-1))
                           .view(torch.bfloat16))
