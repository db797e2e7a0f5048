"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutation is a plausible slip (a dropped term, a wrong sign, a transposed
operand, a swapped leading dimension, round-half-up instead of ties-to-even,
a lost alpha, a wrong subnormal scale, C's order swapped).  The copy is
compiled with gcc into a temporary library and the pin battery runs against it
in a child process, so a mutant that corrupts memory cannot take the test
runner down with it; the real oracle is never modified.
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "mgemm_oracle.c")

MUTATIONS = {
    "dropped_first_k_term": ("for (int64_t k = 0; k < K; ++k) {\n                double a",
                             "for (int64_t k = 1; k < K; ++k) {\n                double a"),
    "beta_sign": ("if (beta != 0.0) v += beta * orc_decode(dtype, C_in, c_index(layoutA, i, j, ldc));\n                if (exact)",
                  "if (beta != 0.0) v -= beta * orc_decode(dtype, C_in, c_index(layoutA, i, j, ldc));\n                if (exact)"),
    "transposed_b": ("return layout == ORC_ROW ? k * ldb + j : j * ldb + k;",
                     "return layout == ORC_ROW ? j * ldb + k : k * ldb + j;"),
    "lda_for_ldb": ("a_index(layoutA, i, k, lda));\n                const double* brow",
                    "a_index(layoutA, i, k, ldb));\n                const double* brow"),
    "round_half_up": ("double r = rint(n);", "double r = floor(n + 0.5);"),
    "lost_alpha": ("double v = alpha * acc[j];", "double v = acc[j];"),
    "f16_subnormal_scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "points_beta_sign": ("if (beta != 0.0) v += beta * orc_decode(dtype, C_in, c_index(layoutA, i, j, ldc));\n        value[p] = v;",
                         "if (beta != 0.0) v -= beta * orc_decode(dtype, C_in, c_index(layoutA, i, j, ldc));\n        value[p] = v;"),
    "points_b_transposed": ("orc_decode(dtype, B, b_index(layoutB, k, j, ldb));\n        double v = alpha * s;",
                            "orc_decode(dtype, B, b_index(layoutB, j, k, ldb));\n        double v = alpha * s;"),
    "c_row_col_swapped": ("return layout == ORC_ROW ? i * ldc + j : j * ldc + i;",
                          "return layout == ORC_ROW ? j * ldc + i : i * ldc + j;"),
}

CHILD = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r})
    import oracle
    from tests.test_oracle_pins import PIN_CHECKS
    oracle._use_library({lib!r})
    caught = []
    for check in PIN_CHECKS:
        try:
            check()
        except (AssertionError, ValueError):
            caught.append(check.__name__)
    print("CAUGHT", ",".join(caught))
    sys.exit(3 if caught else 0)
""")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    str(mutated), "-o", str(lib), "-lm"], check=True)
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=str(lib))],
                       capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, OMP_NUM_THREADS="2"))
    # exit 3: a pin failed cleanly; a negative code: the mutant crashed the battery.
    assert r.returncode != 0, "no pin caught the planted mistake %s\n%s" % (name, r.stdout)


# Planted mistakes in the SiLU epilogue (plain numpy, so the mutants are
# Python functions swapped in for oracle.silu_epilogue in this process).
def _silu_no_prerounding(dtype, c_exact):
    import numpy as np
    c = np.asarray(c_exact, np.float64)
    return c / (1.0 + np.exp(-c))


def _silu_wrong_exp_sign(dtype, c_exact):
    import numpy as np
    c = oracle.round_to(dtype, c_exact)
    with np.errstate(over="ignore"):
        return c / (1.0 + np.exp(c))


def _sigmoid_only(dtype, c_exact):
    import numpy as np
    c = oracle.round_to(dtype, c_exact)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-c))


@pytest.mark.parametrize("mutant", [_silu_no_prerounding, _silu_wrong_exp_sign, _sigmoid_only],
                         ids=lambda f: f.__name__)
def test_planted_silu_mistake_is_caught(mutant, monkeypatch):
    from tests.test_oracle_pins import check_silu_epilogue
    monkeypatch.setattr(oracle, "silu_epilogue", mutant)
    with pytest.raises(AssertionError):
        check_silu_epilogue()


def _swiglu_no_t_rounding(dtype, g_exact, u_exact):
    return oracle.silu_epilogue(dtype, g_exact) * oracle.round_to(dtype, u_exact)


def _swiglu_gate_on_u(dtype, g_exact, u_exact):
    t = oracle.round_to(dtype, oracle.silu_epilogue(dtype, u_exact))
    return t * oracle.round_to(dtype, g_exact)


@pytest.mark.parametrize("mutant", [_swiglu_no_t_rounding, _swiglu_gate_on_u],
                         ids=lambda f: f.__name__)
def test_planted_swiglu_mistake_is_caught(mutant, monkeypatch):
    from tests.test_oracle_pins import check_swiglu
    monkeypatch.setattr(oracle, "swiglu", mutant)
    with pytest.raises(AssertionError):
        check_swiglu()


# ---------------------------------------------------------------------------
# FP8 oracle (oracle/fp8.py): plausible slips swapped in for its functions.
# ---------------------------------------------------------------------------
from oracle import fp8 as _fp8   # noqa: E402


def _quantize_blockwise(x):
    # Scale from the first 128 elements only (Example 5-7's wrong order).
    x = np.asarray(x, np.float64)
    head = x[:, :128]
    q, s = _REAL_QUANTIZE(head)
    rest = x[:, 128:]
    if rest.shape[1] == 0:
        return q, s
    t = (rest.astype(np.float32) * np.float32(448)) / np.maximum(np.abs(head).max(axis=1), 1e-30).astype(np.float32)[:, None]
    return np.concatenate([q, _fp8.e4m3_encode(np.clip(t, -448, 448))], axis=1), s


def _quantize_multiply(x):
    x = np.asarray(x, np.float64)
    x32 = x.astype(np.float32)
    amax = np.max(np.abs(x32), axis=1)
    s = (amax / np.float32(448)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        t = x32 * s[:, None]                       # multiplies by the scale instead of dividing
    return _fp8.e4m3_encode(t), s


def _encode_half_away(t):
    t = np.asarray(t, np.float64)
    vals = _fp8.e4m3_values()[:0x7F]
    a = np.minimum(np.abs(t), 448.0)
    lo = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    pick = (vals[hi] - a) <= (a - vals[lo])        # ties go up
    mag = np.where(pick, hi, lo).astype(np.uint8)
    code = mag | np.where(np.signbit(t), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(t), np.uint8(0x7F), code).astype(np.uint8)


def _values_bias8():
    v = _REAL_VALUES()
    return np.where(np.isnan(v), v, v / 2.0)       # exponent bias 8 instead of 7


def _gemm_sb_per_row(M, N, K, alpha, qa, lda, sa, qb, ldb, sb, beta=0.0, c0=None):
    sb2 = np.resize(np.asarray(sa, np.float32), N)  # row scales used for the columns too
    return _REAL_GEMM(M, N, K, alpha, qa, lda, sa, qb, ldb, sb2, beta, c0)


def _gemm_qb_transposed(M, N, K, alpha, qa, lda, sa, qb, ldb, sb, beta=0.0, c0=None):
    qb = np.asarray(qb, np.uint8)
    B = _fp8.e4m3_decode(qb[: N * ldb].reshape(N, ldb)[:, :K])
    Bt = np.resize(B.T.ravel(), N * K).reshape(N, K)   # read as K x N
    return _REAL_GEMM(M, N, K, alpha, qa, lda, sa, _fp8.e4m3_encode(Bt).ravel(), K, sb, beta, c0)


_REAL_QUANTIZE, _REAL_VALUES, _REAL_GEMM = _fp8.quantize_rows, _fp8.e4m3_values, _fp8.fp8_gemm

FP8_MUTANTS = [("quantize_rows", _quantize_blockwise), ("quantize_rows", _quantize_multiply),
               ("e4m3_encode", _encode_half_away), ("e4m3_values", _values_bias8),
               ("fp8_gemm", _gemm_sb_per_row), ("fp8_gemm", _gemm_qb_transposed)]


@pytest.mark.parametrize("attr,mutant", FP8_MUTANTS, ids=lambda m: getattr(m, "__name__", m))
def test_planted_fp8_mistake_is_caught(attr, mutant, monkeypatch):
    from tests.test_oracle_fp8 import FP8_PINS
    monkeypatch.setattr(_fp8, attr, mutant)
    failed = []
    for check in FP8_PINS:
        try:
            check()
        except AssertionError:
            failed.append(check.__name__)
    assert failed, "mutant %s passed every FP8 pin" % mutant.__name__
