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
