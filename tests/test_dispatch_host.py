"""Host logic of the measured dispatch table (no device needed).

mgemm_weighted_choice picks, among variants timed on several shapes, the one
with the smallest total time weighted by each shape's call count ("Chapter 5:
Operators and Runtime", section 5.4.5, Example 5-9).  Pinned to the
example's printed numbers (tests/golden/pages_numbers.json).
"""
import json
import os
from fractions import Fraction

import pytest

import dense_gemm_mgemm_amd as mg

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
EX = GOLD["shape_mix_choice"]


@pytest.fixture(scope="module")
def lib():
    try:
        return mg.load()
    except OSError as e:
        pytest.skip(str(e))


def times():
    # rows: shapes A, B; columns: old, new implementation
    return [[EX["old_us"][0], EX["new_us"][0]], [EX["old_us"][1], EX["new_us"][1]]]


def test_example_totals_and_choice(lib):
    t = times()
    for calls, totals, want in ((EX["calls_equal"], EX["totals_equal_us"], 0),
                                (EX["calls_skewed"], EX["totals_skewed_us"], 1)):
        got = [sum(c * t[s][v] for s, c in enumerate(calls)) for v in range(2)]
        assert got == totals
        assert mg.mgemm_weighted_choice(t, calls) == want
    assert round(EX["totals_skewed_us"][0] / EX["totals_skewed_us"][1], 1) == EX["speedup_skewed"]


def test_example_threshold(lib):
    # The new implementation wins exactly when A's share of the calls exceeds
    # 2/3; at 2/3 the totals tie and the lower index (the old one) is kept.
    t = times()
    thr = Fraction(EX["threshold_share_of_A"])
    for a in range(0, 31):
        for b in range(0, 31):
            if a + b == 0:
                continue
            want = 1 if Fraction(a, a + b) > thr else 0
            assert mg.mgemm_weighted_choice(t, [a, b]) == want, (a, b)


def test_unrunnable_variants_and_zero_calls(lib):
    inf, nan = float("inf"), float("nan")
    # Variant 0 cannot run shape 1: out, unless shape 1 is never called.
    t = [[1.0, 5.0, 3.0], [inf, 5.0, nan]]
    assert mg.mgemm_weighted_choice(t, [1, 1]) == 1
    assert mg.mgemm_weighted_choice(t, [1, 0]) == 0
    assert mg.mgemm_weighted_choice([[inf, nan]], [1]) == -1
    assert mg.mgemm_weighted_choice([[2.0, -1.0]], [1]) == 0       # negative time: out
    assert mg.mgemm_weighted_choice([[3.0, 2.0]]) == 1               # calls omitted: one each


def test_invalid_arguments(lib):
    assert mg.mgemm_weighted_choice([[1.0]], [-1]) == -1
    assert mg.mgemm_weighted_choice([[1.0]], [float("nan")]) == -1
    assert lib.mgemm_weighted_choice(0, 1, None, None) == -1
    assert lib.mgemm_weighted_choice(1, 0, None, None) == -1
