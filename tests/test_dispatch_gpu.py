"""Measured dispatch table on the GPU: mgemm_tune fills a handle's table, the
table steers mgemm_run (exact shapes, then power-of-two buckets), survives an
export/import round trip, and results stay within the oracle's tolerance."""
import sys

import pytest
import torch

import dense_gemm_mgemm_amd as mg
import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture()
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.load()
    handle = mg.mgemm_create()
    yield handle
    mg.mgemm_destroy(handle)


def sel(h, M, N, K, dtype="bf16"):
    return mg.mgemm_select_variant(h, "row", "row", M, N, K, 1.0, 256, K, 256, N, 0.0, 256, N,
                                   dtype)


# The FFN share at the pages' row mix (Example 5-12 of section 5.5.3: eight
# calls of 256 rows for each of 1536 and 2048), plus a K-heavy shape.
SHAPES = [(256, 1536, 4096), (1536, 1536, 4096), (2048, 1536, 4096), (512, 4096, 8192)]
CALLS = [8, 1, 1, 1]


def test_tune_steers_dispatch_and_round_trips(h):
    model = {s: sel(h, *s) for s in SHAPES}
    say("model:", model)
    res = mg.mgemm_tune(h, "bf16", "row", "row", SHAPES, CALLS)
    for r in res:
        # The fastest measured variant; the model's pick is timed as well
        # (separately when the tuner's split list does not hold it).  The
        # ratio is reported, not asserted: a clock dip on a busy box can move
        # either time without anything being wrong.
        say("tuned", r, "model/chosen = %.3f" % (r["model_us"] / r["chosen_us"]))
        assert r["chosen_us"] > 0 and r["model_us"] > 0
    text = mg.mgemm_table_export(h)
    say(text)
    lines = [l for l in text.splitlines() if l and not l.startswith("#")]
    assert sum(l.startswith("exact ") for l in lines) == len(SHAPES)
    assert any(l.startswith("bucket ") for l in lines)
    tuned = {s: sel(h, *s) for s in SHAPES}
    for s, r in zip(SHAPES, res):
        assert tuned[s][0] == r["chosen"][0], (s, tuned[s], r)
    # Clearing the table gives the model back; importing the text restores it.
    mg.mgemm_table_clear(h)
    assert {s: sel(h, *s) for s in SHAPES} == model
    mg.mgemm_table_import(h, text)
    assert {s: sel(h, *s) for s in SHAPES} == tuned
    # A shape that was not tuned takes its bucket's choice: 1000 rows round
    # up to 1024 like 1024 rows would (log2 buckets of M, N and K).
    h2 = mg.mgemm_create()
    try:
        mg.mgemm_tune(h2, "bf16", "row", "row", [(1024, 1536, 4096), (700, 1536, 4096)], [8, 1])
        b = [l for l in mg.mgemm_table_export(h2).splitlines() if l.startswith("bucket ")]
        assert len(b) == 1 and b[0].split()[4:7] == ["10", "11", "12"], b
        kname, ks_req = b[0].split()[7], int(b[0].split()[8])
        got = sel(h2, 1000, 1536, 4096)
        assert got[0] == kname, (got, b)
    finally:
        mg.mgemm_destroy(h2)


def test_tuned_results_match_oracle(h):
    case = W.ffn_share_bf16()
    mg.mgemm_tune(h, "bf16", "row", "row", [(case.M, case.N, case.K)])
    say("tuned share:", sel(h, case.M, case.N, case.K))
    out = P.run_gpu(h, case)
    P.check_tolerance(case, *out, rows=P.sample_rows(case.M, 192, extra=8))
    # Integer data at a shape of the same bucket: bit-exact through the bucket entry.
    ci = W.Case("bucket_int", 1000, 1536, 4096, "bf16", kindA="int", kindB="int", seeds=(1, 2, 3))
    P.check_bit_exact(ci, *P.run_gpu(h, ci))


def test_table_import_errors_leave_table_unchanged(h):
    good = "exact bf16 1 0 64 64 64 h_dma_256x192 2 1.0\n"
    mg.mgemm_table_import(h, good)
    before = mg.mgemm_table_export(h)
    for bad in ("exact bf16 1 0 64 64 64 no_such_kernel 1 1.0\n",
                "exact bf16 1 0 64 64 h_dma_256x192 1 1.0\n",
                "exact bf16 1 0 64 64 64 f32_fast 3 1.0\n",       # split on a kernel without one
                "bucket f16 1 0 99 1 1 h_dma_256x256 1 1.0\n",
                "sometimes bf16 1 0 64 64 64 general 1 1.0\n",
                good + "exact bf16 1 0 64 64 64 general 1 1.0 trailing\n"):
        with pytest.raises(mg.MgemmError) as ei:
            mg.mgemm_table_import(h, bad)
        assert ei.value.status == mg.MGEMM_ERR_INVALID_ARG
        assert mg.mgemm_table_export(h) == before
    # Blank lines and comments are fine; an entry for a variant that cannot
    # run the call falls through to the model.
    mg.mgemm_table_import(h, "\n# comment\n\nexact f32 1 0 33 33 33 f32_fast 1 1.0\n")
    name, _ = mg.mgemm_select_variant(h, "row", "row", 33, 33, 33, 1.0, 256, 33, 256, 33, 0.0,
                                      256, 33, "f32")
    assert name != "f32_fast"      # 33-float rows are not 16-byte aligned
    case = W.Case("fallthrough", 33, 33, 33, "f32", kindA="int", kindB="int", seeds=(4, 5, 6))
    P.check_bit_exact(case, *P.run_gpu(h, case))


def test_tune_argument_errors(h):
    for shapes, calls in (([], None), ([(0, 4, 4)], None), ([(4, 4, 4)], [-1.0])):
        with pytest.raises(mg.MgemmError) as ei:
            if shapes:
                mg.mgemm_tune(h, "bf16", "row", "row", shapes, calls)
            else:
                st = mg.load().mgemm_tune(h, 2, 0, 0, 0, None, None, None, None, None, None)
                raise mg.MgemmError(st, "mgemm_tune")
        assert ei.value.status == mg.MGEMM_ERR_INVALID_ARG


def test_tune_other_dtypes_and_layouts(h):
    # FP32 (aligned and ragged), column-major FP16, skinny BF16 and the mixed
    # layout pairs (weights stored out x in included): the
    # tuner measures whatever can run each one, the table steers mgemm_run,
    # and the results stay exact on integer data.
    cases = [("f32", "row", "row", [(1000, 1000, 1000), (512, 512, 2048)]),
             ("f32", "col", "row", [(512, 512, 1024)]),
             ("f16", "col", "col", [(512, 1024, 2048)]),
             ("bf16", "row", "row", [(16, 12288, 4096), (64, 6144, 1024)]),
             ("bf16", "row", "col", [(512, 1024, 2048), (16, 4096, 2048)])]
    for dtype, la, lb, shapes in cases:
        res = mg.mgemm_tune(h, dtype, la, lb, shapes)
        for r in res:
            say("tuned", dtype, la, lb, r, "model/chosen = %.3f" % (r["model_us"] / r["chosen_us"]))
            assert r["chosen_us"] > 0 and r["model_us"] > 0, r
        for (M, N, K) in shapes:
            case = W.Case("tuned_int", M, N, K, dtype, layoutA=la, layoutB=lb, kindA="int",
                          kindB="int", seeds=(M, N, K))
            P.check_bit_exact(case, *P.run_gpu(h, case))
    text = mg.mgemm_table_export(h)
    assert "exact f32" in text and "exact f16" in text and "exact bf16" in text
