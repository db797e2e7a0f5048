"""mgemm_run_noalloc (no handle, no allocation: static scratch array) against
mgemm_run_variant (the handle's workspace), through the C ABI.

Integer-valued inputs make every partial sum exact, so the two entry points
must give the same bits whatever split each one runs, and both must equal
the oracle's.  Each pair of calls runs the larger problem first and a
smaller one second on the same static array, so the second call sees the
first call's leftovers (partials, counters back at zero)."""
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


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.load()
    handle = mg.mgemm_create()
    yield handle
    mg.mgemm_destroy(handle)


def _run(case, inputs, kernel, ksplit, h=None):
    A, B, C0 = inputs
    Cin = W.c_initial(case, C0)
    dA, dB, dC = A.cuda(), B.cuda(), Cin.cuda()
    args = (case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha, dA, case.lda, dB,
            case.ldb, case.beta, dC, case.ldc, case.dtype)
    if h is None:
        mg.mgemm_run_noalloc(kernel, ksplit, *args)
    else:
        mg.mgemm_run_variant(h, kernel, ksplit, *args)
    torch.cuda.synchronize()
    return A, B, C0, Cin, dC.cpu()


def _int_case(name, M, N, K, dtype, la="row", lb="row", beta=0.0, seeds=(1, 2, 3), **kw):
    return W.Case(name, M, N, K, dtype, layoutA=la, layoutB=lb, kindA="int", kindB="int",
                  kindC="int", beta=beta, seeds=seeds, **kw)


# (larger case, smaller case, kernel, ksplit): every form that uses scratch
# memory, then the library's own choice.
PAIRS = [
    (_int_case("skinny16", 16, 12288, 4096, "bf16", seeds=(11, 12, 13)),
     _int_case("skinny5", 5, 1000, 512, "bf16", beta=-0.5, seeds=(14, 15, 16)),
     "skinny_sk", 4),
    (_int_case("share", 1024, 1536, 4096, "bf16", seeds=(21, 22, 23)),
     _int_case("share_small", 300, 520, 1024, "bf16", beta=2.0, seeds=(24, 25, 26)),
     "h_dma_128x192", 4),
    (_int_case("col", 1024, 1024, 2048, "f16", la="col", lb="col", seeds=(31, 32, 33)),
     _int_case("col_small", 512, 256, 512, "f16", la="col", lb="col", seeds=(34, 35, 36)),
     "h_dma_256x256", 3),
    (_int_case("ktail", 520, 1536, 1000, "bf16", seeds=(71, 72, 73)),
     _int_case("ktail_small", 300, 520, 104, "bf16", beta=-0.5, seeds=(74, 75, 76)),
     "h_dma_128x192", 3),
    (_int_case("m64", 64, 12288, 4096, "bf16", seeds=(61, 62, 63)),
     _int_case("m40", 40, 1000, 1024, "bf16", beta=-1.0, seeds=(64, 65, 66)),
     "h_dma_64x192", 4),
    (_int_case("auto_share", 1024, 1536, 4096, "bf16", seeds=(41, 42, 43)),
     _int_case("auto_skinny", 16, 4096, 4096, "f16", seeds=(44, 45, 46)),
     "auto", 0),
    (_int_case("auto_ragged", 1000, 12290, 4095, "f32", lda=4095, ldb=12290, ldc=12290,
               seeds=(51, 52, 53)),
     _int_case("auto_f32", 200, 136, 72, "f32", seeds=(54, 55, 56)),
     "auto", 0),
]


@pytest.mark.parametrize("big,small,kernel,ksplit", PAIRS, ids=[p[0].name for p in PAIRS])
def test_noalloc_matches_handle_entry(h, big, small, kernel, ksplit):
    for case in (big, small):
        say("noalloc", case.name, (case.M, case.N, case.K), case.dtype, kernel, ksplit)
        inputs = case.make()
        ref = _run(case, inputs, kernel, ksplit, h=h)
        got = _run(case, inputs, kernel, ksplit)
        assert torch.equal(got[4].view(torch.int16 if case.dtype != "f32" else torch.int32),
                           ref[4].view(torch.int16 if case.dtype != "f32" else torch.int32)), case.name
        P.check_bit_exact(case, *got)


def test_noalloc_refuses_splits_beyond_its_scratch():
    # Stream-K on the ragged FP32 workload needs 128 MiB of partial tiles; a
    # 2048 x 2048 FP16 product cut into 8 ranges of 256 x 256 tiles needs
    # 128 MiB: both exceed the 32 MiB array.  Nothing is launched and C is
    # untouched.
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for case, kernel, ksplit in (
            (_int_case("ragged", 1000, 12290, 4095, "f32", lda=4095, ldb=12290, ldc=12290), "f32_sk", 1),
            (_int_case("big_split", 2048, 2048, 4096, "f16"), "h_dma_256x256", 8)):
        say("noalloc refuses", case.name, kernel, ksplit)
        A, B, C0 = case.make()
        Cin = W.c_initial(case, C0)
        dC = Cin.cuda()
        with pytest.raises(mg.MgemmError) as ei:
            mg.mgemm_run_noalloc(kernel, ksplit, case.layoutA, case.layoutB, case.M, case.N, case.K,
                                 1.0, A.cuda(), case.lda, B.cuda(), case.ldb, 0.0, dC, case.ldc,
                                 case.dtype)
        assert ei.value.status == mg.MGEMM_ERR_SCRATCH
        torch.cuda.synchronize()
        assert torch.equal(dC.cpu().view(torch.int16 if case.dtype != "f32" else torch.int32),
                           Cin.view(torch.int16 if case.dtype != "f32" else torch.int32))
    # A variant that cannot run the shape at all is still "unsupported".
    case = _int_case("odd", 64, 64, 33, "f16")
    A, B, _ = case.make()
    with pytest.raises(mg.MgemmError) as ei:
        mg.mgemm_run_noalloc("h_dma_256x256", 1, "row", "row", 64, 64, 33, 1.0, A.cuda(), 33,
                             B.cuda(), 64, 0.0, torch.empty(64 * 64, dtype=torch.float16,
                                                            device="cuda"), 64, "f16")
    assert ei.value.status == mg.MGEMM_ERR_UNSUPPORTED
