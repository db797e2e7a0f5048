"""The clock-stamp measurement hook (mgemm_set_clock_stamps): the kernels
that record stamps write one (cycles, ticks) pair per workgroup within the
buffer's capacity, the clock they give is plausible, results are the same
bits with the hook on or off, and a NULL buffer turns it off."""
import sys

import pytest
import torch

import dense_gemm_mgemm_amd as mg
import workloads as W

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


def _launch(h, case, dA, dB, dC, kernel, ks):
    mg.mgemm_run_variant(h, kernel, ks, case.layoutA, case.layoutB, case.M, case.N, case.K,
                         case.alpha, dA, case.lda, dB, case.ldb, case.beta, dC, case.ldc,
                         case.dtype)


# (case, kernel, ksplit, workgroups launched)
CASES = [
    (W.Case("sq", 1024, 1024, 1024, "f16", kindA="int", kindB="int", seeds=(1, 2, 3)),
     "h_dma_256x256", 1, 16),
    (W.Case("share", 1024, 1536, 4096, "bf16", kindA="int", kindB="int", seeds=(4, 5, 6)),
     "h_dma_128x192", 4, 8 * 8 * 4),
    (W.Case("skinny", 16, 4096, 4096, "bf16", kindA="int", kindB="int", seeds=(7, 8, 9)),
     "skinny_sk", 4, 16 * 4),
    (W.Case("m64", 64, 3072, 4096, "bf16", kindA="int", kindB="int", seeds=(10, 11, 12)),
     "h_dma_64x192", 4, 16 * 4),
]


@pytest.mark.parametrize("case,kernel,ks,wgs", CASES, ids=[c[0].name for c in CASES])
def test_stamps_cover_the_grid_and_leave_results_alone(h, case, kernel, ks, wgs):
    A, B, C0 = case.make()
    dA, dB = A.cuda(), B.cuda()
    ref = W.c_initial(case, C0).cuda()
    _launch(h, case, dA, dB, ref, kernel, ks)
    cap = wgs + 8
    buf = torch.zeros(4 * cap, dtype=torch.int64, device="cuda")
    got = W.c_initial(case, C0).cuda()
    mg.mgemm_set_clock_stamps(h, buf, cap)
    try:
        _launch(h, case, dA, dB, got, kernel, ks)
    finally:
        mg.mgemm_set_clock_stamps(h, None, 0)
    torch.cuda.synchronize()
    bits = torch.int16 if case.dtype != "f32" else torch.int32
    assert torch.equal(got.view(bits), ref.view(bits))
    st = buf.view(cap, 4).cpu()
    written = (st[:, 3] > st[:, 2]) & (st[:, 1] > st[:, 0])
    assert int(written[:wgs].sum()) == wgs and int(written[wgs:].sum()) == 0, st
    mhz = 100.0 * (st[:wgs, 1] - st[:wgs, 0]).double() / (st[:wgs, 3] - st[:wgs, 2]).double()
    say(case.name, kernel, "MHz min/median/max", mhz.min().item(), mhz.median().item(),
        mhz.max().item())
    assert bool((mhz > 100).all()) and bool((mhz < 2600).all())
    # A smaller capacity: only the first workgroups write; the hook off: nothing.
    small = torch.zeros(4 * 4, dtype=torch.int64, device="cuda")
    mg.mgemm_set_clock_stamps(h, small, 2)
    try:
        _launch(h, case, dA, dB, got, kernel, ks)
    finally:
        mg.mgemm_set_clock_stamps(h, None, 0)
    off = torch.zeros(4 * cap, dtype=torch.int64, device="cuda")
    _launch(h, case, dA, dB, got, kernel, ks)
    torch.cuda.synchronize()
    s2 = small.view(4, 4).cpu()
    assert bool((s2[:2, 3] > s2[:2, 2]).all()) and bool((s2[2:] == 0).all())
    assert int(off.count_nonzero()) == 0


def test_set_clock_stamps_rejects_bad_arguments(h):
    buf = torch.zeros(8, dtype=torch.int64, device="cuda")
    for args in ((buf, 0), (buf, -1)):
        with pytest.raises(mg.MgemmError) as ei:
            mg.mgemm_set_clock_stamps(h, *args)
        assert ei.value.status == mg.MGEMM_ERR_INVALID_ARG


def test_fp8_stamps_cover_the_grid_and_leave_results_alone(h):
    """The FP8 MFMA kernel (256x192 tiles: 2 x 4 workgroups here) records
    stamps; its codes and scaled output are the same bits with the hook on."""
    M, N, K = 512, 768, 1024
    g = torch.Generator().manual_seed(21)
    x = (torch.rand(M, K, generator=g) * 2 - 1).to(torch.bfloat16).cuda()
    w = (torch.rand(N, K, generator=g) * 2 - 1).to(torch.bfloat16).cuda()
    qx = torch.empty(M * K, dtype=torch.uint8, device="cuda")
    qw = torch.empty(N * K, dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    sw = torch.empty(N, dtype=torch.float32, device="cuda")
    mg.mgemm_quantize_fp8(h, M, K, x, K, "bf16", qx, K, sx)
    mg.mgemm_quantize_fp8(h, N, K, w, K, "bf16", qw, K, sw)

    def run(out):
        mg.mgemm_run_fp8(h, "f8_mfma_256x192", M, N, K, 1.0, qx, K, sx, qw, K, sw, 0.0, out, N,
                         "bf16", ksplit=1)

    ref = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    run(ref)
    wgs, cap = 2 * 4, 16
    buf = torch.zeros(4 * cap, dtype=torch.int64, device="cuda")
    got = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    mg.mgemm_set_clock_stamps(h, buf, cap)
    try:
        run(got)
    finally:
        mg.mgemm_set_clock_stamps(h, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    st = buf.view(cap, 4).cpu()
    written = (st[:, 3] > st[:, 2]) & (st[:, 1] > st[:, 0])
    assert int(written[:wgs].sum()) == wgs and int(written[wgs:].sum()) == 0, st
