"""The library's calls captured in a HIP graph (through torch.cuda.CUDAGraph)
and replayed: every path whose kernels share the handle's workspace (split-K
partials and arrival counters, stream-K pieces) and the two-kernel FP8 step.
Each replay follows eager work of the program's own (C poisoned with NaN, an
unrelated product, a synchronisation) and must give the eager call's bits:
the counters return to zero inside every call and no call records a memset,
so replays see the same state as the first launch."""
import sys

import numpy as np
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


def replay_matches_eager(call, out, replays=3):
    """Run `call` eagerly, capture it, then replay it `replays` times with
    unrelated eager work in between; each replay must reproduce the eager
    output exactly."""
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    x = torch.randn(256, 256, device="cuda")
    for r in range(replays):
        out.fill_(float("nan"))
        x = x @ x.T * 1e-3
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs from the eager call" % r
    return ref


GEMM_CASES = [
    # (case, kernel, K ranges) -- FP32 stream-K, the 16-bit two-launch split,
    # the skinny last-arrival split, and the library's own choice for the FFN.
    (W.Case("graph_sk", 1000, 3000, 2000, "f32", lda=2001, seeds=(21, 22, 23)), "f32_sk", 1),
    (W.ffn_share_bf16(), "h_dma_256x192", 5),
    (W.Case("graph_skinny", 16, 12288, 4096, "bf16", kindA="normal", kindB="normal",
            seeds=(24, 25, 26)), "skinny_sk", 4),
    (W.ffn_bf16(), "auto", 0),
    (W.Case("graph_mid_m", 128, 12288, 4096, "bf16", kindA="normal", kindB="normal",
            seeds=(27, 28, 29)), "h_dma_128x192", 4),
    (W.Case("graph_sk_short_m", 16, 6000, 2000, "f32", lda=2001, seeds=(30, 31, 32)), "f32_sk", 1),
    # A K tail (K = 1000) on the split direct-to-LDS kernel, and FP16 rows that
    # are not 16-byte aligned (buffer loads) through the library's choice.
    (W.Case("graph_ktail", 520, 1536, 1000, "bf16", kindA="normal", kindB="normal",
            seeds=(33, 34, 35)), "h_dma_128x192", 3),
    (W.Case("graph_unaligned", 600, 700, 1002, "f16", kindA="normal", kindB="normal",
            lda=1002, ldb=702, seeds=(36, 37, 38)), "auto", 0),
]


@pytest.mark.parametrize("case,kernel,ksplit", GEMM_CASES,
                         ids=["%s-%s" % (c.name, k) for c, k, _ in GEMM_CASES])
def test_gemm_graph_replay(h, case, kernel, ksplit):
    A, B, C0 = case.make()
    dA, dB = A.cuda(), B.cuda()
    dC = P.c_initial(case, None).cuda()
    args = (case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha, dA, case.lda, dB,
            case.ldb, 0.0, dC, case.ldc, case.dtype)
    say("graph", case.name, kernel, ksplit)
    ref = replay_matches_eager(lambda: mg.mgemm_run_variant(h, kernel, ksplit, *args), dC)
    # The eager result itself agrees with the oracle on sampled rows.
    Cin = P.c_initial(case, None)
    P.check_tolerance(case, A, B, None, Cin, ref.cpu(), rows=P.sample_rows(case.M, 64),
                      cols=[0, case.N // 2, case.N - 1])


def test_gated_split_graph_replay(h):
    case = W.ffn_gated_share_bf16()
    X, Wg, Wu = W.gated_inputs(case)
    dX, dWg, dWu = X.cuda(), Wg.cuda(), Wu.cuda()
    dZ = P.c_initial(case, None).cuda()
    say("graph gated", case.name)
    replay_matches_eager(lambda: mg.mgemm_run_gated_ex(h, 4, case.M, case.N, case.K, dX, case.lda,
                                                       dWg, dWu, case.ldb, dZ, case.ldc,
                                                       case.dtype), dZ)


def test_fp8_step_graph_replay(h):
    case = W.fp8_ffn_bf16()
    A, B, _ = case.make()
    M, N, K = case.M, case.N, case.K
    dX, dW = A.cuda(), B.cuda()
    qx = torch.empty(M * K, dtype=torch.uint8, device="cuda")
    qw = torch.empty(N * K, dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    sw = torch.empty(N, dtype=torch.float32, device="cuda")
    mg.mgemm_quantize_fp8(h, N, K, dW, case.ldb, case.dtype, qw, K, sw)
    dC = P.c_initial(case, None).cuda()
    say("graph fp8", case.name)

    def step():
        mg.mgemm_quantize_fp8(h, M, K, dX, case.lda, case.dtype, qx, K, sx)
        mg.mgemm_run_fp8(h, "auto", M, N, K, case.alpha, qx, K, sx, qw, K, sw, 0.0, dC, case.ldc,
                         case.dtype)

    replay_matches_eager(step, dC)
    assert not np.isnan(dC.float().cpu().numpy()).any()
