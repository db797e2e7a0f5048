"""FP16 subnormal inputs and outputs (GPU).

Every A element is an FP16 subnormal (or zero), j * 2^-24 with |j| < 1024,
and B holds small integers, so every product and every partial sum is an
integer multiple of 2^-24 below 2^-3 in magnitude: exact in FP32 in any
order.  A kernel that honours subnormal inputs must then give the oracle's
bits; one that flushed them would give zeros.  With alpha = 2^-12 the outputs
themselves fall in the FP16 subnormal range, where they must round to
nearest even like any other value (not flush to zero).
"""
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


CASES = [
    # (M, N, K, layoutA, layoutB, kernels)
    (300, 200, 512, "row", "row", ["auto", "h_dma_256x256", "h_dma_256x192", "h_dma_128x192",
                                   "h_mfma_256x256", "h_mfma_128x128", "general"]),
    (256, 264, 512, "col", "col", ["auto", "h_dma_256x256", "h_dma_256x192"]),
    (296, 200, 512, "row", "col", ["auto", "h_dma_256x256", "h_dma_128x192"]),
    (48, 1000, 1024, "row", "row", ["auto", "h_dma_64x192", "skinny_sk", "skinny"]),
]


@pytest.mark.parametrize("M,N,K,la,lb,kernels", CASES, ids=["%dx%dx%d_%s%s" % c[:5] for c in CASES])
@pytest.mark.parametrize("alpha", [1.0, 2.0 ** -12], ids=["normal_out", "subnormal_out"])
def test_fp16_subnormal_inputs_bit_exact(h, M, N, K, la, lb, kernels, alpha):
    case = W.Case("f16sub", M, N, K, "f16", layoutA=la, layoutB=lb, kindA="f16sub",
                  kindB="int", alpha=alpha, seeds=(M + 7, N + 8, K + 9))
    inputs = case.make()
    A = inputs[0]
    a = A.float().numpy()
    nz = a[np.isfinite(a) & (a != 0)]
    assert nz.size and np.abs(nz).max() < 2.0 ** -14       # every nonzero A is subnormal
    for kernel in kernels:
        say("f16 subnormal inputs", (M, N, K), la, lb, "alpha", alpha, kernel)
        out = P.run_gpu(h, case, kernel, inputs=inputs)
        P.check_bit_exact(case, *out)
        if alpha < 1.0:
            c = P.logical(case, out[4].float().numpy())
            small = np.abs(c[(c != 0) & np.isfinite(c)])
            assert small.size and small.min() < 2.0 ** -14   # subnormal outputs are present
