"""GPU parity: libmgemm against the CPU oracle, through the C ABI.

Every test here needs an MI355X and the built libmgemm.so (marker `gpu`).
Each workload family of the pages is run at its full size (sampled rows and
columns where the oracle would take too long) and every kernel variant is
forced on problems it supports, so that no dispatch branch goes unchecked.
"""
import itertools
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


def supported(h, case, kernel, inputs):
    """Run a forced kernel; returns None if the variant declines the problem."""
    try:
        return P.run_gpu(h, case, kernel, inputs=inputs)
    except mg.MgemmError as e:
        if e.status == mg.MGEMM_ERR_UNSUPPORTED:
            return None
        raise


# ---------------------------------------------------------------------------
# FP32 SGEMM 256^3: random (tolerance) and integer-valued (bit-exact)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kernel", ["auto"] + P.KERNELS_F32)
def test_sgemm_256_uniform(h, kernel):
    case = W.sgemm_256()
    say("sgemm_256_uniform", kernel)
    P.check_tolerance(case, *P.run_gpu(h, case, kernel))


@pytest.mark.parametrize("kernel", ["auto"] + P.KERNELS_F32)
def test_sgemm_256_integer_bit_exact(h, kernel):
    case = W.sgemm_256(int_valued=True)
    say("sgemm_256_int", kernel)
    P.check_bit_exact(case, *P.run_gpu(h, case, kernel))


def test_sgemm_4096_stratified(h):
    case = W.sgemm_4096()
    say("sgemm_4096 auto")
    rep = P.check_stratified(case, *P.run_gpu(h, case))
    say(rep)
    assert rep["tiles_256_reached"] == rep["tiles_256"]


def test_ragged_f32_stratified(h):
    case = W.ragged_f32()
    say("ragged_f32 auto")
    rep = P.check_stratified(case, *P.run_gpu(h, case))
    say(rep)
    assert rep["tiles_256_reached"] == rep["tiles_256"]


# ---------------------------------------------------------------------------
# FP16 column-major contest shapes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", W.HGEMM_SHAPES[:2])
@pytest.mark.parametrize("kernel", ["auto"] + P.KERNELS_16)
def test_hgemm_colmajor_small(h, shape, kernel):
    case = W.hgemm_colmajor(*shape)
    say("hgemm", shape, kernel)
    out = supported(h, case, kernel, case.make())
    if out is None:
        pytest.skip("%s declines this problem" % kernel)
    P.check_tolerance(case, *out)


def test_hgemm_colmajor_8k_stratified(h):
    # The largest workload, in the launch configuration the benchmark times
    # (the library's own choice): every 64 x 64 block of C gets four oracle
    # points, every tile-boundary row and column is compared whole (logical
    # rows of column-major C are canonical columns and vice versa, so both),
    # and no canary may survive anywhere in C.
    case = W.hgemm_colmajor(*W.HGEMM_SHAPES[2])
    say("hgemm 8k auto")
    rep = P.check_stratified(case, *P.run_gpu(h, case))
    say(rep)
    assert rep["tiles_256_reached"] == rep["tiles_256"] == 1024


# ---------------------------------------------------------------------------
# BF16 FFN projection and the skinny M sweep on the same W
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kernel", ["auto"] + P.KERNELS_16)
def test_ffn_bf16_sampled(h, kernel):
    case = W.ffn_bf16()
    say("ffn", kernel)
    out = supported(h, case, kernel, case.make())
    if out is None:
        pytest.skip("%s declines this problem" % kernel)
    rep = P.check_stratified(case, *out)
    say(rep)
    assert rep["tiles_256_reached"] == rep["tiles_256"]


@pytest.mark.parametrize("kernel", ["auto", "skinny", "skinny_sk"])
@pytest.mark.parametrize("M", W.SKINNY_M)
def test_skinny_bf16_full(h, M, kernel):
    case = W.ffn_bf16(M)
    say("skinny", M, kernel)
    P.check_tolerance(case, *P.run_gpu(h, case, kernel))


# Shapes that give the split-K skinny kernel 1, 3, 4, 16, 5 and 2 K ranges
# (one-round and multi-round reductions), a ragged last column block and
# ragged M, with beta != 0: integer data, so every split order must give the
# oracle's bits.  Each case runs twice in a row, which also checks that the
# arrival counters are back at zero.
SPLIT_SHAPES = [(16, 512, 32), (5, 1000, 96), (64, 12288, 4096), (3, 256, 4096), (33, 2056, 160),
                (20, 6144, 64)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_skinny_split_k_bit_exact(h, M, N, K):
    for dtype in ("bf16", "f16"):
        case = W.Case("split", M, N, K, dtype, kindA="int", kindB="int", kindC="int",
                      alpha=1.0, beta=-0.5, seeds=(M, N, K))
        inputs = case.make()
        for rep in range(2):
            say("skinny_sk", dtype, (M, N, K), rep)
            P.check_bit_exact(case, *P.run_gpu(h, case, "skinny_sk", inputs=inputs))


# FP32 with operands that are not 16-byte aligned and K that is not a multiple
# of the K slice: every load width of the unaligned kernel (A 1 or 4 floats,
# B 1, 2 or 4 floats), a K shorter than one slice, beta != 0.  Integer data:
# bit-exact.  (M, N, K, lda, ldb, ldc)
UNALIGNED_F32 = [(300, 514, 100, 101, 514, 514), (260, 257, 64, 64, 257, 257),
                 (520, 300, 77, 80, 302, 300), (256, 256, 31, 33, 258, 256),
                 (129, 96, 200, 203, 100, 97)]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", UNALIGNED_F32)
def test_f32_unaligned_bit_exact(h, M, N, K, lda, ldb, ldc):
    case = W.Case("f32u", M, N, K, "f32", lda=lda, ldb=ldb, ldc=ldc, alpha=1.0, beta=-0.5,
                  kindA="int", kindB="int", kindC="int", seeds=(M, N, K))
    inputs = case.make()
    for k in ("auto", "f32_fast_u", "f32_sk"):
        out = supported(h, case, k, inputs)
        if out is None:
            assert k != "auto"
            continue
        say("f32 unaligned", (M, N, K, lda, ldb, ldc), k)
        P.check_bit_exact(case, *out)


# The 16-byte FP32 kernel on the two mixed layout pairs (row-major A with
# column-major B: B' K-contiguous; column-major A with row-major B: A'
# M-contiguous after the transpose identity): edge tiles in both directions,
# beta != 0, integer data: bit-exact.  (M, N, K, layoutA, layoutB)
F32_MIXED = [(300, 516, 160, "row", "col"), (300, 516, 160, "col", "row"),
             (520, 260, 96, "row", "col"), (260, 520, 64, "col", "row")]


@pytest.mark.parametrize("M,N,K,la,lb", F32_MIXED)
def test_f32_fast_mixed_layouts_bit_exact(h, M, N, K, la, lb):
    case = W.Case("f32mix", M, N, K, "f32", layoutA=la, layoutB=lb, alpha=1.0, beta=-0.5,
                  kindA="int", kindB="int", kindC="int", seeds=(M, N, K + 7))
    inputs = case.make()
    for k in ("auto", "f32_fast"):
        say("f32 mixed", (M, N, K, la, lb), k)
        P.check_bit_exact(case, *P.run_gpu(h, case, k, inputs=inputs))


@pytest.mark.parametrize("la,lb", [("row", "col"), ("col", "row")])
def test_sgemm_4096_mixed_layouts_sampled(h, la, lb):
    case = W.Case("sgemm_4096_%s_%s" % (la, lb), 4096, 4096, 4096, "f32", layoutA=la,
                  layoutB=lb, seeds=(2001, 2002, 2003))
    say(case.name)
    out = P.run_gpu(h, case)
    P.check_tolerance(case, *out, rows=P.sample_rows(case.M, 128), cols=[0, 127, 128, 4095])


# Stream-K FP32 (one workgroup per CU, equal shares of the (tile, K slice)
# pairs): shares that cut tiles into two or three pieces, a single tile whose
# 157 slices are each a piece of their own, unaligned operands and K tails;
# integer data with beta != 0, so every piece order must give the oracle's
# bits.  (M, N, K, lda, ldb, ldc)
STREAM_K_F32 = [(1000, 6000, 700, 701, 6002, 6000), (512, 4096, 1024, 1024, 4096, 4096),
                (200, 200, 5000, 5001, 202, 200), (300, 514, 100, 101, 514, 514),
                (2048, 2304, 96, 96, 2304, 2304),
                # Short M: 32- and 64-row stream-K tiles.
                (1, 3000, 1000, 1000, 3000, 3000), (17, 1030, 700, 701, 1030, 1030),
                (40, 2048, 512, 512, 2048, 2048), (64, 12288, 4096, 4096, 12288, 12288),
                (100, 2600, 800, 801, 2600, 2600)]


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", STREAM_K_F32)
def test_f32_stream_k_bit_exact(h, M, N, K, lda, ldb, ldc):
    case = W.Case("f32sk", M, N, K, "f32", lda=lda, ldb=ldb, ldc=ldc, alpha=1.0, beta=-0.5,
                  kindA="int", kindB="int", kindC="int", seeds=(M + 1, N, K))
    say("f32 stream-K", (M, N, K, lda, ldb, ldc))
    P.check_bit_exact(case, *P.run_gpu(h, case, "f32_sk"))


@pytest.mark.parametrize("kernel", ["f32_fast_u", "f32_mfma", "f32_sk"])
def test_ragged_f32_forced(h, kernel):
    case = W.ragged_f32()
    say("ragged_f32", kernel)
    out = P.run_gpu(h, case, kernel)
    P.check_tolerance(case, *out, rows=P.sample_rows(case.M, 256, extra=8), cols=[0, 255, 256, 12289])


# ---------------------------------------------------------------------------
# Small and ragged shapes, integer data, every variant: bit-exact
# ---------------------------------------------------------------------------
SIZES = [1, 2, 3, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _sweep_shapes(n, seed):
    rng = np.random.default_rng(seed)
    shapes = [(1, 1, 1), (257, 255, 129), (64, 64, 64), (65, 63, 33), (16, 257, 31)]
    while len(shapes) < n:
        shapes.append(tuple(int(x) for x in rng.choice(SIZES, 3)))
    return shapes


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_small_shape_sweep_bit_exact(h, dtype):
    kernels = ["auto"] + (P.KERNELS_F32 if dtype == "f32" else P.KERNELS_16 + ["skinny", "skinny_sk"])
    ran = {k: 0 for k in kernels}
    for si, (M, N, K) in enumerate(_sweep_shapes(14, 7 + len(dtype))):
        for (la, lb), (alpha, beta) in itertools.product(
                itertools.product(["row", "col"], ["row", "col"]), [(1.0, 0.0), (1.0, -0.5)]):
            pad = si % 3
            case = W.Case("sweep", M, N, K, dtype, layoutA=la, layoutB=lb,
                          lda=(K if la == "row" else M) + pad, ldb=(N if lb == "row" else K) + pad,
                          ldc=(N if la == "row" else M) + pad, alpha=alpha, beta=beta,
                          kindA="int", kindB="int", kindC="int", seeds=(si, si + 100, si + 200))
            inputs = case.make()
            for k in kernels:
                out = supported(h, case, k, inputs)
                if out is None:
                    continue
                ran[k] += 1
                try:
                    P.check_bit_exact(case, *out)
                except AssertionError:
                    say("FAILED", dtype, (M, N, K), la, lb, alpha, beta, k)
                    raise
    say("ran", ran)
    assert ran["auto"] > 0 and ran["general"] > 0


# Mid-size shapes through the library's own choice of kernel, tile height and
# split of K (the time model's branches: 64-, 128- and 256-row tiles, split
# and unsplit, tile grids with an odd number of M-tiles), integer data, whole
# C bit-exact.  K = 1000 (not a multiple of 32: rows of 1000 elements are not
# 16-byte aligned) reaches the register-staged kernel's buffer loads.
MID_M = [65, 96, 130, 200, 256, 300, 384, 512, 640, 777, 1000, 1024, 1536]
MID_N = [64, 96, 192, 200, 384, 520, 1000, 1024, 1536, 2048]
MID_K = [64, 96, 256, 512, 640, 1000, 1024, 2048]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_mid_shape_auto_dispatch_bit_exact(h, dtype):
    rng = np.random.default_rng({"f32": 41, "f16": 42, "bf16": 43}[dtype])
    chosen = {}
    for si in range(8 if dtype == "f32" else 12):
        M, N, K = int(rng.choice(MID_M)), int(rng.choice(MID_N)), int(rng.choice(MID_K))
        la, lb = (["row", "col"][int(i)] for i in rng.integers(0, 2, 2))
        beta = [0.0, -0.5][si % 2]
        case = W.Case("mid", M, N, K, dtype, layoutA=la, layoutB=lb, alpha=1.0, beta=beta,
                      kindA="int", kindB="int", kindC="int", seeds=(900 + si, 950 + si, 990 + si))
        say("mid auto", dtype, (M, N, K), la, lb, beta)
        inputs = case.make()
        sel = mg.mgemm_select_variant(h, la, lb, M, N, K, 1.0, 256, case.lda, 256, case.ldb,
                                      beta, 256, case.ldc, dtype)
        chosen["%dx%dx%d %s/%s" % (M, N, K, la, lb)] = "%s/k%d" % sel
        P.check_bit_exact(case, *P.run_gpu(h, case, "auto", inputs=inputs))
    say("mid auto choices", dtype, chosen)


# K not a multiple of 32 on the direct-to-LDS kernel: the range that ends at
# the last whole slice stages one more, partial slice by ordinary loads with
# zeros past K.  Tails of 1, 7, 8, 9 and 31 elements (partial and whole
# 8-element runs of K-contiguous operands), every tile form, the four layout
# pairs (NN, B' K-contiguous, A' M-contiguous, and the transposed NN),
# unsplit and split; beta != 0; integer data, whole C bit-exact.
KTAIL_SHAPES = [(296, 200, 33), (264, 392, 103), (136, 520, 72), (520, 264, 255),
                (48, 776, 161), (1000, 600, 1001)]


def _up8(x):
    return (x + 7) // 8 * 8


@pytest.mark.parametrize("M,N,K", KTAIL_SHAPES)
def test_h_dma_k_tail_bit_exact(h, M, N, K):
    ran = {}
    for dtype in ("bf16", "f16"):
        for la, lb in itertools.product(["row", "col"], ["row", "col"]):
            # Leading dimensions rounded up to multiples of 8 (the kernel's
            # alignment rule), so K-contiguous rows end inside an 8-element run.
            case = W.Case("ktail", M, N, K, dtype, layoutA=la, layoutB=lb,
                          lda=_up8(K if la == "row" else M), ldb=_up8(N if lb == "row" else K),
                          alpha=1.0, beta=-0.5, kindA="int", kindB="int", kindC="int",
                          seeds=(M + 1, N + 2, K + 3))
            inputs = case.make()
            for kernel in ("h_dma_256x256", "h_dma_256x192", "h_dma_128x192", "h_dma_64x192"):
                for ks in (1, 2, 3):
                    try:
                        out = P.run_gpu(h, case, kernel, inputs=inputs, ksplit=ks)
                    except mg.MgemmError as e:
                        assert e.status == mg.MGEMM_ERR_UNSUPPORTED
                        continue
                    say("k tail", dtype, (M, N, K), la, lb, kernel, ks)
                    P.check_bit_exact(case, *out)
                    ran[(la, lb)] = ran.get((la, lb), 0) + 1
            say("k tail auto", dtype, (M, N, K), la, lb)
            P.check_bit_exact(case, *P.run_gpu(h, case, "auto", inputs=inputs))
    say("k tail forced runs per layout pair", ran)
    assert len(ran) == 4, ran


# 16-bit operands that are not 16-byte aligned run the register-staged kernel
# with buffer loads: every tile form when they are dword-aligned, the 128x128
# form when only 2-byte aligned.  Sizes are multiples of 8 and every leading
# dimension is padded by `pad` elements, so the alignment is fixed: pad 4 ->
# 8 bytes, 2 or 6 -> 4, 1 or 3 -> 2.  Every layout pair, edge tiles, ragged
# K, beta != 0; the library's own choice and every forced form; integer data,
# whole C bit-exact.
UNALIGNED_16 = [(264, 136, 104, 4), (520, 392, 200, 2), (136, 264, 328, 1), (1000, 600, 512, 4),
                (648, 1000, 1000, 1), (392, 520, 72, 6), (200, 72, 136, 3)]


def load_width(*lds):
    bits = 16
    for ld in lds:
        bits |= 2 * ld
    return bits & -bits


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K,pad", UNALIGNED_16)
def test_h_mfma_unaligned_bit_exact(h, dtype, M, N, K, pad):
    for si, (la, lb) in enumerate(itertools.product(["row", "col"], ["row", "col"])):
        lda = (K if la == "row" else M) + pad
        ldb = (N if lb == "row" else K) + pad
        ldc = (N if la == "row" else M) + pad
        case = W.Case("h_unaligned", M, N, K, dtype, layoutA=la, layoutB=lb, lda=lda, ldb=ldb,
                      ldc=ldc, alpha=1.0, beta=-0.5, kindA="int", kindB="int", kindC="int",
                      seeds=(M + si, N + si, K + pad))
        aw = load_width(lda, ldb)
        assert aw == {4: 8, 2: 4, 6: 4, 1: 2, 3: 2}[pad]
        sel = mg.mgemm_select_variant(h, la, lb, M, N, K, 1.0, 256, lda, 256, ldb, -0.5, 256, ldc,
                                      dtype)
        wide = ("h_mfma_256x256", "h_mfma_256x192")
        assert sel[0] == "h_mfma_128x128" or (aw >= 4 and sel[0] in wide), sel
        inputs = case.make()
        for kernel in ("auto", "h_mfma_128x128") + (wide if aw >= 4 else ()):
            say("h_mfma unaligned", dtype, (M, N, K), la, lb, "pad", pad, "width", aw, kernel)
            P.check_bit_exact(case, *P.run_gpu(h, case, kernel, inputs=inputs))
        if aw < 4:
            for kernel in wide:
                with pytest.raises(mg.MgemmError) as ei:
                    P.run_gpu(h, case, kernel, inputs=inputs)
                assert ei.value.status == mg.MGEMM_ERR_UNSUPPORTED


# Base addresses 2, 4 and 8 bytes past a 16-byte boundary (views into larger
# buffers), aligned leading dimensions: load widths 2, 4 and 8 bytes.
@pytest.mark.parametrize("offset", [1, 2, 4])
def test_h_mfma_unaligned_base_bit_exact(h, offset):
    M, N, K = 264, 200, 96
    case = W.Case("h_base", M, N, K, "bf16", alpha=1.0, beta=-0.5, kindA="int", kindB="int",
                  kindC="int", seeds=(7 + offset, 8, 9))
    A, B, C0 = case.make()
    Cin = W.c_initial(case, C0)

    def at_offset(t):
        big = torch.zeros(t.numel() + 16, dtype=t.dtype, device="cuda")
        view = big[offset:offset + t.numel()]
        view.copy_(t.reshape(-1).cuda())
        return big, view

    keep_a, dA = at_offset(A)
    keep_b, dB = at_offset(B)
    dC = Cin.cuda()
    assert dA.data_ptr() % 16 == 2 * offset % 16
    say("h_mfma unaligned base", offset)
    mg.mgemm_run(h, "row", "row", M, N, K, 1.0, dA, case.lda, dB, case.ldb, -0.5, dC, case.ldc,
                 "bf16")
    torch.cuda.synchronize()
    P.check_bit_exact(case, A, B, C0, Cin, dC.cpu())
    del keep_a, keep_b


# ---------------------------------------------------------------------------
# Fused SiLU epilogue (mgemm_run_ex): every variant, small shapes with integer
# data (exact GEMM), the pages' FFN projection Y = SiLU(XW) and a skinny case
# with random data, K = 0.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_silu_epilogue_every_variant(h, dtype):
    kernels = ["auto"] + (P.KERNELS_F32 if dtype == "f32" else P.KERNELS_16 + ["skinny", "skinny_sk"])
    ran = {k: 0 for k in kernels}
    for (M, N, K), (la, lb) in itertools.product([(257, 255, 129), (64, 520, 96), (300, 256, 64)],
                                                  [("row", "row"), ("col", "col")]):
        # Values small enough that SiLU is far from linear for most outputs.
        case = W.Case("silu", M, N, K, dtype, layoutA=la, layoutB=lb, alpha=0.25, beta=-0.5,
                      kindA="int", kindB="int", kindC="int", seeds=(M, N, K))
        inputs = case.make()
        for k in kernels:
            try:
                out = P.run_gpu(h, case, k, inputs=inputs, epilogue="silu")
            except mg.MgemmError as e:
                if e.status == mg.MGEMM_ERR_UNSUPPORTED:
                    continue
                raise
            ran[k] += 1
            say("silu", dtype, (M, N, K), la, lb, k)
            P.check_silu(case, *out, exact_gemm=True)
    say("ran", ran)
    assert ran["auto"] > 0 and ran["general"] > 0


def test_silu_ffn_bf16_sampled(h):
    case = W.ffn_bf16()
    say("silu ffn")
    out = P.run_gpu(h, case, "auto", epilogue="silu")
    P.check_silu(case, *out, rows=P.sample_rows(case.M, 256, extra=8))


@pytest.mark.parametrize("M", [1, 16])
def test_silu_skinny(h, M):
    case = W.ffn_bf16(M)
    say("silu skinny", M)
    P.check_silu(case, *P.run_gpu(h, case, "auto", epilogue="silu"))


def test_silu_k_zero_and_bad_epilogue(h):
    case = W.Case("silu_k0", 40, 48, 0, "bf16", alpha=1.0, beta=0.75, kindC="normal",
                  seeds=(1, 2, 3))
    P.check_silu(case, *P.run_gpu(h, case, "auto", epilogue="silu"), exact_gemm=True)
    A = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(mg.MgemmError) as ei:
        mg.mgemm_run_ex(h, "auto", "row", "row", 4, 4, 4, 1.0, A, 4, A, 4, 0.0, A, 4, "f32",
                        epilogue=7)
    assert ei.value.status == mg.MGEMM_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# Gated pair Z = SiLU(X W_g) * (X W_u) (mgemm_run_gated)
# ---------------------------------------------------------------------------
def _run_gated(h, case, inputs, ksplit=None):
    X, Wg, Wu = inputs
    Z = P.c_initial(case, None)
    dZ = Z.cuda()
    args = (case.M, case.N, case.K, X.cuda(), case.lda, Wg.cuda(), Wu.cuda(), case.ldb, dZ,
            case.ldc, case.dtype)
    if ksplit is None:
        mg.mgemm_run_gated(h, *args)
    else:
        mg.mgemm_run_gated_ex(h, ksplit, *args)
    torch.cuda.synchronize()
    return Z, dZ.cpu()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(300, 200, 64), (256, 96, 32), (130, 520, 96), (37, 104, 160),
                                   (300, 200, 72), (136, 520, 40)])
def test_gated_pair_integer(h, dtype, M, N, K):
    case = W.Case("gated", M, N, K, dtype, kindA="int", kindB="int", seeds=(M, N, K),
                  extra={"gated": True, "seed_u": K + 7})
    inputs = W.gated_inputs(case)
    Zin, Zout = _run_gated(h, case, inputs)
    say("gated", dtype, (M, N, K))
    P.check_gated(case, *inputs, Zout, exact_gemm=True)
    pad = P.padding_mask(case)
    assert np.array_equal(W.storage_view(Zout)[pad], W.storage_view(Zin)[pad])


def test_gated_pair_ffn_sampled(h):
    case = W.ffn_gated_bf16()
    inputs = W.gated_inputs(case)
    say("gated ffn")
    _, Zout = _run_gated(h, case, inputs)
    P.check_gated(case, *inputs, Zout, rows=P.sample_rows(case.M, 256, extra=8))


def test_gated_pair_unsupported_and_k_zero(h):
    A = torch.zeros(4096, dtype=torch.float32, device="cuda")
    with pytest.raises(mg.MgemmError) as ei:
        mg.mgemm_run_gated(h, 16, 64, 64, A, 64, A, A, 64, A, 64, "f32")
    assert ei.value.status == mg.MGEMM_ERR_UNSUPPORTED
    Z = torch.full((16 * 64,), 3.0, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    mg.mgemm_run_gated(h, 16, 64, 0, B, 1, B, B, 64, Z, 64, "bf16")
    torch.cuda.synchronize()
    assert torch.count_nonzero(Z).item() == 0


# ---------------------------------------------------------------------------
# Split K in the direct-to-LDS kernel (mgemm_run_variant / mgemm_run_gated_ex)
# ---------------------------------------------------------------------------
# Ragged M and N edges, K from 5 to 128 slices, beta != 0; requested splits
# above the slice count are clamped.  Integer data: every split must give the
# oracle's bits.
WORKSPACE_BYTES = 128 << 20      # FP32 partials a handle holds (mgemm_create)
SPLITK_SHAPES = [(300, 200, 640), (256, 192, 1024), (513, 776, 320), (37, 104, 160),
                 (1024, 1536, 4096)]


@pytest.mark.parametrize("M,N,K", SPLITK_SHAPES)
def test_h_dma_split_k_bit_exact(h, M, N, K):
    for dtype in ("bf16", "f16"):
        case = W.Case("hsplit", M, N, K, dtype, kindA="int", kindB="int", kindC="int",
                      alpha=1.0, beta=-0.5, seeds=(M, N, K))
        inputs = case.make()
        for kernel in ("h_dma_256x256", "h_dma_256x192", "h_dma_128x192", "h_dma_64x192"):
            bn = 256 if kernel.endswith("256") else 192
            bm = 128 if "_128x" in kernel else (64 if "_64x" in kernel else 256)
            tiles = -(-M // bm) * -(-N // bn)
            for ks in (1, 2, 3, 5, 8, 32):
                say("h_dma split", dtype, (M, N, K), kernel, ks)
                nk = K // 32
                ranges = -(-nk // -(-nk // min(ks, nk)))
                if tiles * ranges * 4 * bm * bn > WORKSPACE_BYTES:
                    # The FP32 partials (256 x bn per tile and range) would
                    # not fit the handle's workspace: refused, nothing runs.
                    with pytest.raises(mg.MgemmError) as ei:
                        P.run_gpu(h, case, kernel, inputs=inputs, ksplit=ks)
                    assert ei.value.status == mg.MGEMM_ERR_UNSUPPORTED
                    continue
                P.check_bit_exact(case, *P.run_gpu(h, case, kernel, inputs=inputs, ksplit=ks))


# The direct-to-LDS kernel with a K-contiguous B' (row-major A times a
# column-major B: weights stored out x in): ragged edges in both directions, N
# not a multiple of 8, both widths, unsplit and split, plain and SiLU; integer
# data, so every form must give the oracle's bits.
BKC_SHAPES = [(300, 200, 640), (256, 192, 1024), (513, 777, 320), (37, 100, 160)]


@pytest.mark.parametrize("M,N,K", BKC_SHAPES)
def test_h_dma_b_k_contiguous_bit_exact(h, M, N, K):
    for dtype in ("bf16", "f16"):
        case = W.Case("hbkc", M, N, K, dtype, layoutB="col", kindA="int", kindB="int",
                      kindC="int", alpha=1.0, beta=-0.5, seeds=(M, N, K + 1))
        inputs = case.make()
        for kernel in ("h_dma_256x256", "h_dma_256x192", "h_dma_128x192", "h_dma_64x192"):
            for ks in (1, 3):
                say("h_dma B K-contiguous", dtype, (M, N, K), kernel, ks)
                P.check_bit_exact(case, *P.run_gpu(h, case, kernel, inputs=inputs, ksplit=ks))
        case_s = W.Case("hbkc_silu", M, N, K, dtype, layoutB="col", kindA="int", kindB="int",
                        kindC="int", alpha=0.25, beta=-0.5, seeds=(M, N, K + 2))
        P.check_silu(case_s, *P.run_gpu(h, case_s, "h_dma_256x192", epilogue="silu"),
                     exact_gemm=True)


# Column-major A times row-major B: after the transpose identity A' is
# M-contiguous and staged like the 256-wide B slot (transposed reads).  M and N
# multiples of 8, ragged against the tiles.
AMC_SHAPES = [(304, 200, 640), (256, 192, 1024), (520, 776, 320), (40, 104, 160)]


@pytest.mark.parametrize("M,N,K", AMC_SHAPES)
def test_h_dma_a_m_contiguous_bit_exact(h, M, N, K):
    for dtype in ("bf16", "f16"):
        case = W.Case("hamc", M, N, K, dtype, layoutA="col", kindA="int", kindB="int",
                      kindC="int", alpha=1.0, beta=-0.5, seeds=(M, N, K + 3))
        inputs = case.make()
        for kernel in ("h_dma_256x256", "h_dma_256x192"):
            for ks in (1, 3):
                say("h_dma A M-contiguous", dtype, (M, N, K), kernel, ks)
                P.check_bit_exact(case, *P.run_gpu(h, case, kernel, inputs=inputs, ksplit=ks))
        case_s = W.Case("hamc_silu", M, N, K, dtype, layoutA="col", kindA="int", kindB="int",
                        kindC="int", alpha=0.25, beta=-0.5, seeds=(M, N, K + 4))
        P.check_silu(case_s, *P.run_gpu(h, case_s, "h_dma_256x256", epilogue="silu"),
                     exact_gemm=True)


# The skinny split kernel with K-contiguous weights (C = X W^T, W stored
# out x in): every M class, N not a multiple of 8, one to eight K ranges,
# beta != 0; integer data: bit-exact.
@pytest.mark.parametrize("M", [1, 5, 16, 33, 64])
def test_skinny_weights_out_by_in_bit_exact(h, M):
    for dtype in ("bf16", "f16"):
        case = W.Case("skinny_wt", M, 1000, 1024, dtype, layoutB="col", kindA="int", kindB="int",
                      kindC="int", alpha=1.0, beta=-0.5, seeds=(M, 1000, 1024))
        inputs = case.make()
        for ks in (1, 3, 8):
            say("skinny W^T", dtype, M, ks)
            P.check_bit_exact(case, *P.run_gpu(h, case, "skinny_sk", inputs=inputs, ksplit=ks))


@pytest.mark.parametrize("M", W.SKINNY_M)
def test_skinny_weights_out_by_in_ffn_sampled(h, M):
    case = W.Case("skinny_wt_ffn", M, 12288, 4096, "bf16", layoutB="col", kindA="normal",
                  kindB="normal", scaleB=0.02, seeds=(4001, 4002, 4003))
    sel = mg.mgemm_select_variant(h, "row", "col", M, 12288, 4096, 1.0, 256, 4096, 256, 4096,
                                  0.0, 256, 12288, "bf16")
    say("skinny W^T ffn", M, sel)
    assert sel[0] == ("skinny_sk" if M <= 16 else "h_dma_64x192")
    out = P.run_gpu(h, case)
    P.check_tolerance(case, *out, cols=[0, 255, 256, 12287])


def test_ffn_bf16_weights_out_by_in_sampled(h):
    # x W^T with W stored 12288 x 4096 (out x in): B column-major.
    case = W.Case("ffn_bf16_wt", 1024, 12288, 4096, "bf16", layoutB="col", kindA="normal",
                  kindB="normal", scaleB=0.02, seeds=(4001, 4002, 4003))
    sel = mg.mgemm_select_variant(h, "row", "col", 1024, 12288, 4096, 1.0, 256, 4096, 256, 4096,
                                  0.0, 256, 12288, "bf16")
    say("ffn W^T", sel)
    assert sel[0].startswith("h_dma")
    out = P.run_gpu(h, case)
    P.check_tolerance(case, *out, rows=P.sample_rows(case.M, 256), cols=[0, 191, 192, 12287])


def test_h_dma_split_k_silu(h):
    for dtype in ("bf16", "f16"):
        case = W.Case("hsplit_silu", 300, 520, 640, dtype, alpha=0.25, beta=-0.5, kindA="int",
                      kindB="int", kindC="int", seeds=(3, 4, 5))
        inputs = case.make()
        for kernel, ks in (("h_dma_256x256", 4), ("h_dma_256x192", 7)):
            say("h_dma split silu", dtype, kernel, ks)
            out = P.run_gpu(h, case, kernel, inputs=inputs, epilogue="silu", ksplit=ks)
            P.check_silu(case, *out, exact_gemm=True)


def test_ffn_share_split_auto(h):
    case = W.ffn_share_bf16()
    name, ks = mg.mgemm_select_variant(h, case.layoutA, case.layoutB, case.M, case.N, case.K,
                                       case.alpha, 256, case.lda, 256, case.ldb, case.beta, 256,
                                       case.ldc, case.dtype)
    say("ffn share auto:", name, ks)
    assert name.startswith("h_dma") and ks > 1
    out = P.run_gpu(h, case)
    P.check_tolerance(case, *out, rows=P.sample_rows(case.M, 192, extra=8))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(300, 200, 160), (130, 520, 96), (37, 104, 160), (300, 200, 104)])
def test_gated_pair_split_k_integer(h, dtype, M, N, K):
    # K stays small: G and U grow with K and their product must stay inside
    # the FP16 range for most outputs.
    case = W.Case("gated_split", M, N, K, dtype, kindA="int", kindB="int", seeds=(M, N, K),
                  extra={"gated": True, "seed_u": K + 9})
    inputs = W.gated_inputs(case)
    for ks in (2, 3, 5, 32):
        say("gated split", dtype, (M, N, K), ks)
        Zin, Zout = _run_gated(h, case, inputs, ksplit=ks)
        P.check_gated(case, *inputs, Zout, exact_gemm=True)
        pad = P.padding_mask(case)
        assert np.array_equal(W.storage_view(Zout)[pad], W.storage_view(Zin)[pad])


def test_gated_share_sampled(h):
    case = W.ffn_gated_share_bf16()
    inputs = W.gated_inputs(case)
    say("gated share auto")
    _, Zout = _run_gated(h, case, inputs)
    P.check_gated(case, *inputs, Zout, rows=P.sample_rows(case.M, 192, extra=8))


def test_skinny_forced_splits_bit_exact(h):
    for M, N, K in [(64, 12288, 4096), (5, 1000, 96)]:
        case = W.Case("sk_forced", M, N, K, "bf16", kindA="int", kindB="int", kindC="int",
                      alpha=1.0, beta=-0.5, seeds=(M, N, K))
        inputs = case.make()
        for ks in (1, 2, 7, 32):
            say("skinny_sk forced", (M, N, K), ks)
            P.check_bit_exact(case, *P.run_gpu(h, case, "skinny_sk", inputs=inputs, ksplit=ks))


def test_split_k_argument_errors(h):
    A = torch.zeros(4096, dtype=torch.bfloat16, device="cuda")
    args = ("row", "row", 64, 64, 64, 1.0, A, 64, A, 64, 0.0, A, 64, "bf16")
    for kernel, ks, want in (("h_dma_256x256", 33, mg.MGEMM_ERR_INVALID_ARG),
                             ("h_dma_256x256", -1, mg.MGEMM_ERR_INVALID_ARG),
                             ("auto", 2, mg.MGEMM_ERR_INVALID_ARG),
                             ("h_mfma_128x128", 2, mg.MGEMM_ERR_UNSUPPORTED)):
        with pytest.raises(mg.MgemmError) as ei:
            mg.mgemm_run_variant(h, kernel, ks, *args)
        assert ei.value.status == want, (kernel, ks)
    # Partials larger than the workspace: refused before anything is launched.
    with pytest.raises(mg.MgemmError) as ei:
        mg.mgemm_run_variant(h, "h_dma_256x256", 32, "row", "row", 8192, 8192, 16384, 1.0, A,
                             16384, A, 8192, 0.0, A, 8192, "bf16")
    assert ei.value.status == mg.MGEMM_ERR_UNSUPPORTED
    with pytest.raises(mg.MgemmError) as ei:
        mg.mgemm_run_gated_ex(h, 40, 64, 64, 64, A, 64, A, A, 64, A, 64, "bf16")
    assert ei.value.status == mg.MGEMM_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# Contract details
# ---------------------------------------------------------------------------
def test_beta_zero_ignores_nan_c(h):
    for dtype in ("f32", "f16", "bf16"):
        case = W.Case("nanC", 96, 80, 40, dtype, kindA="int", kindB="int", seeds=(1, 2, 3))
        A, B, _ = case.make()
        dA, dB = A.cuda(), B.cuda()
        dC = torch.full((case.c_numel(),), float("nan"), dtype=W.TORCH_DTYPES[dtype], device="cuda")
        mg.mgemm_run(h, "row", "row", 96, 80, 40, 1.0, dA, 40, dB, 80, 0.0, dC, 80, dtype)
        torch.cuda.synchronize()
        assert torch.isfinite(dC.float()).all()


def test_degenerate_shapes(h):
    dtype = "f32"
    C0 = torch.arange(12, dtype=torch.float32, device="cuda").reshape(3, 4).contiguous()
    A = torch.ones(3, 5, device="cuda")
    B = torch.ones(5, 4, device="cuda")
    C = C0.clone()
    mg.mgemm_run(h, "row", "row", 0, 4, 5, 1.0, A, 5, B, 4, 2.0, C, 4, dtype)   # M = 0: no-op
    mg.mgemm_run(h, "row", "row", 3, 0, 5, 1.0, A, 5, B, 4, 2.0, C, 4, dtype)   # N = 0: no-op
    torch.cuda.synchronize()
    assert torch.equal(C, C0)
    mg.mgemm_run(h, "row", "row", 3, 4, 0, 1.0, A, 1, B, 4, 2.0, C, 4, dtype)   # K = 0: C = 2C
    torch.cuda.synchronize()
    assert torch.equal(C, 2 * C0)
    C = C0.clone()
    nanA = torch.full((3, 5), float("nan"), device="cuda")
    mg.mgemm_run(h, "row", "row", 3, 4, 5, 0.0, nanA, 5, B, 4, -1.0, C, 4, dtype)  # alpha = 0
    torch.cuda.synchronize()
    assert torch.equal(C, -C0)
    C = C0.clone()
    mg.mgemm_run(h, "row", "row", 3, 4, 0, 1.0, None, 1, None, 4, 0.0, C, 4, dtype)  # K=0, beta=0
    torch.cuda.synchronize()
    assert torch.equal(C, torch.zeros_like(C0))


def test_invalid_arguments_leave_c_untouched(h):
    C0 = torch.arange(16, dtype=torch.float32, device="cuda")
    A = torch.ones(16, device="cuda")
    C = C0.clone()
    bad = [
        dict(M=-1), dict(lda=3), dict(ldb=3), dict(ldc=3), dict(layoutA=7), dict(dtype=9),
        dict(C=None), dict(A=None),
    ]
    for b in bad:
        kw = dict(layoutA="row", layoutB="row", M=4, N=4, K=4, alpha=1.0, A=A, lda=4, B=A, ldb=4,
                  beta=0.0, C=C, ldc=4, dtype="f32")
        kw.update(b)
        with pytest.raises(mg.MgemmError) as ei:
            mg.mgemm_run(h, kw["layoutA"], kw["layoutB"], kw["M"], kw["N"], kw["K"], kw["alpha"],
                         kw["A"], kw["lda"], kw["B"], kw["ldb"], kw["beta"], kw["C"], kw["ldc"],
                         kw["dtype"])
        assert ei.value.status == mg.MGEMM_ERR_INVALID_ARG, b
    with pytest.raises(mg.MgemmError) as ei:
        mg.mgemm_run_kernel(h, "f32_mfma", "row", "row", 4, 4, 4, 1.0, A, 4, A, 4, 0.0, C, 4, "f16")
    assert ei.value.status == mg.MGEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(C, C0)


def test_deterministic_run_to_run(h):
    # Stream-K: the pieces of a tile are summed in K order whoever arrives last.
    case = W.Case("det_sk", 1000, 3000, 2000, "f32", lda=2001, seeds=(5, 6, 7))
    inputs = case.make()
    outs = [W.storage_view(P.run_gpu(h, case, "f32_sk", inputs=inputs)[4]) for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), case.name
    for case in (W.Case("det32", 1000, 1200, 777, "f32", seeds=(5, 6, 7)),
                 W.Case("det16", 1024, 1280, 1000, "bf16", kindA="normal", kindB="normal",
                        seeds=(5, 6, 7)),
                 W.Case("det_skinny", 16, 12288, 4096, "bf16", kindA="normal", kindB="normal",
                        seeds=(5, 6, 7))):
        inputs = case.make()
        outs = [W.storage_view(P.run_gpu(h, case, inputs=inputs)[4]) for _ in range(3)]
        for o in outs[1:]:
            assert np.array_equal(o, outs[0]), case.name
    # A split of K adds its ranges in a fixed order: the same bits every run.
    case = W.Case("det_split", 1024, 1280, 4096, "bf16", kindA="normal", kindB="normal",
                  seeds=(5, 6, 7))
    inputs = case.make()
    outs = [W.storage_view(P.run_gpu(h, case, "h_dma_256x192", inputs=inputs, ksplit=6)[4])
            for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), case.name


def test_non_default_stream(h):
    case = W.Case("stream", 300, 200, 100, "f16", kindA="int", kindB="int", seeds=(8, 9, 10))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = P.run_gpu(h, case, stream=s)
    P.check_bit_exact(case, *out)


def test_two_handles_on_two_streams(h):
    # Each handle owns its split-K workspace and arrival counters, so split
    # calls of two handles on two streams may run at the same time: the
    # two-launch split and the skinny last-arrival split, interleaved without
    # synchronisation, both give the oracle's bits.
    h2 = mg.mgemm_create()
    try:
        jobs = [(h, W.Case("two_share", 1024, 1536, 4096, "bf16", kindA="int", kindB="int",
                           kindC="int", beta=-0.5, seeds=(81, 82, 83)), "h_dma_128x192", 4),
                (h2, W.Case("two_skinny", 16, 6144, 4096, "bf16", kindA="int", kindB="int",
                            kindC="int", beta=-0.5, seeds=(84, 85, 86)), "skinny_sk", 4)]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        state = []
        for hh, case, kernel, ks in jobs:
            A, B, C0 = case.make()
            Cin = P.c_initial(case, C0)
            state.append((A, B, C0, Cin, A.cuda(), B.cuda(), C0.cuda()))
        torch.cuda.synchronize()
        outs = [None, None]
        for rep in range(4):
            for j, ((hh, case, kernel, ks), s) in enumerate(zip(jobs, streams)):
                A, B, C0, Cin, dA, dB, dC0 = state[j]
                with torch.cuda.stream(s):
                    dC = Cin.cuda()          # fresh C each time: beta reads it
                    mg.mgemm_run_variant(hh, kernel, ks, case.layoutA, case.layoutB, case.M,
                                         case.N, case.K, case.alpha, dA, case.lda, dB, case.ldb,
                                         case.beta, dC, case.ldc, case.dtype, stream=s)
                    outs[j] = dC
        torch.cuda.synchronize()
        for j, (hh, case, kernel, ks) in enumerate(jobs):
            A, B, C0, Cin = state[j][:4]
            say("two handles", case.name, kernel, ks)
            P.check_bit_exact(case, A, B, C0, Cin, outs[j].cpu())
    finally:
        torch.cuda.synchronize()
        mg.mgemm_destroy(h2)


def test_unaligned_16bit_operands(h):
    # Operands one element past a 16-byte boundary, odd leading dimensions.
    M, N, K = 130, 70, 90
    case = W.Case("unaligned", M, N, K, "bf16", lda=K + 1, ldb=N + 3, ldc=N + 1,
                  kindA="int", kindB="int", seeds=(11, 12, 13))
    A, B, _ = case.make()
    dA = torch.empty(A.numel() + 1, dtype=A.dtype, device="cuda")
    dB = torch.empty(B.numel() + 1, dtype=B.dtype, device="cuda")
    dA[1:] = A.cuda()
    dB[1:] = B.cuda()
    Cin = P.c_initial(case, None)
    dC = torch.empty(Cin.numel() + 1, dtype=Cin.dtype, device="cuda")
    dC[1:] = Cin.cuda()
    mg.mgemm_run(h, "row", "row", M, N, K, 1.0, dA.data_ptr() + 2, case.lda, dB.data_ptr() + 2,
                 case.ldb, 0.0, dC.data_ptr() + 2, case.ldc, "bf16")
    torch.cuda.synchronize()
    P.check_bit_exact(case, A, B, None, Cin, dC[1:].cpu())


def test_dispatch_choices(h):
    def sel(case):
        return mg.mgemm_select_kernel(h, case.layoutA, case.layoutB, case.M, case.N, case.K,
                                      case.alpha, 256, case.lda, 256, case.ldb, case.beta, 256,
                                      case.ldc, case.dtype)
    assert sel(W.sgemm_4096()) == "f32_fast"
    for la, lb in (("row", "col"), ("col", "row")):
        assert sel(W.Case("mixed", 4096, 4096, 4096, "f32", layoutA=la, layoutB=lb)) == "f32_fast"
    assert sel(W.ragged_f32()) == "f32_sk"
    assert sel(W.hgemm_colmajor(8192, 8192, 16384)) == "h_dma_256x256"
    assert sel(W.ffn_bf16()) == "h_dma_256x192"
    assert all(sel(W.ffn_bf16(m)) == ("skinny_sk" if m <= 16 else "h_dma_64x192")
               for m in W.SKINNY_M)
    say("dispatch:", {c.name: sel(c) for c in [W.hgemm_colmajor(*s) for s in W.HGEMM_SHAPES]
                      + [W.ffn_bf16()] + [W.ffn_bf16(m) for m in W.SKINNY_M]})


def test_skinny_dispatch_rules(h):
    # The model's choices for M <= 64: whole-K for K <= 2048; the split skinny
    # kernel only for M <= 16 on a B wide enough for its ranges to fill the
    # CUs; 64-row tiles otherwise; and no K split whose ranges start a multiple
    # of 2 MiB apart in a B with a power-of-two row pitch (8 KiB here).  Each
    # choice is then run through mgemm_run and compared bit for bit with the
    # oracle on integer data.
    def sel(M, N, K):
        return mg.mgemm_select_variant(h, "row", "row", M, N, K, 1.0, 256, K, 256, N, 0.0, 256, N,
                                       "bf16")
    assert sel(16, 1024, 2048) == ("skinny", 1)
    assert sel(64, 12288, 2048) == ("skinny", 1)
    assert sel(64, 1024, 2048)[0] == "h_dma_64x192"
    assert sel(1, 12288, 4096)[0] == "skinny_sk"
    assert sel(32, 1536, 4096)[0] == "h_dma_64x192"
    for M, N, K in ((32, 4096, 4096), (32, 4096, 8192), (1, 4096, 12288), (64, 4096, 4096)):
        name, ks = sel(M, N, K)
        nks = -(-(K // 32) // ks)
        say("skinny rule", (M, N, K), name, ks)
        assert ks > 1 and (nks * 32 * N * 2) % (2 << 20) != 0, (M, N, K, name, ks)
    for M, N, K in ((32, 1536, 4096), (32, 4096, 8192), (1, 4096, 12288), (16, 1024, 2048),
                    (64, 1024, 2048)):
        case = W.Case("skinny_rule", M, N, K, "bf16", kindA="int", kindB="int", seeds=(M, N, K))
        say("skinny rule parity", (M, N, K), sel(M, N, K))
        P.check_bit_exact(case, *P.run_gpu(h, case))
