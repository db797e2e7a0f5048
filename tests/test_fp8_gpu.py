"""FP8 E4M3 path on the GPU against the FP8 oracle (oracle/fp8.py), through
the C ABI: per-row quantisation bit-exact (codes and scales), the FP8 GEMM
bit-exact on integer codes with power-of-two scales and within the FP32
accumulation tolerance on the FFN-sized problem."""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_mgemm_amd as mg
import oracle
import workloads as W
from oracle import fp8
from tests import parity as P

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


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


def quantize_gpu(h, x: torch.Tensor, ldq=None):
    """x: CPU tensor (M x K, any float type).  Returns (codes M x ldq uint8, scales)."""
    M, K = x.shape
    ldq = ldq or K
    dx = x.contiguous().cuda()
    q = torch.full((M * ldq,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    dt = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[x.dtype]
    mg.mgemm_quantize_fp8(h, M, K, dx, K, dt, q, ldq, s)
    torch.cuda.synchronize()
    return q.cpu().numpy().reshape(M, ldq), s.cpu().numpy()


def special_rows(K):
    rng = np.random.default_rng(K)
    rows = []
    r = np.zeros(K); r[::3] = -0.0; rows.append(r)                          # zeros, signed
    r = rng.standard_normal(K); r[K // 2] = np.nan; rows.append(r)           # NaN
    r = rng.standard_normal(K); r[1] = -np.inf; rows.append(r)               # inf
    # Scale 1 (amax 448): exact halfway values between E4M3 neighbours.
    v = fp8.e4m3_values()[:0x7F]
    mids = (v[:-1] + v[1:]) / 2
    r = np.resize(np.concatenate([mids, -mids]), K); r[0] = 448.0; rows.append(r)
    # Huge dynamic range: most elements land in the E4M3 subnormals.
    r = rng.standard_normal(K) * np.exp(rng.uniform(-12, 0, K)); rows.append(r)
    return np.array(rows)


@pytest.mark.parametrize("xtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,K,pad", [(37, 300, 8), (64, 4096, 8), (5, 1, 3), (9, 136, 8),
                                     (16, 1000, 3)])
def test_quantize_bit_exact(h, xtype, M, K, pad):
    # pad 8 with K % 8 == 0 takes the 16-byte load / 8-byte store path.
    rng = np.random.default_rng(M * 1000 + K)
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-15, 15, (M, 1)))
    if K >= 8:
        x = np.concatenate([x, special_rows(K)])
    xt = torch.from_numpy(x).to(TORCH[xtype])
    xv = xt.float().double().numpy()                   # the stored values, exactly
    say("quantize", xtype, x.shape)
    q, s = quantize_gpu(h, xt, ldq=K + pad)
    qo, so = fp8.quantize_rows(xv)
    assert np.array_equal(q[:, :K], qo), np.argwhere(q[:, :K] != qo)[:5]
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)) or \
        np.array_equal(s, so, equal_nan=True)
    assert np.all(q[:, K:] == 0xA5)                     # row padding untouched


@pytest.mark.parametrize("xtype", ["f32", "bf16"])
def test_quantize_dense_grid(h, xtype):
    # Rows whose largest magnitude is 448 have the factor 1, so every element
    # is encoded as itself: a dense grid of [-448, 448] (ties between
    # neighbours, subnormal codes, binade edges) against the oracle's encoder,
    # through both quantisation kernels (register rows and long rows).
    v = fp8.e4m3_values()[:0x7F]
    grid = np.concatenate([np.linspace(-448, 448, 8191), (v[:-1] + v[1:]) / 2, -(v[:-1] + v[1:]) / 2,
                           np.ldexp(np.arange(0, 600), -14), -np.ldexp(np.arange(0, 600), -14),
                           [448.0, -0.0, 0.0]])
    for K in (4096, 20000):
        row = np.resize(grid, K)
        row[0] = 448.0
        xt = torch.from_numpy(row[None, :]).to(TORCH[xtype])
        q, s = quantize_gpu(h, xt, ldq=K)
        qo, so = fp8.quantize_rows(xt.float().double().numpy())
        bad = np.argwhere(q != qo)
        assert bad.size == 0, (K, [(xt[0, j].item(), q[0, j], qo[0, j]) for _, j in bad[:8]])
        assert s[0] == so[0] == 1.0


def int_codes(rng, rows, K):
    ints = rng.integers(-16, 17, (rows, K)).astype(np.float64)
    return fp8.e4m3_encode(ints), ints


# K = 100, 208 and 1000 end with a partial 64-code slice (36, 16 and 40 codes,
# the first and last inside a 16-code run), which the MFMA kernels stage by
# ordinary loads; the leading dimensions are multiples of 16 (their rule).
@pytest.mark.parametrize("M,N,K", [(300, 200, 640), (256, 256, 64), (513, 776, 320),
                                   (37, 104, 100), (1, 1, 64), (130, 520, 208),
                                   (513, 200, 1000)])
@pytest.mark.parametrize("ctype", ["f32", "f16", "bf16"])
def test_fp8_gemm_integer_bit_exact(h, M, N, K, ctype):
    rng = np.random.default_rng(M + N + K)
    k16 = (K + 15) // 16 * 16
    lda, ldb, ldc = k16 + 16, k16 + 32, N + 3
    qa, ia = int_codes(rng, M, K)
    qb, ib = int_codes(rng, N, K)
    sa = (2.0 ** rng.integers(-4, 3, M)).astype(np.float32)
    sb = (2.0 ** rng.integers(-4, 3, N)).astype(np.float32)
    pa = np.zeros((M, lda), np.uint8); pa[:, :K] = qa
    pb = np.zeros((N, ldb), np.uint8); pb[:, :K] = qb
    c0 = rng.integers(-8, 9, (M, ldc)).astype(np.float64)
    c0_bits = oracle.encode(ctype, c0)
    alpha, beta = 0.5, -2.0
    exact = fp8.fp8_gemm(M, N, K, alpha, pa.ravel(), lda, sa, pb.ravel(), ldb, sb, beta, c0[:, :N])
    want = oracle.encode(ctype, exact)
    ran = 0
    for kernel, ks in (("auto", 0), ("f8_mfma_256x256", 1), ("f8_mfma_256x256", 3),
                       ("f8_mfma_256x192", 0), ("f8_mfma_256x192", 32), ("f8_mfma_128x192", 1),
                       ("f8_mfma_128x192", 5), ("f8_general", 1)):
        dA = torch.from_numpy(pa.ravel()).cuda()
        dB = torch.from_numpy(pb.ravel()).cuda()
        dsa, dsb = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda()
        host_view = {"f32": np.float32, "f16": np.float16, "bf16": np.int16}[ctype]
        dC = torch.from_numpy(c0_bits.view(host_view).copy().ravel()).cuda()
        try:
            mg.mgemm_run_fp8(h, kernel, M, N, K, alpha, dA, lda, dsa, dB, ldb, dsb, beta, dC, ldc,
                             ctype, ksplit=ks)
        except mg.MgemmError as e:
            raise AssertionError("%s declined %s: %s" % (kernel, (M, N, K), e))
        torch.cuda.synchronize()
        got = dC.cpu().numpy().view(c0_bits.dtype).reshape(M, ldc)
        say("fp8 gemm", (M, N, K), ctype, kernel, ks)
        bad = np.argwhere(got[:, :N] != want)
        assert bad.size == 0, (kernel, bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])
        assert np.array_equal(got[:, N:], c0_bits[:, N:])   # ldc padding untouched
        ran += 1
    assert ran == 8


def fp8_inputs(case):
    """(X bf16/f16 CPU tensor M x K, W CPU tensor N x K) of an FP8 workload."""
    A, B, _ = case.make()
    X = A.view(case.M, case.lda)[:, : case.K]
    Wt = B.view(case.N, case.ldb)[:, : case.K]
    return X, Wt


def check_fp8_tolerance(case, qa, sa, qb, sb, got, rows):
    exact = fp8.fp8_gemm(len(rows), case.N, case.K, 1.0, qa[rows].ravel(), case.K, sa[rows],
                         qb.ravel(), case.K, sb)
    tol = P.tol_f32_rel(case.K) * float(np.max(np.abs(exact)))
    half_ulp = P._ulp(case.dtype, oracle.round_to(case.dtype, exact)) / 2
    err = np.abs(got - exact)
    bad = np.argwhere(~(err <= tol + half_ulp))
    assert bad.size == 0, (case.name, bad[:5], got[tuple(bad[0])], exact[tuple(bad[0])])
    return float(np.max(err))


@pytest.mark.parametrize("case", [W.fp8_ffn_bf16(), W.fp8_quant_example()], ids=lambda c: c.name)
def test_fp8_workload_sampled(h, case):
    X, Wt = fp8_inputs(case)
    say("fp8 workload", case.name)
    qa, sa = quantize_gpu(h, X)
    qb, sb = quantize_gpu(h, Wt)
    # The codes of this very run are the oracle's (checked row by row here on a
    # sample, and bit-exactly in test_quantize_bit_exact).
    rows = P.sample_rows(case.M, 256, extra=8)
    qo, so = fp8.quantize_rows(X.float().double().numpy()[rows])
    assert np.array_equal(qa[rows], qo) and np.array_equal(sa[rows], so)
    dC = torch.empty(case.M * case.N, dtype=TORCH[case.dtype], device="cuda")
    mg.mgemm_run_fp8(h, "auto", case.M, case.N, case.K, 1.0, torch.from_numpy(qa.ravel()).cuda(),
                     case.K, torch.from_numpy(sa).cuda(), torch.from_numpy(qb.ravel()).cuda(),
                     case.K, torch.from_numpy(sb).cuda(), 0.0, dC, case.N, case.dtype)
    torch.cuda.synchronize()
    got = dC.float().cpu().numpy().astype(np.float64).reshape(case.M, case.N)[rows]
    err = check_fp8_tolerance(case, qa, sa, qb, sb, got, rows)
    say("max err", err)


def test_fp8_deterministic_and_errors(h):
    case = W.fp8_ffn_bf16()
    M, N, K = 512, 1024, 4096
    rng = np.random.default_rng(1)
    qa = torch.from_numpy(rng.integers(0, 0x7E, M * K, dtype=np.uint8)).cuda()
    qb = torch.from_numpy(rng.integers(0x80, 0xFE, N * K, dtype=np.uint8)).cuda()
    sa = torch.rand(M, device="cuda")
    sb = torch.rand(N, device="cuda")
    outs = []
    for _ in range(3):
        C = torch.empty(M * N, dtype=torch.bfloat16, device="cuda")
        mg.mgemm_run_fp8(h, "auto", M, N, K, 1.0, qa, K, sa, qb, K, sb, 0.0, C, N, "bf16")
        torch.cuda.synchronize()
        outs.append(C.view(torch.int16).cpu())
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    for kernel, want in (("h_dma_256x256", mg.MGEMM_ERR_INVALID_ARG), ("f8_mfma_256x256", None)):
        args = (M, N, K, 1.0, qa, K, sa, qb, K, sb, 0.0, C, N, "bf16")
        if want is None:
            mg.mgemm_run_fp8(h, kernel, *args)
            continue
        with pytest.raises(mg.MgemmError) as ei:
            mg.mgemm_run_fp8(h, kernel, *args)
        assert ei.value.status == want
    for kernel, ks, want in (("auto", 2, mg.MGEMM_ERR_INVALID_ARG),
                             ("f8_mfma_256x256", 33, mg.MGEMM_ERR_INVALID_ARG),
                             ("f8_general", 2, mg.MGEMM_ERR_UNSUPPORTED)):
        with pytest.raises(mg.MgemmError) as ei:
            mg.mgemm_run_fp8(h, kernel, M, N, K, 1.0, qa, K, sa, qb, K, sb, 0.0, C, N, "bf16",
                             ksplit=ks)
        assert ei.value.status == want, (kernel, ks)
    # A split forced on the 8k problem needs more partials than the workspace holds.
    with pytest.raises(mg.MgemmError) as ei:
        mg.mgemm_run_fp8(h, "f8_mfma_256x256", 8192, 8192, 16384, 1.0, qa, 16384, sa, qb, 16384,
                         sb, 0.0, C, 8192, "bf16", ksplit=8)
    assert ei.value.status == mg.MGEMM_ERR_UNSUPPORTED
    with pytest.raises(mg.MgemmError) as ei:       # lda below K
        mg.mgemm_run_fp8(h, "auto", M, N, K, 1.0, qa, K - 1, sa, qb, K, sb, 0.0, C, N, "bf16")
    assert ei.value.status == mg.MGEMM_ERR_INVALID_ARG
    with pytest.raises(mg.MgemmError) as ei:       # unaligned codes for the MFMA kernel
        mg.mgemm_run_fp8(h, "f8_mfma_256x256", M, N, K, 1.0, qa.data_ptr() + 1, K, sa, qb, K, sb,
                         0.0, C, N, "bf16")
    assert ei.value.status == mg.MGEMM_ERR_UNSUPPORTED
    with pytest.raises(mg.MgemmError) as ei:
        mg.mgemm_quantize_fp8(h, 4, 8, qa, 7, "bf16", qb, 8, sa)
    assert ei.value.status == mg.MGEMM_ERR_INVALID_ARG
    # K == 0: C = beta * C.
    C2 = torch.full((4 * 4,), 2.0, dtype=torch.float32, device="cuda")
    mg.mgemm_run_fp8(h, "auto", 4, 4, 0, 1.0, None, 1, None, None, 1, None, 0.5, C2, 4, "f32")
    torch.cuda.synchronize()
    assert torch.all(C2 == 1.0)
