"""64-bit offsets: operands of more than 2^31 elements.

One MI355X holds 288 GB, so a single operand can exceed 2^31 elements (here
4.9-9.8 GB each); every offset the kernels form (row times leading dimension)
must then be 64-bit.  The operands come from the counter-hashed generator
(values -1, 0, 1, filled on the device); the oracle recomputes a grid of
rows x columns of C from the host's copy of just those rows and columns, and
with integer data the GPU must give its bits.  Rows past the 2^31-element
offset and the last rows and columns are always in the grid, and no output
may keep the canary written before the call.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_mgemm_amd as mg
import oracle
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


# (name, dtype, layout of A and B (C follows A), M, N, K)
CASES = [
    ("f16_rows_A", "f16", "row", 300000, 256, 8192),      # A: 2.46e9 elements
    ("f16_col_B", "f16", "col", 256, 300000, 8192),       # B stored N x K: 2.46e9
    ("bf16_skinny_W", "bf16", "row", 16, 40960, 65536),    # W: 2.68e9
    ("f32_rows_A", "f32", "row", 600000, 128, 4096),      # A: 2.46e9 (9.8 GB)
]


def _pick(n, big_from, rng, extra=12):
    """Edges, tile boundaries, the first index past a 2^31-element offset and
    random indices below n."""
    base = {0, 1, n - 1, n - 2, min(n - 1, 64), min(n - 1, 128), min(n - 1, 255), min(n - 1, 256)}
    if big_from is not None and big_from < n:
        base |= {big_from - 1, big_from, min(n - 1, big_from + 1)}
    base |= set(int(x) for x in rng.integers(0, n, extra))
    return np.array(sorted(i for i in base if 0 <= i < n), np.int64)


@pytest.mark.parametrize("name,dtype,lay,M,N,K", CASES, ids=[c[0] for c in CASES])
def test_operands_beyond_2_31_elements(h, name, dtype, lay, M, N, K):
    dev = "cuda"
    sa, sb = 9001, 9002
    if lay == "row":
        A = W.hashed_operand(M, K, sa, dtype, dev)        # A[m, k] at m*K + k
        B = W.hashed_operand(K, N, sb, dtype, dev)        # B[k, n] at k*N + n
        lda, ldb, ldc = K, N, N
    else:
        A = W.hashed_operand(K, M, sa, dtype, dev)        # A[m, k] at k*M + m
        B = W.hashed_operand(N, K, sb, dtype, dev)        # B[k, n] at n*K + k
        lda, ldb, ldc = M, K, M
    ibits = torch.int32 if dtype == "f32" else torch.int16
    canary = W.CANARY[dtype]              # a quiet NaN, positive as a signed integer
    C = torch.full((M * N,), canary, dtype=ibits, device=dev).view(W.TORCH_DTYPES[dtype])
    sel = mg.mgemm_select_variant(h, lay, lay, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc, dtype)
    say(name, "M N K", M, N, K, "variant", sel)
    mg.mgemm_run(h, lay, lay, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc, dtype)
    torch.cuda.synchronize()
    left = int((C.view(ibits) == canary).sum())
    assert left == 0, "%d outputs never written" % left

    rng = np.random.default_rng(M + N + K)
    # The first row (or column) whose operand offset passes 2^31 elements.
    big_m = -(-(2 ** 31) // K) if lay == "row" else None
    big_n = -(-(2 ** 31) // K) if lay == "col" else None
    if name.startswith("bf16_skinny"):
        big_n = None
    rows, cols = _pick(M, big_m, rng), _pick(N, big_n, rng)
    ks = np.arange(K)
    if lay == "row":
        a_sub = W.hashed_values(rows, ks, K, sa)                  # rows x K
        b_sub = W.hashed_values(ks, cols, N, sb)                  # K x cols
    else:
        a_sub = W.hashed_values(ks, rows, M, sa).T
        b_sub = W.hashed_values(cols, ks, K, sb).T
    R, Cn = len(rows), len(cols)
    a_bits = W.storage_view(W.cast(np.ascontiguousarray(a_sub).reshape(-1), dtype))
    b_bits = W.storage_view(W.cast(np.ascontiguousarray(b_sub).reshape(-1), dtype))
    want = np.zeros(R * Cn, a_bits.dtype)
    oracle.gemm("row", "row", R, Cn, K, 1.0, a_bits, K, b_bits, Cn, 0.0, None, want, Cn, dtype,
                want_exact=False)
    want = want.reshape(R, Cn)
    Cv = C.view(ibits)
    if lay == "row":
        got = Cv.view(M, N)[torch.as_tensor(rows, device=dev)][:, torch.as_tensor(cols, device=dev)]
    else:
        got = Cv.view(N, M)[torch.as_tensor(cols, device=dev)][:, torch.as_tensor(rows, device=dev)].T
    got = got.contiguous().cpu().numpy().view(want.dtype)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d of %d sampled outputs differ, first at row %d col %d" % (
        name, len(bad), got.size, rows[bad[0][0]], cols[bad[0][1]])
    say(name, "checked", R, "x", Cn, "outputs; rows from", rows[0], "to", rows[-1])
    del A, B, C
    torch.cuda.empty_cache()
