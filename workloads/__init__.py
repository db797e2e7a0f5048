"""Seeded synthetic inputs for the GEMM workloads.

This module only draws numbers and lays them out in memory.  It holds none of
the GEMM's arithmetic, so both the CPU oracle and the HIP library can consume
its output without sharing any of the method's code.

Recipe (stated in the design notes as well):
  * numpy ``default_rng`` (PCG64), one seed per operand;
  * values drawn in float64, then cast round-to-nearest-even to the storage
    type (float32 / float16 by numpy, bfloat16 by torch from float32);
  * operand buffers are laid out with their leading dimension; the gap between
    the logical extent and the leading dimension is filled with NaN so that a
    kernel reading outside the logical matrix poisons its own result.

Workload shapes are those of the pages: square FP32 SGEMM (the SGEMM report's
4096^3 main table), the FP16 column-major contest shapes (the MTT S4000 GEMM
write-up, its grading section), and the Qwen3-8B FFN projection C = X W with
M = 1024, K = 4096, N = 12288 (Chapter 5 "Operators and Runtime", section 5.2).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
STORAGE_NP = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def draw(kind: str, seed: int, n: int, scale: float = 1.0) -> np.ndarray:
    """n float64 samples: 'uniform' U[-1,1], 'normal' N(0, scale^2), 'int' U{-4..4}."""
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        return rng.uniform(-1.0, 1.0, n)
    if kind == "normal":
        return rng.normal(0.0, scale, n)
    if kind == "int":
        return rng.integers(-4, 5, n).astype(np.float64)
    if kind == "smallint":                        # U{-2..2}: keeps long sums tiny
        return rng.integers(-2, 3, n).astype(np.float64)
    if kind == "f16sub":                          # FP16 subnormals (and zero): j * 2^-24, |j| < 1024
        return rng.integers(-1023, 1024, n).astype(np.float64) * 2.0 ** -24
    raise ValueError(kind)


def cast(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 -> CPU tensor of the storage dtype, round-to-nearest-even."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(x64.astype(np.float16)))
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(torch.bfloat16)
    raise ValueError(dtype)


def operand(kind: str, seed: int, rows: int, cols: int, layout: str, ld: int, dtype: str,
            scale: float = 1.0) -> torch.Tensor:
    """A rows x cols matrix stored flat with leading dimension ld.

    row-major: element (r, c) at r*ld + c (buffer rows*ld);
    col-major: element (r, c) at c*ld + r (buffer cols*ld).
    Padding between the extent and ld holds NaN.
    """
    outer, inner = (rows, cols) if layout == "row" else (cols, rows)
    if ld < max(1, inner):
        raise ValueError("leading dimension too small")
    vals = draw(kind, seed, rows * cols, scale).reshape(rows, cols)
    if layout == "col":
        vals = vals.T
    buf = np.full((max(outer, 1), ld), np.nan)
    buf[:outer, :inner] = vals
    return cast(buf.reshape(-1)[: max(outer, 1) * ld], dtype)


# ---------------------------------------------------------------------------
# Operands too large to draw on the host (more than 2^31 elements): element
# (r, c) of a matrix with `cols` columns is a function of the counter
# r * cols + c and a seed, so a device fills the whole buffer and the host
# recomputes only the rows and columns it checks.  Values are -1, 0 or 1
# (exact in every storage type; integer sums stay exact in FP32).  The mixing
# steps are the 32-bit finaliser of MurmurHash3 (Appleby), applied to the
# counter's low and high words.
# ---------------------------------------------------------------------------
_M32 = 0xFFFFFFFF


def _fmix32_np(h):
    h = h & _M32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & _M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & _M32
    h ^= h >> 16
    return h


def hashed_values(rows: np.ndarray, cols: np.ndarray, ncols: int, seed: int) -> np.ndarray:
    """float64 values of elements (rows[i], cols[j]) of a counter-hashed
    matrix with `ncols` columns (an outer grid, len(rows) x len(cols))."""
    n = (np.asarray(rows, np.uint64)[:, None] * np.uint64(ncols) +
         np.asarray(cols, np.uint64)[None, :])
    h = _fmix32_np((n & np.uint64(_M32)) ^ np.uint64(seed & _M32))
    h = _fmix32_np(h ^ (n >> np.uint64(32)))
    return (h % np.uint64(3)).astype(np.float64) - 1.0


def _fmix32_torch(h):
    h = h & _M32
    h = h ^ (h >> 16)
    h = (h * 0x85EBCA6B) & _M32
    h = h ^ (h >> 13)
    h = (h * 0xC2B2AE35) & _M32
    h = h ^ (h >> 16)
    return h


def hashed_operand(nrows: int, ncols: int, seed: int, dtype: str, device,
                   chunk: int = 1 << 26) -> torch.Tensor:
    """The whole nrows x ncols counter-hashed matrix, row-major, filled on
    `device` a few rows at a time (int64 arithmetic: every product of a
    32-bit value and a 32-bit constant fits, and only its low 32 bits are
    kept)."""
    out = torch.empty(nrows * ncols, dtype=TORCH_DTYPES[dtype], device=device)
    step = max(1, chunk // max(ncols, 1))
    c = torch.arange(ncols, dtype=torch.int64, device=device)
    for r0 in range(0, nrows, step):
        r = torch.arange(r0, min(nrows, r0 + step), dtype=torch.int64, device=device)
        n = r[:, None] * ncols + c[None, :]
        h = _fmix32_torch((n & _M32) ^ (seed & _M32))
        h = _fmix32_torch(h ^ (n >> 32))
        out[r0 * ncols:(r0 + len(r)) * ncols] = ((h % 3) - 1).reshape(-1).to(out.dtype)
    return out


# Canary bit patterns written into C before a call whose beta is 0 (quiet
# NaNs): an output the library never wrote still holds one afterwards.
CANARY = {"f32": 0x7FA5A5A5, "f16": 0x7E5A, "bf16": 0x7FA5}


def c_initial(case: "Case", C0):
    """Initial C buffer (CPU): a copy of C0 when beta != 0, else canary bits
    everywhere."""
    if C0 is not None:
        return C0.clone()
    n = case.c_numel()
    if case.dtype == "f32":
        return torch.full((n,), CANARY["f32"], dtype=torch.int32).view(torch.float32)
    t = torch.full((n,), CANARY[case.dtype], dtype=torch.int16)   # both patterns < 0x8000
    return t.view(torch.float16 if case.dtype == "f16" else torch.bfloat16)


def storage_view(t: torch.Tensor) -> np.ndarray:
    """The raw bits of a CPU tensor as a numpy uint array (for the oracle)."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


@dataclass
class Case:
    """One GEMM problem: shapes, layouts, leading dimensions, dtype and seeds."""
    name: str
    M: int
    N: int
    K: int
    dtype: str
    layoutA: str = "row"
    layoutB: str = "row"
    lda: int | None = None
    ldb: int | None = None
    ldc: int | None = None
    alpha: float = 1.0
    beta: float = 0.0
    kindA: str = "uniform"
    kindB: str = "uniform"
    kindC: str = "uniform"
    scaleA: float = 1.0
    scaleB: float = 1.0
    seeds: tuple = (1, 2, 3)
    extra: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.lda is None:
            self.lda = max(1, self.K if self.layoutA == "row" else self.M)
        if self.ldb is None:
            self.ldb = max(1, self.N if self.layoutB == "row" else self.K)
        if self.ldc is None:
            self.ldc = max(1, self.N if self.layoutA == "row" else self.M)

    def make(self):
        """(A, B, C0) CPU tensors; C0 is None when beta == 0."""
        A = operand(self.kindA, self.seeds[0], self.M, self.K, self.layoutA, self.lda, self.dtype,
                    self.scaleA)
        B = operand(self.kindB, self.seeds[1], self.K, self.N, self.layoutB, self.ldb, self.dtype,
                    self.scaleB)
        C0 = None
        if self.beta != 0.0:
            C0 = operand(self.kindC, self.seeds[2], self.M, self.N, self.layoutA, self.ldc,
                         self.dtype)
        return A, B, C0

    def c_numel(self) -> int:
        outer = self.M if self.layoutA == "row" else self.N
        return max(outer, 1) * self.ldc


# The five workload families, at their full sizes.
def sgemm_256(int_valued: bool = False) -> Case:
    k = "int" if int_valued else "uniform"
    return Case("sgemm_256" + ("_int" if int_valued else ""), 256, 256, 256, "f32",
                kindA=k, kindB=k, seeds=(1001, 1002, 1003))


def sgemm_4096() -> Case:
    return Case("sgemm_4096", 4096, 4096, 4096, "f32", seeds=(2001, 2002, 2003))


def hgemm_colmajor(M: int, N: int, K: int) -> Case:
    return Case("hgemm_col_%dx%dx%d" % (M, N, K), M, N, K, "f16", layoutA="col", layoutB="col",
                seeds=(3001, 3002, 3003))


HGEMM_SHAPES = [(256, 256, 512), (512, 1024, 2048), (8192, 8192, 16384)]


def ffn_bf16(M: int = 1024) -> Case:
    seeds = (4001, 4002, 4003) if M == 1024 else (5001, 4002, 5003)
    return Case("ffn_bf16_m%d" % M, M, 12288, 4096, "bf16", kindA="normal", kindB="normal",
                scaleA=1.0, scaleB=0.02, seeds=seeds)


def ffn_share_bf16() -> Case:
    """One GPU's share of the FFN projection when its 12288 output columns are
    split over 8 GPUs: X[1024x4096] W[4096x1536], same distributions as
    ffn_bf16() (its own matrices: W is drawn at the share's shape)."""
    return Case("ffn_share_bf16_1024x1536x4096", 1024, 1536, 4096, "bf16", kindA="normal",
                kindB="normal", scaleA=1.0, scaleB=0.02, seeds=(4101, 4102, 4103))


def ffn_bf16_silu() -> Case:
    """The FFN projection with the fused activation, Y = SiLU(XW) (same inputs
    as ffn_bf16(); the epilogue is named in `extra`)."""
    c = ffn_bf16()
    c.name = "ffn_bf16_silu_m1024"
    c.extra = {"epilogue": "silu"}
    return c


def ffn_gated_bf16(M: int = 1024) -> Case:
    """Gate/up pair of the FFN: X[Mx4096] with W_g and W_u [4096x12288], both
    N(0, 0.02^2).  X and W_g are those of ffn_bf16(); W_u has its own seed
    (extra["seed_u"]).  Z = SiLU(X W_g) * (X W_u)."""
    c = ffn_bf16(M)
    c.name = "ffn_gated_bf16_m%d" % M
    c.extra = {"gated": True, "seed_u": 4004}
    return c


def ffn_gated_share_bf16() -> Case:
    """The gated pair at one GPU's share (N = 12288 / 8 = 1536)."""
    c = ffn_share_bf16()
    c.name = "ffn_gated_share_bf16_1024x1536x4096"
    c.extra = {"gated": True, "seed_u": 4104}
    return c


def fp8_ffn_bf16() -> Case:
    """FP8 form of the FFN projection: X[1024x4096] BF16 ~ N(0,1) quantised per
    row each call; the weights W ~ N(0, 0.02^2), stored as 12288 rows of 4096
    (one row per output column, i.e. B column-major) and quantised per row
    once; BF16 output."""
    return Case("fp8_ffn_1024x12288x4096", 1024, 12288, 4096, "bf16", layoutB="col",
                kindA="normal", kindB="normal", scaleA=1.0, scaleB=0.02,
                seeds=(4301, 4302, 4303), extra={"fp8": True})


def fp8_quant_example() -> Case:
    """The shapes of the separate-versus-fused quantisation example: FP16
    A[4096x4096] ~ N(0,1), FP8 weights for 1536 output columns, FP16 output."""
    return Case("fp8_4096x1536x4096", 4096, 1536, 4096, "f16", layoutB="col", kindA="normal",
                kindB="normal", scaleA=1.0, scaleB=0.02, seeds=(4311, 4312, 4313),
                extra={"fp8": True})


def gated_inputs(case: Case):
    """(X, W_g, W_u) CPU tensors of a gated-pair case."""
    X, Wg, _ = case.make()
    Wu = operand(case.kindB, case.extra["seed_u"], case.K, case.N, "row", case.ldb, case.dtype,
                 case.scaleB)
    return X, Wg, Wu


SKINNY_M = [1, 16, 64]


def ragged_f32() -> Case:
    return Case("ragged_f32_1000x12290x4095", 1000, 12290, 4095, "f32", lda=4095, ldb=12290,
                ldc=12290, kindA="normal", kindB="normal", seeds=(5101, 5102, 5103))
