"""Resource arithmetic for dense GEMM: FLOPs, bytes, intensity, waves, roofline.

Host-side bookkeeping used by the benchmark and by the tile-size reasoning.
Every formula is the one the pages print; the tests pin each one to a number a
page prints for a worked example.
"""
from __future__ import annotations

import math

# MI355X published peaks (dense, no sparsity).
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "fp8": 5033.2, "f32": 157.3, "f64": 78.6}
PEAK_HBM_GBS = 8000.0
N_CU = 256
N_XCD = 8


def gemm_flops(M: int, N: int, K: int) -> int:
    """2*M*N*K: one multiply and one add per term (SGEMM report, section
    "main example K3" GFLOP/s line; zwxr.cn SGEMM post section 1.1; Chapter 5
    "Operators and Runtime" section 5.2.1, F_gemm)."""
    return 2 * M * N * K


def min_bytes(M: int, N: int, K: int, es_in: int, es_out: int | None = None) -> int:
    """Every operand crosses the memory interface once: es*(MK + KN) + es_out*MN
    (Chapter 5 section 5.2.1, V_once; K1 GEMM resource model, part 2)."""
    es_out = es_in if es_out is None else es_out
    return es_in * (M * K + K * N) + es_out * M * N


def tiled_bytes(M: int, N: int, K: int, m: int, n: int, es_in: int,
                es_out: int | None = None) -> int:
    """Traffic when each m x n output tile reads its own A strip and B strip
    with no reuse between tiles: A is read ceil(N/n) times, B ceil(M/m) times,
    C written once (Chapter 5 section 5.2.2, Example 5-3; K1 GEMM resource
    model, part 2)."""
    es_out = es_in if es_out is None else es_out
    return (es_in * M * K * math.ceil(N / n) + es_in * K * N * math.ceil(M / m)
            + es_out * M * N)


def tile_local_bytes(m: int, n: int, k: int, es_in: int = 2, es_acc: int = 4) -> int:
    """Working set of one tile with one input buffer: 2mk + 2kn + 4mn bytes for
    16-bit inputs and an FP32 accumulator (Chapter 5 section 5.2.2, Example 5-3)."""
    return es_in * m * k + es_in * k * n + es_acc * m * n


def tile_intensity(bm: int, bn: int) -> float:
    """Per-tile reuse BM*BN/(BM+BN) (MTT S4000 GEMM write-up, section 1)."""
    return bm * bn / (bm + bn)


def waves(tiles: int, slots: int) -> tuple[int, float]:
    """(number of waves, efficiency tiles / (waves*slots)) (K1 GEMM resource
    model, part 4)."""
    w = math.ceil(tiles / slots)
    return w, tiles / (w * slots)


def roofline_time(flops: float, nbytes: float, peak_flops: float, peak_bw: float):
    """(t_compute, t_memory, bound) in seconds (K1 GEMM resource model, part 5)."""
    tc, tm = flops / peak_flops, nbytes / peak_bw
    return tc, tm, ("compute" if tc >= tm else "memory")


def pipeline_time(n: int, t_move: float, t_compute: float) -> float:
    """Two-slot pipeline T = t_m + (n-1)*max(t_m, t_c) + t_c (Chapter 5
    section 5.3.2, Example 5-5)."""
    return t_move + (n - 1) * max(t_move, t_compute) + t_compute


def tol_half(K: int) -> float:
    """FP16/BF16 absolute tolerance 0.01*sqrt(K/512) (MTT S4000 GEMM write-up,
    sections 1 and 8)."""
    return 0.01 * math.sqrt(K / 512.0)


def tol_f32_rel(K: int) -> float:
    """FP32 tolerance factor 1e-4*sqrt(K/256), applied relative to max|C|."""
    return 1e-4 * math.sqrt(max(K, 1) / 256.0)


def ulp_half(x: float, dtype: str) -> float:
    """Spacing of the output format at |x| (FP16: 11 significant bits, smallest
    normal 2^-14; BF16: 8 significant bits, smallest normal 2^-126)."""
    p, emin = (11, -14) if dtype == "f16" else (8, -126) if dtype == "bf16" else (24, -126)
    ax = abs(x)
    if ax == 0:
        return 2.0 ** (emin - p + 1)
    e = math.frexp(ax)[1]
    return 2.0 ** max(e - p, emin - p + 1)
