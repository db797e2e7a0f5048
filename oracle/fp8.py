"""CPU oracle for the FP8 E4M3 path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it; it shares no code with the HIP library.

What it computes ("Chapter 5: Operators and Runtime", ai-infra-book):

* The E4M3FN format (section 5.4.3, Example 5-7): one sign bit, four exponent
  bits (bias 7), three mantissa bits; exponent field 0 holds the subnormals
  m * 2^-9; the all-ones exponent with mantissa 7 is NaN, so the largest
  finite value is 1.75 * 2^8 = 448 and there is no infinity.
* Per-row quantisation (Example 5-7): the scale of a row comes from the
  largest magnitude of the WHOLE row, read before any element is quantised;
  each element is mapped to x * 448 / amax, rounded to a representable value,
  and dequantised as q * amax / 448.  The worked example: a row whose blocks
  start with 1 and 10 stores the 1 as 44 (44.8 rounded), which dequantises to
  55/56, not to the 1.0 a block-by-block scale would give.
* The FP8 GEMM (section 5.4.4, Example 5-8: FP8 activations with a scale per
  row, FP8 weights): C = round(alpha * sa[m] * sb[n] * sum_k qa[m,k] qb[n,k]
  + beta * C), where qb holds the weight matrix one output column per row
  (N x K) with its own per-row scale sb.  The scales factor out of the K sum.

Readings where the pages are silent (each also listed in the design notes):
* Rounding to E4M3 is to nearest, ties to the even mantissa; magnitudes
  above 448 saturate to 448 (the row's largest element can land a rounding
  above 448 after scaling).
* Each element is scaled by the row's factor 448 / amax (Example 5-7 scales
  the 1 "by 448/10"): r = 448 / amax is formed once per row in FP32
  (correctly rounded), then t = x * r in FP32 (one rounding), and the stored
  scale is amax / 448 in FP32; FP32 because the quantised code is an
  integer decision that both sides must take in the same precision.
* A row of zeros has scale 0 and codes of signed zero; a row holding a NaN
  has a NaN scale and NaN codes (0x7F) everywhere; a row holding +-inf (and
  no NaN) has an infinite scale, codes 0x7F for the infinite elements and
  signed zeros elsewhere.  Every NaN is stored as 0x7F.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 codes (float64; NaN for 0x7F and 0xFF)."""
    v = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            v[code] = np.nan
        elif e == 0:
            v[code] = sign * m * 2.0 ** -9
        else:
            v[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


_VALUES = e4m3_values()
# Non-negative finite codes in increasing value order (0x00 .. 0x7E).
_POS_CODES = np.arange(0x7F)
_POS_VALUES = _VALUES[_POS_CODES]


def e4m3_decode(codes) -> np.ndarray:
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(t) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even mantissa, magnitudes
    above 448 saturate, NaN -> 0x7F, the sign of zero is kept)."""
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    # Index of the largest representable value <= a (a <= 448 after the clip).
    ac = np.minimum(a, E4M3_MAX)
    lo = np.searchsorted(_POS_VALUES, ac, side="right") - 1
    lo = np.clip(lo, 0, len(_POS_VALUES) - 1)
    hi = np.minimum(lo + 1, len(_POS_VALUES) - 1)
    d_lo = ac - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - ac
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (_POS_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = mag | np.where(np.signbit(t), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(t), np.uint8(NAN_CODE), code).astype(np.uint8)


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row E4M3 quantisation of a matrix of exactly representable values
    (float64 holding FP32/FP16/BF16 elements).  Returns (codes uint8 M x K,
    scales float32 M): x ~ decode(codes) * scale."""
    x = np.asarray(x, dtype=np.float64)
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x, equal_nan=True), "inputs must be FP32 values"
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(x32), axis=1)                       # NaN if the row holds one
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        r = (np.float32(E4M3_MAX) / amax).astype(np.float32)      # per-row factor, float32
        t = x32 * r[:, None]                                      # float32 product
    t = np.where((amax == 0)[:, None], x32, t)                    # a zero row keeps its zeros
    return e4m3_encode(t), scale


def fp8_gemm(M, N, K, alpha, qa, lda, sa, qb, ldb, sb, beta=0.0, c0=None):
    """Unrounded FP64 value of C = alpha * sa[m] * sb[n] * sum_k qa[m,k] qb[n,k]
    + beta * c0 (M x N).  qa, qb: flat uint8 code buffers with row strides lda,
    ldb (qb holds one row of K codes per output column); sa, sb: float32.

    A product of two E4M3 values is a multiple of 2^-18 below 2^18 (36
    significant bits at most), so a partial sum of up to 2^17 of them needs at
    most 53 bits and is exact in FP64: for K <= 2^17 the K sum is exact in any
    order; the scaling is one FP64 rounding more.  Larger K is refused."""
    if K > 2 ** 17:
        raise ValueError("fp8_gemm: K = %d exceeds 2^17, where the FP64 sum stops being exact" % K)
    qa = np.asarray(qa, np.uint8)
    qb = np.asarray(qb, np.uint8)
    A = e4m3_decode(np.lib.stride_tricks.as_strided(qa, (M, K), (lda, 1))) if M and K else \
        np.zeros((M, K))
    B = e4m3_decode(np.lib.stride_tricks.as_strided(qb, (N, K), (ldb, 1))) if N and K else \
        np.zeros((N, K))
    with np.errstate(invalid="ignore", over="ignore"):
        S = A @ B.T
        c = alpha * (np.asarray(sa, np.float64)[:M, None] * np.asarray(sb, np.float64)[None, :N]) * S
        if c0 is not None and beta != 0.0:
            c = c + beta * np.asarray(c0, np.float64)
    return c
