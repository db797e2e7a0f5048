"""Pins of the FP8 E4M3 oracle (oracle/fp8.py) against what the pages and the
format fix, independent of the oracle's own code: the OCP E4M3FN definition,
an independent library conversion (torch.float8_e4m3fn), the worked example
of a whole-row scale (Example 5-7), closed forms of the GEMM on integer codes
and the traffic arithmetic of Example 5-8 that motivates a separate
quantisation kernel."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def check_format():
    v = fp8.e4m3_values()
    assert v[0x7E] == 448.0 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x38] == 1.0 and v[0xB8] == -1.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                          # 127 distinct, increasing
    assert np.array_equal(v[0x80:0xFF], -pos)
    # Spacing: 2^-9 up to 2^-5, then 2^(e-10) within each binade [2^(e-7), 2^(e-6)).
    for e in range(1, 16):
        lo = 2.0 ** (e - 7)
        binade = pos[(pos >= lo) & (pos < 2 * lo)]
        assert np.allclose(np.diff(binade), lo / 8)


def check_encode_against_library():
    # Every FP32 value on a dense grid of [-448, 448] (ties, subnormals,
    # binade edges) rounds like torch's float8_e4m3fn conversion.
    grid = np.concatenate([np.linspace(-448, 448, 200001), fp8.e4m3_values()[:0x7F] * 1.0,
                           (fp8.e4m3_values()[:0x7E] + fp8.e4m3_values()[1:0x7F]) / 2,
                           np.ldexp(np.arange(0, 80), -11), -np.ldexp(np.arange(0, 80), -11)])
    g32 = grid.astype(np.float32)
    ours = fp8.e4m3_encode(g32.astype(np.float64))
    ref = torch.from_numpy(g32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert fp8.e4m3_encode(np.array([np.nan, -np.nan]))[0] == 0x7F
    assert fp8.e4m3_encode(np.array([1000.0, -1e30]))[0] == 0x7E       # saturate
    assert fp8.e4m3_encode(np.array([-1e30]))[0] == 0xFE


def check_row_scale_example():
    ex = GOLD["fp8_row_scale"]
    row = np.zeros((1, ex["row_len"]))
    row[0, 0] = ex["block_first"][0]
    row[0, ex["block_len"]] = ex["block_first"][1]
    q, s = fp8.quantize_rows(row)
    assert fp8.e4m3_decode(q[0, 0]) == ex["stored_first"]
    amax = max(ex["block_first"])
    assert Fraction(fp8.e4m3_decode(q[0, 0])) * Fraction(amax) / Fraction(ex["e4m3_max"]) == \
        Fraction(ex["dequant_first"])
    assert s[0] == np.float32(amax) / np.float32(ex["e4m3_max"])
    assert fp8.e4m3_decode(q[0, ex["block_len"]]) == ex["e4m3_max"]
    # The block-by-block scale of the pages' counter-example stores 448 for the 1.
    qb, _ = fp8.quantize_rows(row[:, :ex["block_len"]])
    assert fp8.e4m3_decode(qb[0, 0]) * ex["block_first"][0] / ex["e4m3_max"] == ex["blockwise_dequant_first"]
    assert Fraction(ex["blockwise_dequant_first"]) - Fraction(ex["dequant_first"]) == Fraction(ex["difference"])
    assert abs(float(Fraction(ex["difference"])) - 0.018) < 0.001
    assert ex["scaled_first"] == ex["block_first"][0] * ex["e4m3_max"] / amax


def check_quantize_invariants():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 300)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    x = x.astype(np.float64)
    q, s = fp8.quantize_rows(x)
    deq = fp8.e4m3_decode(q)
    amax = np.max(np.abs(x), axis=1)
    # The largest magnitude of each row maps to +-448 exactly.
    i = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(deq[np.arange(64), i]) == 448.0)
    # Every element is within half a step of its scaled value: 2^-4 relative in
    # the normal range, 2^-10 absolute (in scaled units) below it.
    t = x * 448.0 / amax[:, None]
    err = np.abs(deq - t)
    assert np.all(err <= np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6))
    assert np.allclose(s.astype(np.float64), amax / 448.0, rtol=2 ** -23)
    # Zero row: zero scale, signed zeros kept; NaN row: all NaN; inf row.
    z = np.array([[0.0, -0.0, 0.0]])
    qz, sz = fp8.quantize_rows(z)
    assert sz[0] == 0 and qz.tolist() == [[0x00, 0x80, 0x00]]
    qn, sn = fp8.quantize_rows(np.array([[1.0, np.nan, -2.0]]))
    assert np.isnan(sn[0]) and np.all(qn == 0x7F)
    qi, si = fp8.quantize_rows(np.array([[1.0, np.inf, -2.0]]))
    assert np.isinf(si[0]) and qi.tolist() == [[0x00, 0x7F, 0x80]]


def check_fp8_gemm_closed_forms():
    rng = np.random.default_rng(3)
    M, N, K = 7, 5, 33
    ia = rng.integers(-16, 17, (M, K))
    ib = rng.integers(-16, 17, (N, K))
    qa, qb = fp8.e4m3_encode(ia.astype(np.float64)), fp8.e4m3_encode(ib.astype(np.float64))
    assert np.array_equal(fp8.e4m3_decode(qa), ia)           # small integers are exact
    sa = (2.0 ** rng.integers(-3, 4, M)).astype(np.float32)
    sb = (2.0 ** rng.integers(-3, 4, N)).astype(np.float32)
    c = fp8.fp8_gemm(M, N, K, 1.0, qa.ravel(), K, sa, qb.ravel(), K, sb)
    want = (sa[:, None].astype(np.float64) * sb[None, :]) * (ia @ ib.T)
    assert np.array_equal(c, want)
    # Row stride larger than K; alpha, beta.
    lda, ldb = K + 5, K + 3
    pa = np.zeros((M, lda), np.uint8); pa[:, :K] = qa
    pb = np.zeros((N, ldb), np.uint8); pb[:, :K] = qb
    c0 = rng.integers(-8, 9, (M, N)).astype(np.float64)
    c2 = fp8.fp8_gemm(M, N, K, 0.5, pa.ravel(), lda, sa, pb.ravel(), ldb, sb, beta=-2.0, c0=c0)
    assert np.array_equal(c2, 0.5 * want - 2.0 * c0)
    # One-hot codes pick single products: sa[m] * sb[n] * qa[m,k0] * qb[n,k0].
    oa = np.zeros((M, K), np.uint8); ob = np.zeros((N, K), np.uint8)
    oa[:, 4] = fp8.e4m3_encode(np.full(M, 3.0)); ob[:, 4] = fp8.e4m3_encode(np.full(N, -0.5))
    c3 = fp8.fp8_gemm(M, N, K, 1.0, oa.ravel(), K, sa, ob.ravel(), K, sb)
    assert np.array_equal(c3, -1.5 * sa[:, None].astype(np.float64) * sb[None, :])


def check_fp8_gemm_exact_at_its_limit():
    # The K sum is exact up to K = 2^17: the widest products (448^2, near
    # 2^17.6) and the narrowest (2^-9 * 2^-9 = 2^-18) mixed in one row, compared
    # with the exact integer sum of the products scaled by 2^18; K = 2^17 + 1
    # is refused.
    K = 2 ** 17
    rng = np.random.default_rng(17)
    big = rng.random(K) < 0.5
    va = np.where(big, 448.0, 2.0 ** -9) * np.where(rng.random(K) < 0.5, -1.0, 1.0)
    vb = np.where(big, 448.0, 2.0 ** -9)
    qa, qb = fp8.e4m3_encode(va), fp8.e4m3_encode(vb)
    assert np.array_equal(fp8.e4m3_decode(qa), va) and np.array_equal(fp8.e4m3_decode(qb), vb)
    one = np.ones(1, np.float32)
    c = fp8.fp8_gemm(1, 1, K, 1.0, qa, K, one, qb, K, one)
    exact = sum(int(a * b * 2 ** 18) for a, b in zip(va.tolist(), vb.tolist()))
    assert c[0, 0] == exact / 2 ** 18
    try:
        fp8.fp8_gemm(1, 1, K + 1, 1.0, np.zeros(K + 1, np.uint8), K + 1, one,
                     np.zeros(K + 1, np.uint8), K + 1, one)
        refused = False
    except ValueError:
        refused = True
    assert refused, "K = 2^17 + 1 must be refused"


def check_quant_traffic_example():
    ex = GOLD["fp8_quant_traffic"]
    sep = ex["A_fp16_mib"] + ex["A_fp8_mib"] + ex["col_blocks"] * ex["A_fp8_mib"]
    fused = ex["A_fp16_mib"] + ex["col_blocks"] * ex["A_fp16_mib"]
    wo = ex["row_blocks"] * ex["W_fp8_mib"] + ex["C_fp16_mib"]
    assert (sep, fused, wo) == (ex["separate_input_mib"], ex["fused_input_mib"], ex["weights_output_mib"])
    assert (sep + wo, fused + wo) == (ex["separate_total_mib"], ex["fused_total_mib"])
    mib = 2 ** 20
    assert 4096 * 4096 * 2 == ex["A_fp16_mib"] * mib and 4096 * 1536 == ex["W_fp8_mib"] * mib
    assert (4096 // 128, 1536 // 128) == (ex["row_blocks"], ex["col_blocks"])


FP8_PINS = [check_format, check_encode_against_library, check_row_scale_example,
            check_quantize_invariants, check_fp8_gemm_closed_forms, check_fp8_gemm_exact_at_its_limit,
            check_quant_traffic_example]


@pytest.mark.parametrize("check", FP8_PINS, ids=lambda f: f.__name__)
def test_fp8_pin(check):
    check()
