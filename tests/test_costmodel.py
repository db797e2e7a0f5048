"""Cost-model calculators against the numbers the pages print (tests/golden)."""
import json
import math
import os

import pytest

from dense_gemm_mgemm_amd import costmodel as cm

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
MiB, KiB = 2 ** 20, 2 ** 10


def test_flops_4096():
    g = G["flops_4096"]
    assert cm.gemm_flops(g["M"], g["N"], g["K"]) == g["value"]


def test_ffn_flops_and_once_bytes():
    g = G["ffn_flops_gflop"]
    assert cm.gemm_flops(g["M"], g["N"], g["K"]) / 1e9 == pytest.approx(g["value"], rel=g["rel_tol"])
    g = G["ffn_once_mib"]
    assert cm.min_bytes(g["M"], g["N"], g["K"], g["es"]) == g["value"] * MiB


def test_ffn_tiled_traffic_table():
    g = G["ffn_tiled_mib"]
    # The page divides its rounded 103 GFLOPs (not the exact 2MNK = 103.08e9)
    # by the traffic: 103e9 / 3096 MiB = 31.7, whereas 2MNK would give 31.75.
    fl = G["ffn_flops_gflop"]["value"] * 1e9
    for m, n, mib, kib, ai in g["rows"]:
        t = cm.tiled_bytes(g["M"], g["N"], g["K"], m, n, g["es"])
        assert t == mib * MiB
        assert cm.tile_local_bytes(m, n, g["k"]) == kib * KiB
        assert round(fl / t, 1) == ai


def test_p2_bytes_and_intensity():
    g = G["p2_min_bytes"]
    mn = cm.min_bytes(g["M"], g["N"], g["K"], g["es"])
    assert mn == g["value"]
    g2 = G["p2_tiled_bytes"]
    tb = cm.tiled_bytes(g2["M"], g2["N"], g2["K"], g2["m"], g2["n"], g2["es"])
    assert tb == g2["value"]
    assert round(tb / mn, 1) == g2["ratio"]
    fl = cm.gemm_flops(4096, 4096, 4096)
    assert int(fl / mn) == G["p2_intensity"]["min"]
    assert int(fl / tb) == G["p2_intensity"]["tiled"]


def test_p2_waves():
    g = G["p2_waves"]
    w, eff = cm.waves(g["tiles"], g["slots"])
    assert w == g["waves"] and round(eff, 3) == g["efficiency"]
    w, eff = cm.waves(g["tiles"], g["slots2"])
    assert w == g["waves2"] and round(eff, 3) == g["efficiency2"]


def test_p2_roofline_times():
    g = G["p2_roofline"]
    fl = cm.gemm_flops(4096, 4096, 4096)
    tc, tm, bound = cm.roofline_time(fl, G["p2_min_bytes"]["value"], g["peak_flops"], g["bw"])
    assert round(tc * 1e3, 2) == g["t_compute_ms"] and round(tm * 1e3, 2) == g["t_mem_min_ms"]
    assert bound == "compute"
    tc, tm, bound = cm.roofline_time(fl, G["p2_tiled_bytes"]["value"], g["peak_flops"], g["bw"])
    assert round(tm * 1e3, 2) == g["t_mem_tiled_ms"] and bound == "memory"


def test_p5_pipeline():
    g = G["p5_pipeline"]
    assert round(cm.pipeline_time(g["n"], g["t_move_us"], g["t_compute_us"]), 2) == g["t_pipe_us"]
    assert round(g["n"] * (g["t_move_us"] + g["t_compute_us"]), 2) == g["t_serial_us"]


def test_p4_tolerance_and_tile_ai():
    g = G["p4_tolerance"]
    assert abs(cm.tol_half(g["K"]) - g["value"]) <= g["abs_tol"]
    for bm, bn, ai in G["p4_tile_ai"]["rows"]:
        assert cm.tile_intensity(bm, bn) == ai


def test_ulp():
    assert cm.ulp_half(1.0, "f16") == 2.0 ** -10
    assert cm.ulp_half(100.0, "f16") == 2.0 ** -4        # [64,128): 2^6 * 2^-10
    assert cm.ulp_half(1.0, "bf16") == 2.0 ** -7
    assert cm.ulp_half(1e-6, "f16") == 2.0 ** -24        # subnormal spacing
    assert math.isclose(cm.ulp_half(3.0, "f32"), 2.0 ** -22)
