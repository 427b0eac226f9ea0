"""Pins for the measurement formulas and the dimension-efficiency model (CPU).

Values are the ones the pages print (fixtures in tests/golden cite them):
TraceLens's tile/wave quantization examples and roofline row, FlyDSL's padding
screen figures, and the GEMM guide's worked FP8 example.
"""
import json
import os

import bench
import oracle


def _load(golden_dir, name):
    return json.load(open(os.path.join(golden_dir, name)))


def test_dim_eff_worked_examples(golden_dir):
    g = _load(golden_dir, "dim_eff.json")
    for c in g["cases"]:
        tiles, te, we, de = oracle.dim_eff(c["M"], c["N"], c["mt_m"], c["mt_n"], c["num_cus"])
        assert tiles == c["num_tiles"]
        assert abs(te - c["tile_eff"]) <= c["tol"]
        assert abs(we - c["wq_eff"]) <= c["tol"]
        assert abs(de - c["dim_eff"]) <= c["tol"]
    for c in g["row_waste"]:
        tiles, te, _, _ = oracle.dim_eff(c["M"], 1, c["tile_m"], 1, 1)
        waste = 1.0 - te                       # padded rows / padded total
        assert abs(waste - c["waste_fraction"]) <= c["tol"]
    for c in g["area_ratio"]:
        _, te, _, _ = oracle.dim_eff(c["M"], c["N"], c["mt_m"], c["mt_n"], 256)
        assert abs(1.0 / te - c["padded_over_real"]) <= c["tol"]


def test_metric_formulas(golden_dir):
    g = _load(golden_dir, "metrics.json")
    for c in g["flops"]:
        assert abs(bench.flops(c["M"], c["N"], c["K"]) / 1e9 - c["gflop"]) <= c["tol"]
    for c in g["bytes_fp8_per_token_scales"]:
        mb = bench.alg_bytes(c["M"], c["N"], c["K"], "fp8", scales="per_token") / 1e6
        assert abs(mb - c["mb"]) <= c["tol"]
    for c in g["time_at_rate"]:
        ms = bench.flops(c["M"], c["N"], c["K"]) / (c["tflops"] * 1e12) * 1e3
        assert abs(ms - c["ms"]) <= c["tol"]
        gbps = bench.alg_bytes(c["M"], c["N"], c["K"], "fp8", scales="per_token") / (c["ms"] * 1e-3) / 1e9
        assert abs(gbps - c["gbps"]) <= c["gbps_tol"]
    for c in g["arith_intensity_16bit"]:
        ai = bench.flops(c["M"], c["N"], c["K"]) / bench.alg_bytes(c["M"], c["N"], c["K"], "bf16")
        assert abs(ai - c["flop_per_byte"]) <= c["tol"]
    for c in g["us_to_tflops"]:
        assert abs(bench.tflops_at(c["M"], c["N"], c["K"], c["us"]) - c["tflops"]) <= 0.05


def test_roofline_bounds():
    # 4096^3 bf16 is MFMA bound (54.6 us); 1x11008x4096 is HBM bound (11.3 us)
    assert abs(bench.roofline_us(4096, 4096, 4096, "bf16") - 54.61) < 0.01
    assert abs(bench.roofline_us(1, 11008, 4096, "bf16") - 11.276) < 0.01
    assert bench.alg_bytes(1, 11008, 4096, "bf16") == 90_207_744
    assert bench.alg_bytes(4096, 4096, 4096, "fp8") == 67_108_872


def test_dim_eff_closed_forms():
    # tiles an exact multiple of the CU count: no idle CUs in the last round
    assert oracle.dim_eff(4096, 4096, 256, 256, 256) == (256, 1.0, 1.0, 1.0)
    tiles, te, we, de = oracle.dim_eff(304 * 64, 128, 64, 64, 304)
    assert (tiles, we) == (608, 1.0)
    # one tile more than the CUs: two rounds, the second with one busy CU
    tiles, te, we, de = oracle.dim_eff(257 * 16, 16, 16, 16, 256)
    assert tiles == 257 and abs(we - 257 / 512) < 1e-15
    # padding only in N
    tiles, te, we, de = oracle.dim_eff(64, 100, 64, 64, 1)
    assert tiles == 2 and te == 100 / 128 and we == 1.0
