"""The cycle model must reproduce the figures the pages print (FA4 paper
§3.1.1 Table 1, §3.2.1 Eq. 7-8) before it is trusted with CDNA4 constants."""
import json
import os

from oracle import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_reproduces_table1():
    g = json.load(open(os.path.join(GOLDEN, "fa4_table1_roofline.json")))
    t = g["tile"]
    hw = dict(roofline.B200_SM)
    assert hw["smem_bytes_per_clk"] == g["b200_per_sm"]["smem_bytes_per_clk"]
    assert hw["exp_per_clk"] == g["b200_per_sm"]["exp_per_clk"]
    c = roofline.forward_tile_cycles_b200(t["M"], t["N"], t["d"], hw)
    assert c == {k: float(v) for k, v in g["cycles"].items()}


def test_reproduces_backward_formula():
    g = json.load(open(os.path.join(GOLDEN, "fa4_table1_roofline.json")))["backward"]
    M, N, d = g["M"], g["N"], g["d"]
    assert roofline.backward_tile_mma_cycles(M, N, d) == eval(g["formula"], {}, dict(M=M, N=N, d=d))


def test_mi355x_peak():
    assert abs(roofline.peak_bf16_tflops() - 2516.58) < 0.01


def test_cdna4_tile_model_scales():
    a = roofline.forward_tile_cycles_cdna4(256, 128, 128, rows_per_wave=32)
    b = roofline.forward_tile_cycles_cdna4(256, 128, 128, rows_per_wave=64)
    assert a["mma"] == 4096.0 and a["exp"] == 2048.0
    assert a["lds"] == 2 * b["lds"]
