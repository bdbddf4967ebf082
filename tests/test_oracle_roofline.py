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


def _close(a, b):
    return abs(a - b) <= 1e-9 * max(1.0, abs(b))


def test_cdna4_forward_tile_terms_hand_derived():
    """Each term of the CDNA4 forward tile model against values worked by
    hand from the MI355X rates (the 256 x 128 tile of Table 1's shape):
    d = 128: mma = 4*256*128*128/4096 = 4096 plus 8*8 16x16x32 row-sum
    products of 17.1 cycles over 4 SIMDs = 273.6; exp = 512 v_exp_f32 x 9.1 / 4
    = 1164.8; valu = 3.2 x 512 x 4.3 / 4 = 1761.28; LDS = 8 waves x 128 keys x
    128 dims x 2 bytes = 262144 bytes read row-wise at 213 B/clk plus the same
    transposed at 128 B/clk = 1230.7324 + 2048.  d = 64 halves the matrix
    and LDS terms."""
    c = roofline.forward_tile_cycles_cdna4(256, 128, 128)
    assert _close(c["mma"], 4369.6)
    assert _close(c["exp"], 1164.8)
    assert _close(c["valu"], 1761.28)
    assert _close(c["issue"], 2926.08)
    assert _close(c["lds"], 262144 / 213 + 2048.0)
    assert roofline.bound(c)[0] == "mma"
    c64 = roofline.forward_tile_cycles_cdna4(256, 128, 64)
    assert _close(c64["mma"], 2048 + 273.6)
    assert _close(c64["lds"], 131072 / 213 + 1024.0)
    assert _close(c64["issue"], 2926.08)
    name, frac = roofline.bound(c64)
    assert name == "issue" and _close(frac["mma"], 2321.6 / 2926.08)
    # without the row-sum products the matrix term is the plain 4 M N d / 4096
    assert roofline.forward_tile_cycles_cdna4(256, 128, 128, row_sum_mfma=False)["mma"] == 4096.0


def test_cdna4_gradient_tile_terms_hand_derived():
    """dK/dV tile: 128 keys x 64 streamed query rows, d = 128, four products
    (S, dP, dV, dK): mma = 2*4*128*64*128/4096 = 2048; exp = 128 instructions
    x 9.1 / 4 = 291.2; valu = 6 x 128 x 4.3 / 4 = 825.6; LDS: 4 waves x 64 rows
    x 128 dims x 2 bytes = 65536 bytes, read twice row-wise (Q, dO) and twice
    transposed (dO^T, Q^T) = 2*65536/213 + 2*65536/128.  dQ tile (three
    products, two row-wise and one transposed read) = 1536 and
    2*65536/213 + 65536/128."""
    c = roofline.gradient_tile_cycles_cdna4(128, 64, 128, products=4, row_reads=2, tr_reads=2)
    assert _close(c["mma"], 2048.0) and _close(c["exp"], 291.2) and _close(c["valu"], 825.6)
    assert _close(c["lds"], 2 * 65536 / 213 + 1024.0)
    assert roofline.bound(c)[0] == "mma"
    q = roofline.gradient_tile_cycles_cdna4(128, 64, 128, products=3, row_reads=2, tr_reads=1)
    assert _close(q["mma"], 1536.0) and _close(q["lds"], 2 * 65536 / 213 + 512.0)


def test_cdna4_model_at_b200_rates_is_table1():
    """The CDNA4 forward model with the B200 rates the page states (matrix
    8192 FLOP/clock, 16 exponentials per clock on one unit, 128 bytes per
    clock) and one wavefront per 128 rows reading K and V once each gives
    Table 1's matrix and exponential cycles, 2048 and 2048: the two models
    differ only in the unit rates and the operand reads."""
    b200_like = dict(roofline.MI355X_CU, mma_flops_per_clk=8192.0, simds=1, exp_cycles=64 / 16.0)
    c = roofline.forward_tile_cycles_cdna4(256, 128, 128, row_sum_mfma=False, hw=b200_like)
    assert c["mma"] == 2048.0 and c["exp"] == 2048.0


def test_cdna4_hbm_terms_hand_derived():
    """HBM share per CU: 8e12 / 256 / 2.4e9 = 13.0208 bytes per clock.  dK/dV
    tile of the five-product form writes its dS, 128 x 64 x 2 = 16384 bytes:
    16384 / 13.0208 = 1258.29 cycles, below the 2048 of its products.  The
    dQ = dS K tile (128 query rows, 64 keys, d = 128, 4 waves): mma =
    2*128*64*128/4096 = 512; LDS = 4 waves x (64 x 128 + 64 x 32) x 2 bytes
    = 81920 bytes at half of 128 B/clk = 1280; hbm = 16384 / 13.0208 =
    1258.29: bound by LDS, HBM within 2 %, the products at 40 %.  With 8
    waves the LDS term halves and HBM bounds."""
    assert _close(roofline.hbm_bytes_per_clk(), 8e12 / 256 / 2.4e9)
    g = roofline.gradient_tile_cycles_cdna4(128, 64, 128, products=4, row_reads=2, tr_reads=2, ds_store=True)
    assert _close(g["hbm"], 16384 * 256 * 2.4e9 / 8e12) and _close(g["mma"], 2048.0)
    assert roofline.bound(g)[0] == "mma"
    assert "hbm" not in roofline.gradient_tile_cycles_cdna4(128, 64, 128, products=4, row_reads=2, tr_reads=2)
    c = roofline.ds_product_tile_cycles_cdna4(128, 64, 128)
    assert _close(c["mma"], 512.0) and _close(c["lds"], 1280.0) and _close(c["hbm"], 1258.2912)
    name, frac = roofline.bound(c)
    assert name == "lds" and _close(frac["mma"], 0.4) and _close(frac["hbm"], 1258.2912 / 1280.0)
    c8 = roofline.ds_product_tile_cycles_cdna4(128, 64, 128, waves=8)
    assert _close(c8["lds"], 640.0) and roofline.bound(c8)[0] == "hbm"
    # two wavefronts per 32 rows, half of the dims each: the K tile once per
    # row block, the dS columns twice
    c8h = roofline.ds_product_tile_cycles_cdna4(128, 64, 128, waves=8, d_parts=2)
    assert _close(c8h["lds"], 4 * (64 * 128 + 2 * 64 * 32) * 2 / 128.0) and _close(c8h["lds"], 768.0)
    assert _close(c8h["mma"], 512.0) and roofline.bound(c8h)[0] == "hbm"
    c64 = roofline.ds_product_tile_cycles_cdna4(128, 64, 64)
    assert _close(c64["mma"], 256.0) and _close(c64["lds"], 4 * (64 * 64 + 64 * 32) * 2 / 64.0)
