"""Per-tile cycle model for the attention forward and backward -- test infrastructure.

Method followed: the FA4 paper summary ("FlashAttention-4: Algorithm and
Kernel Pipelining Co-Design for Asymmetric Hardware Scaling"), Key claims:
per-tile roofline of §3.1.1 / Table 1 (forward) and §3.2.1 / Eq. 7-8
(backward).  The kernel's time per tile is bounded by the busiest of three
units: the matrix unit, the exponential unit and on-chip operand memory.

Hardware constants.  B200 per SM, as the pages state them: matrix unit 8192
dense bf16 FLOP per clock (the divisor in Eq. 7), exponential unit 16 per
clock, shared-memory reads 128 bytes per clock.  MI355X (gfx950) per CU, from
AMD's public figures: 4096 dense bf16 FLOP per clock (2.5 PFLOP/s over 256
CUs at 2.4 GHz); the transcendental rate and LDS bandwidth are parameters
that the microbenchmarks measure.

Operand-memory reading (ours; it reproduces Table 1's printed 1536 cycles):
on B200 each 128-row query tile of the 256-row tile issues Q K^T with both
operands in shared memory and P V with V in shared memory, so one tile step
reads (M/128) * (128 d + 2 N d) bf16 values.  On CDNA4 Q stays in registers
and every wavefront that owns ``rows_per_wave`` query rows reads the whole K
and V tile from LDS: (M / rows_per_wave) * 2 N d bf16 values.
"""

B200_SM = dict(name="B200 SM", mma_flops_per_clk=8192.0, exp_per_clk=16.0,
               smem_bytes_per_clk=128.0)

# MI355X per compute unit.  exp and LDS rates are planning values until
# measured; callers override them with measured numbers.
MI355X_CU = dict(name="MI355X CU", mma_flops_per_clk=4096.0, exp_per_clk=16.0,
                 smem_bytes_per_clk=128.0, clock_hz=2.4e9, n_cu=256)


def forward_tile_cycles_b200(M, N, d, hw=B200_SM, qtile_rows=128, elem_bytes=2):
    """Cycles of the three units for one (M query rows) x (N keys) forward tile."""
    mma = 4.0 * M * N * d / hw["mma_flops_per_clk"]           # QK^T and PV
    exp = 1.0 * M * N / hw["exp_per_clk"]                      # one 2^x per score
    n_qt = M // qtile_rows
    smem_bytes = n_qt * (qtile_rows * d + 2 * N * d) * elem_bytes
    smem = smem_bytes / hw["smem_bytes_per_clk"]
    return dict(mma=mma, exp=exp, smem=smem)


def backward_tile_mma_cycles(M, N, d, hw=B200_SM):
    """Five products of 2*M*N*d FLOPs each: 10 M N d / (FLOP per clock)."""
    return 10.0 * M * N * d / hw["mma_flops_per_clk"]


def forward_tile_cycles_cdna4(M, N, d, rows_per_wave, hw=MI355X_CU,
                              other_valu_per_score=3.0, valu_lanes_per_clk=64.0,
                              elem_bytes=2):
    """Per-CU cycles for one forward tile on CDNA4 (4 SIMDs share the CU).

    other_valu_per_score: non-exp vector ops per score (scale-subtract FMA,
    max, add, half a bf16 pack) at ``valu_lanes_per_clk`` lanes per clock per
    CU (4 SIMDs x 16 lanes).
    """
    mma = 4.0 * M * N * d / hw["mma_flops_per_clk"]
    exp = 1.0 * M * N / hw["exp_per_clk"]
    valu = other_valu_per_score * M * N / valu_lanes_per_clk
    lds_bytes = (M / rows_per_wave) * 2 * N * d * elem_bytes
    lds = lds_bytes / hw["smem_bytes_per_clk"]
    return dict(mma=mma, exp=exp, valu=valu, lds=lds)


def peak_bf16_tflops(hw=MI355X_CU):
    """Dense bf16 matrix peak of the whole chip in TFLOP/s."""
    return hw["mma_flops_per_clk"] * hw["n_cu"] * hw["clock_hz"] / 1e12
