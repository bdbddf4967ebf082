"""Per-tile cycle model for the attention forward and backward -- test infrastructure.

Method followed: the FA4 paper summary ("FlashAttention-4: Algorithm and
Kernel Pipelining Co-Design for Asymmetric Hardware Scaling"), Key claims:
per-tile roofline of §3.1.1 / Table 1 (forward) and §3.2.1 / Eq. 7-8
(backward).  A tile's time is bounded by the busiest unit: the matrix unit,
the exponential unit and on-chip operand memory (and, on CDNA4, the vector
ALU's issue, which the exponentials share).

B200 per SM, as the pages state them: matrix unit 8192 dense bf16 FLOP per
clock (the divisor in Eq. 7), exponential unit 16 per clock, shared-memory
reads 128 bytes per clock.  Operand-memory reading (ours; it reproduces
Table 1's printed 1536 cycles): each 128-row query tile of the 256-row tile
issues Q K^T with both operands in shared memory and P V with V in shared
memory, so one tile step reads (M/128) * (128 d + 2 N d) bf16 values.

MI355X (gfx950) per compute unit (4 SIMDs).  The matrix rate is AMD's
published figure (2.5 PFLOP/s dense bf16 = 256 CUs x 2.4 GHz x 4096 FLOP per
clock).  The other rates are measured on MI355X by
exact_attention_50_amd/probes/unit_rates.hip (cycles per wavefront-of-64
instruction on one SIMD, enough independent work to reach throughput):
  * v_mfma_f32_32x32x16_bf16 32.1 cycles (4096 FLOP/clock/CU, as published),
    v_mfma_f32_16x16x32_bf16 17.1 cycles;
  * VALU fp32 (fma, add, max3, cvt_pk_bf16): 4.3 cycles per instruction per
    SIMD when two wavefronts issue (one wavefront alone reaches ~6 and, with
    only 8 independent chains, ~9.5: a dependent VALU instruction waits
    ~40 cycles);
  * v_exp_f32: 9.1 cycles per instruction per SIMD (two wavefronts; ~9.7 for
    one) -- the exponential shares the VALU issue;
  * LDS operand reads with 8 wavefronts per CU: ds_read_b128 213 bytes per
    clock per CU, ds_read_b64_tr_b16 (transposed MFMA operands) 128 bytes
    per clock per CU (half of each with 4 wavefronts: the reads are latency
    bound below 8 wavefronts);
  * an MFMA wavefront and a VALU wavefront sharing a SIMD both keep their own
    rate (32.0 and 6.2 cycles), so matrix and vector work overlap;
  * HBM: the published 8 TB/s, 13.02 bytes per clock per CU at 2.4 GHz.
On CDNA4 Q stays in registers (the B operand of S^T = K Q^T); every
wavefront of ``rows_per_wave`` query rows reads the whole K tile row-wise and
the V tile transposed from LDS.
"""

B200_SM = dict(name="B200 SM", mma_flops_per_clk=8192.0, exp_per_clk=16.0,
               smem_bytes_per_clk=128.0)

MI355X_CU = dict(name="MI355X CU", mma_flops_per_clk=4096.0, clock_hz=2.4e9, n_cu=256, simds=4,
                 mfma16_cycles=17.1,          # v_mfma_f32_16x16x32_bf16, per SIMD
                 valu_cycles=4.3,             # fp32 VALU instruction (wave64), per SIMD
                 exp_cycles=9.1,              # v_exp_f32 (wave64), per SIMD
                 lds_row_bytes_per_clk=213.0,     # ds_read_b128, per CU
                 lds_tr_bytes_per_clk=128.0,      # ds_read_b64_tr_b16, per CU
                 hbm_bytes_per_s=8.0e12)          # published HBM3E bandwidth, whole chip


def hbm_bytes_per_clk(hw=MI355X_CU):
    """One CU's share of the HBM bandwidth per clock at the nominal clock."""
    return hw["hbm_bytes_per_s"] / hw["n_cu"] / hw["clock_hz"]


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


def _per_cu(n_instr, cycles_per_instr, hw):
    """CU cycles for n_instr wave64 instructions spread over the CU's SIMDs."""
    return n_instr * cycles_per_instr / hw["simds"]


def forward_tile_cycles_cdna4(M, N, d, rows_per_wave=32, valu_per_score=3.2, row_sum_mfma=True,
                              hw=MI355X_CU, elem_bytes=2):
    """CU cycles of each unit for one (M query rows) x (N keys) forward tile.

    mma    the S^T and P V products, 4 M N d FLOPs, plus (row_sum_mfma) one
           16x16x32 product per 32 rows and 16 keys that sums the bf16 weights;
    exp    one v_exp_f32 per score (M N / 64 instructions);
    valu   valu_per_score other VALU instructions per score (scale-subtract,
           row max, row sum, half a bf16 pack: about 3.2 in the bf16 kernel);
    issue  exp + valu: both go through the VALU issue of the SIMD;
    lds    every wavefront reads the K tile row-wise and the V tile
           transposed: (M / rows_per_wave) N d bytes of each.
    """
    mma = 4.0 * M * N * d / hw["mma_flops_per_clk"]
    if row_sum_mfma:
        mma += _per_cu((M / 32) * (N / 16), hw["mfma16_cycles"], hw)
    exp = _per_cu(M * N / 64, hw["exp_cycles"], hw)
    valu = _per_cu(valu_per_score * M * N / 64, hw["valu_cycles"], hw)
    tile_bytes = (M / rows_per_wave) * N * d * elem_bytes
    lds = tile_bytes / hw["lds_row_bytes_per_clk"] + tile_bytes / hw["lds_tr_bytes_per_clk"]
    return dict(mma=mma, exp=exp, valu=valu, issue=exp + valu, lds=lds)


def gradient_tile_cycles_cdna4(M_own, N_stream, d, products, row_reads, tr_reads, valu_per_elem=6.0,
                               hw=MI355X_CU, elem_bytes=2, ds_store=False):
    """CU cycles of each unit for one tile of a gradient kernel: a workgroup
    owning M_own rows (keys for dK/dV, queries for dQ) against N_stream
    streamed rows, with ``products`` matrix products of 2 M N d FLOPs each
    (4 for dK/dV: S, dP, dV, dK; 3 for dQ: S, dP, dQ), one exponential and
    valu_per_elem other VALU instructions per (own, streamed) pair, and
    row_reads / tr_reads streamed-tile reads per wavefront of 32 own rows
    (row-wise and transposed: Q, dO / K, V read as each kind of operand).
    ds_store (the dK/dV kernel of the five-product form): the tile's dS,
    M N bf16 values, is written to HBM -- hbm = those bytes at the CU's
    share of the HBM bandwidth (the streamed tiles come from L2)."""
    mma = 2.0 * products * M_own * N_stream * d / hw["mma_flops_per_clk"]
    exp = _per_cu(M_own * N_stream / 64, hw["exp_cycles"], hw)
    valu = _per_cu(valu_per_elem * M_own * N_stream / 64, hw["valu_cycles"], hw)
    tile_bytes = (M_own / 32) * N_stream * d * elem_bytes
    lds = (row_reads * tile_bytes / hw["lds_row_bytes_per_clk"]
           + tr_reads * tile_bytes / hw["lds_tr_bytes_per_clk"])
    c = dict(mma=mma, exp=exp, valu=valu, issue=exp + valu, lds=lds)
    if ds_store:
        c["hbm"] = M_own * N_stream * 2 / hbm_bytes_per_clk(hw)
    return c


def ds_product_tile_cycles_cdna4(M_own, N_stream, d, waves=4, d_parts=1, hw=MI355X_CU):
    """CU cycles of each unit for one tile of the dQ = dS K kernel of the
    five-product form: a workgroup of ``waves`` wavefronts owning M_own query
    rows against N_stream keys, each 32 rows taken by ``d_parts`` wavefronts
    with d / d_parts of the dims each.  mma = one product, 2 M N d FLOPs;
    lds = every wavefront reads its share of the K tile transposed
    (N d / d_parts bf16) and its 32 columns of the dS tile transposed
    (N x 32 bf16), at the transposed-read rate, halved below 8 wavefronts
    per CU (the reads are latency bound there); hbm = the dS tile, M N bf16
    values, streamed from HBM once (K is re-read from L2); no exponentials,
    no VALU work to speak of."""
    mma = 2.0 * M_own * N_stream * d / hw["mma_flops_per_clk"]
    tr_bytes = (M_own / 32) * d_parts * (N_stream * d / d_parts + N_stream * 32) * 2
    rate = hw["lds_tr_bytes_per_clk"] * (1.0 if waves >= 8 else 0.5)
    lds = tr_bytes / rate
    hbm = M_own * N_stream * 2 / hbm_bytes_per_clk(hw)
    return dict(mma=mma, exp=0.0, valu=0.0, issue=0.0, lds=lds, hbm=hbm)


def bound(cycles):
    """The unit with the most cycles among mma, issue, lds (and hbm where
    the tile has HBM traffic of its own), and each unit's share of the tile
    time (predicted busy fractions)."""
    units = {k: cycles[k] for k in ("mma", "issue", "lds", "hbm") if k in cycles}
    name = max(units, key=units.get)
    top = units[name]
    return name, {k: v / top for k, v in units.items()}


def peak_bf16_tflops(hw=MI355X_CU):
    """Dense bf16 matrix peak of the whole chip in TFLOP/s."""
    return hw["mma_flops_per_clk"] * hw["n_cu"] * hw["clock_hz"] / 1e12
