// Fused exact-attention forward with e4m3 (FP8) operands, for gfx950.
//
// The method is that of the bf16 forward (FlashAttention-4 paper as
// summarised on "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design
// for Asymmetric Hardware Scaling", Method: online softmax over key tiles,
// conditional rescaling of the running output while the row max grows by at
// most tau, one division by the row sum at the end); the summary's precision
// discussion names FP8 as the next operand format.  Here Q, K and V arrive as
// e4m3 bytes with one dequantisation factor per tensor:
//   S = (scale * q_descale * k_descale) * Q8 K8^T        (fp32 accumulation)
//   P = 2^(S log2(e) - m_ref), rounded to e4m3 (P <= 2^tau <= 256 < 448)
//   O = v_descale * (P8 V8) / l,  l = sum of the fp32 P (before rounding)
// where each descale is the per-tensor factor times, optionally, a factor
// of the (batch, head) slice.
//   LSE from the fp32 scores and l, as in the bf16 forward.
//
// CDNA4 mapping (ours): the 256-row workgroup, the two wave groups alternating
// matrix and softmax phases, and the 2-stage K and V rings of 128-key tiles of
// the bf16 forward, with
//   * products v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3, scales 1): A and
//     B lanes hold 32 consecutive k (lane l: row l % 32, k 32 (l / 32) .. +31);
//     the C layout is the bf16 32x32 one, so the softmax code is unchanged;
//   * e4m3 tiles of 128 keys x 128 bytes; the 16-byte chunk c of K row r sits
//     at chunk position c ^ ((r >> 1) & 7), so 16 consecutive rows read at one
//     chunk meet 16 distinct 16-byte bank slots; V rows have a permutation of
//     their own that suits the rows a transposed read touches (swzv);
//   * S^T = K Q^T: K is the A operand (two 16-byte reads of one row), Q^T the
//     B operand in registers;
//   * O^T += V^T P^T per 64 keys: P^T (B operand) is two S^T accumulators
//     rounded to e4m3, so lane (r, g) holds the keys
//     32 (j / 16) + 8 ((j % 16) / 4) + 4 g + j % 4 at k-slot 32 g + j; the V^T A
//     operand follows that order through ds_read_b64_tr_b8, which gives lane i
//     of a 16-lane group byte i % 8 of the 8-byte chunks addressed by lanes
//     2 m + i / 8 (m = 0..7): the even lanes address dims 0-7 and the odd
//     lanes dims 8-15 of the same 8 keys, four reads give the 32 k-slots.

#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_tiles.hpp"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves8 = 8;
constexpr int kThreads8 = kWaves8 * 64;
constexpr int kQW8 = 32;                 // query rows per wave
constexpr int kBM8 = kWaves8 * kQW8;     // query rows per workgroup
constexpr int kBN8 = 128;                // keys per tile
constexpr int kD8 = 128;                 // head dimension = bytes per row
constexpr int kTile8 = kBN8 * kD8;       // 16 KiB
constexpr int kRing8 = 4 * kTile8;       // K stages 0, 1 then V stages 0, 1
constexpr int kLds8 = kRing8 > kWaves8 * RowStore<kD8>::kBytes ? kRing8 : kWaves8 * RowStore<kD8>::kBytes;
static_assert(2 * (kTile8 / 2 + kBN8 * 4) + 2 * kTile8 <= kLds8, "MXFP4 ring exceeds the LDS allocation");
constexpr int kAhead8 = 2;               // operands in flight per wave (64-cycle products)

struct Fwd8Params {
  const uint8_t* q;      // e4m3 [BH, Sq, 128], or MXFP4 elements [BH, Sq, 64]
  const uint8_t* k;      // e4m3 [BH, Sk, 128], or MXFP4 elements [BH, Sk, 64]
  const uint8_t* v;
  const uint8_t* qsc;    // MXFP4 only: E8M0 scales [BH, Sq, 4] and [BH, Sk, 4]
  const uint8_t* ksc;
  bf16* o;
  float* lse;
  int BH, Sq, Sk, n_qblocks;
  int paired;        // causal, n_qblocks even: workgroup (r, bh) runs ranks r and n_qblocks - 1 - r
  float s_log2;      // scale * q_descale * k_descale * log2(e) (MXFP4: scale * log2(e))
  float v_descale;
  const float* hd;   // null, or per-slice factors [3][BH] (q, k, v)
  float tau;
  // BS: per-block factors [BH][nqb], [BH][nkb], [BH][nkb] (128-row blocks)
  const float* qbs;
  const float* kbs;
  const float* vbs;
  int nqb, nkb;
};

// the 16-byte chunk c of K tile row r sits at byte r * kD8 + 16 * (c ^ swz8(r)):
// the 16 consecutive rows one 16-byte read instruction meets at chunk c land
// on 16 distinct 16-byte bank slots (even and odd rows fall in opposite
// halves of the 64 banks, and (r >> 1) & 7 spreads each half's 8 rows)
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
// V tiles: chunk c of row r at c ^ swzv(r).  A V^T read's 32 lanes of one
// pass address rows r0, r0 + 2, r0 + 8, r0 + 10 of each parity (r0 in
// {0, 1, 4, 5} + 16 k), two 16-byte chunks 2 db, 2 db + 1 each; row bits 1
// and 3 select the chunk pair, so the four rows of a parity cover the 8 bank
// slots of their half once (swz8 maps them to two pairs: a 2-way conflict)
__device__ __forceinline__ int swzv(int r) { return (r & 2) | ((r >> 1) & 4); }
// d = 64: 64-byte rows, four to a 256-byte bank line.  K chunk c of row r at
// c ^ swz64(r): the four rows of a read pass that share a line (r, r + 4,
// r + 8, r + 12) take distinct chunks.  V at c ^ swzv64(r): a transposed
// read pass touches rows r0 + i and r0 + 8 + i (i < 4) that share a line,
// two chunks each, so row bit 3 picks the chunk pair.
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swzv64(int r) { return (r >> 2) & 2; }
template <int D8>
__device__ __forceinline__ int k_swz(int r) { return D8 == 128 ? swz8(r) : swz64(r); }
template <int D8>
__device__ __forceinline__ int v_swz(int r) { return D8 == 128 ? swzv(r) : swzv64(r); }

// e4m3 x e4m3 products written out as single instructions (the compiler
// moves its own form of this product past barriers to the first use of the
// result, which keeps every operand of a phase live at once).  The code
// around them owns two latencies: the s_nop 1 in front covers a VALU write of
// an operand just before, and drain8() (24 wait states, tied to the
// accumulators) separates the last product of a phase from VALU reads.
__device__ __forceinline__ void mfma8_acc(f32x16& d, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

__device__ __forceinline__ void mfma8_init(f32x16& d, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void drain8(f32x16& a, f32x16& b, f32x16& c, f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void drain8(f32x16& a, f32x16& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

// MXFP4 x MXFP4 products (E2M1 elements, 4 VGPRs per operand) with E8M0
// block scales: v_mfma_scale_f32_32x32x64_f8f6f4 with cbsz = blgp = 4 (both
// operands E2M1).  Lane l's 32 elements (k = 32 (l / 32) .. +31 of the 64)
// are one microscaling block; each scale operand holds the lanes' scale bytes
// of k-step kc in byte kc, selected by op_sel (low bit of the byte index) and
// op_sel_hi (high bit).  Checked on MI355X against a float64 product of
// random E2M1 codes with random per-lane scales.  The same hazards as
// mfma8_acc; drain8() covers these products too.
// k-step 1 (byte 1 of each scale operand), accumulating
__device__ __forceinline__ void mfma4_acc1(f32x16& d, const i32x4& a, const i32x4& b, uint32_t sa, uint32_t sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,1,0] op_sel_hi:[0,0,0] cbsz:4 blgp:4"
               : "+v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// k-step 0 (byte 0), from zero
__device__ __forceinline__ void mfma4_init(f32x16& d, const i32x4& a, const i32x4& b, uint32_t sa, uint32_t sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
               : "=&v"(d) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// MXFP4 K tiles: 128 rows of 64 bytes (128 E2M1 elements), the 16-byte chunk
// c of row r at byte r * 64 + 16 * (c ^ swz4(r)), so 16 consecutive rows read
// at one chunk meet 16 distinct 16-byte bank slots; then the rows' E8M0
// scale dwords (4 blocks of 32 dims each), 128 x 4 bytes.
constexpr int kRow4 = kD8 / 2;                 // bytes per MXFP4 row
constexpr int kTileK4 = kBN8 * kRow4;          // 8 KiB
constexpr int kStageK4 = kTileK4 + kBN8 * 4;   // + scale dwords
__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

// The lane's scale bytes for the two 64-dim k-steps (byte kc = block 2 kc + g,
// g = lane / 32) out of a row's 4 scale bytes.
__device__ __forceinline__ uint32_t scale_pair(uint32_t row_scales, int g) {
  return __builtin_amdgcn_perm(0u, row_scales, g ? 0x0c0c0301u : 0x0c0c0200u);
}

// k-slot j of lane group g (0, 1) -> key of the 64-key step
__device__ __forceinline__ int slot_key(int g, int j) { return 32 * (j / 16) + 8 * ((j % 16) / 4) + 4 * g + (j % 4); }

// a tile of 128 rows of D8 bytes, memory-to-LDS with the chunk permutation
// (K or V): one 16-byte load per lane covers 1024 / D8 whole rows (8 at
// d = 128, 16 at d = 64); the waves share the tile's loads
template <int D8, bool V_TILE>
__device__ __forceinline__ void dma_tile8(__amdgpu_buffer_rsrc_t src, int row0, char* tile, int wave, int lane) {
  constexpr int kLanesPerRow = D8 / 16, kRowsPerLoad = 64 / kLanesPerRow;
  static_assert(kBN8 % (kRowsPerLoad * kWaves8) == 0, "the waves share the loads evenly");
#pragma unroll
  for (int i = 0; i < kBN8 / kRowsPerLoad / kWaves8; ++i) {
    const int blk = i * kWaves8 + wave;   // wave-uniform
    const int row = blk * kRowsPerLoad + lane / kLanesPerRow;
    const int sw = V_TILE ? v_swz<D8>(row) : k_swz<D8>(row);
    const unsigned off = (unsigned)(row0 + row) * D8 + 16 * ((lane % kLanesPerRow) ^ sw);
    lds_dma16(src, off, tile + blk * kRowsPerLoad * D8);
  }
}

// an MXFP4 K tile memory-to-LDS: one 16-byte load per lane covers 16 rows
// (each wave one of the 8), then the scale dwords of its 128 rows (waves 0
// and 1, 64 rows each)
__device__ __forceinline__ void dma_tile4(__amdgpu_buffer_rsrc_t src, __amdgpu_buffer_rsrc_t ssrc, int row0, char* tile,
                                          int wave, int lane) {
  const int blk = wave;   // wave-uniform
  const int row = blk * 16 + lane / 4;
  const unsigned off = (unsigned)(row0 + row) * kRow4 + 16 * ((lane % 4) ^ swz4(row));
  lds_dma16(src, off, tile + blk * 16 * kRow4);
  if (wave < 2) lds_dma4(ssrc, (unsigned)(row0 + 64 * wave + lane) * 4, tile + kTileK4 + 64 * wave * 4);
}

// FP4QK: Q and K in MXFP4 (S^T on the scaled fp4 products), V and P in e4m3.
// BS: one dequantisation factor per 128-row block of Q, K and V: Q's folds
// into the wave's score factor (a wave's 32 rows lie in one block), K's into
// the tile's (a 128-key tile is one block); V's enters the exponent: the tile
// rounds r P to e4m3, r = its V factor / the head's largest, sums P itself
// for the row sum (the tile's partial sums times 1 / r), and the epilogue
// multiplies O by the largest factor.
template <bool CAUSAL, bool FP4QK, bool BS, int D8>
__device__ __forceinline__ void fwd8_block(const Fwd8Params& p, const int rank, const int bh) {
  static_assert(!(FP4QK && BS), "block factors are for the e4m3 operands");
  static_assert(D8 == 128 || (D8 == 64 && !FP4QK), "head dimension 128, or 64 with e4m3 operands");
  constexpr int kTileD = kBN8 * D8;   // bytes of an e4m3 K or V tile
  static_assert(kBN8 == kFp8ScaleBlock && kFp8ScaleBlock % kQW8 == 0, "a tile is one K / V block, a wave in one Q block");
  constexpr int kKB = kBN8 / 32;   // 32-key blocks of S^T per tile
  constexpr int kKC = D8 / 64;    // 64-dim steps of S^T
  constexpr int kKS = kBN8 / 64;   // 64-key steps of P V
  constexpr int kDB = D8 / 32;    // 32-dim blocks of O^T
  constexpr int kNV = kKS * kDB;   // P V products per tile
  constexpr int kNK = kKB * kKC;   // K Q^T products per tile
  extern __shared__ __attribute__((aligned(16))) char smem[];

  // opaque per block, so that nothing derived from the lane index is hoisted
  // out of the paired launch's loop and held live across a whole block
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  float s_log2 = p.s_log2, v_descale = p.v_descale;
  if (p.hd) {
    s_log2 *= p.hd[bh] * p.hd[p.BH + bh];
    v_descale *= p.hd[2 * p.BH + bh];
  }
  const int qb = CAUSAL ? (p.n_qblocks - 1 - rank) : rank;
  constexpr int kRowQK = FP4QK ? kRow4 : D8;   // bytes per Q / K row
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)bh * p.Sq * kRowQK, (unsigned)p.Sq * kRowQK);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (size_t)bh * p.Sk * kRowQK, (unsigned)p.Sk * kRowQK);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (size_t)bh * p.Sk * D8, (unsigned)p.Sk * D8);

  const int q_wave_lo = qb * kBM8 + wave * kQW8;
  const int q_lane = q_wave_lo + r32;

  // block factors: the wave's Q block into the score factor; the head's
  // largest V factor (each lane takes every 64th block, then a wave max).
  // Per tile the vector phase needs the tile's score factor and log2 r: lane
  // l holds those of tile w0 + l of a 64-tile window (refilled every 64
  // tiles), read per tile with readlane, so no tile waits on a memory load
  // (a vector-memory wait would also wait for the tile loads in flight).
  const float* kbs_head = BS ? p.kbs + (size_t)bh * p.nkb : nullptr;
  const float* vbs_head = BS ? p.vbs + (size_t)bh * p.nkb : nullptr;
  float inv_vmax = 1.0f, c_win = 0.0f, lr_win = 0.0f;
  auto fill_window = [&](int w0) __attribute__((always_inline)) {
    const int b = min(w0 + lane, p.nkb - 1);
    c_win = s_log2 * kbs_head[b];
    lr_win = __builtin_amdgcn_logf(vbs_head[b] * inv_vmax);
  };
  if constexpr (BS) {
    s_log2 *= p.qbs[(size_t)bh * p.nqb + min(q_wave_lo / kFp8ScaleBlock, p.nqb - 1)];
    float vmax = 0.0f;
    for (int b = lane; b < p.nkb; b += 64) vmax = __builtin_fmaxf(vmax, vbs_head[b]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) vmax = __builtin_fmaxf(vmax, __shfl_xor(vmax, off));
    v_descale = vmax;
    inv_vmax = 1.0f / vmax;
    fill_window(0);
  }

  // Q^T operand, k-step kc: lane holds Q[q_lane][64 kc + 32 g .. +31]
  i32x8 qf[kKC];
  // MXFP4: lane holds the 32 elements Q[q_lane][64 kc + 32 g .. +31] (16
  // bytes) per k-step, and the scale bytes of those blocks (byte kc)
  i32x4 qf4[kKC];
  uint32_t q_sc = 0;
  __amdgpu_buffer_rsrc_t rks = rk;
  if constexpr (FP4QK) {
#pragma unroll
    for (int kc = 0; kc < kKC; ++kc)
      qf4[kc] = __builtin_bit_cast(i32x4, load16(rq, (unsigned)q_lane * kRow4 + 32 * kc + 16 * g));
    const __amdgpu_buffer_rsrc_t rqs = make_rsrc(p.qsc + (size_t)bh * p.Sq * 4, (unsigned)p.Sq * 4);
    const uint32_t qrow = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rqs, (int)((unsigned)q_lane * 4), 0, 0);
    q_sc = scale_pair(qrow, g);
    rks = make_rsrc(p.ksc + (size_t)bh * p.Sk * 4, (unsigned)p.Sk * 4);
  } else {
#pragma unroll
    for (int kc = 0; kc < kKC; ++kc) {
      qf[kc].lo = __builtin_bit_cast(i32x4, load16(rq, (unsigned)q_lane * D8 + 64 * kc + 32 * g));
      qf[kc].hi = __builtin_bit_cast(i32x4, load16(rq, (unsigned)q_lane * D8 + 64 * kc + 32 * g + 16));
    }
  }

  // K operand addresses: row 32 kb + r32 has the chunk permutation of r32
  const int k_sw = k_swz<D8>(r32);
  const int k_row = r32 * D8;
  // V^T operand addresses: read q of a 64-key step; this lane, as a source
  // lane of its 16-lane group, addresses the key of k-slot 8 q + m (m = (lane
  // % 16) / 2) and the dims 32 db + 16 half + 8 par .. +7 (half = group of
  // 16 lanes within the wave half, par = lane parity)
  const int par = lane & 1;
  const int m8 = (lane & 15) >> 1;
  const int half = (lane >> 4) & 1;
  // offset of read q, dims 32 db + ..: row slot_key(g, 8 q + m8) (the key of
  // step ks adds 64 rows, which keeps the permutation), chunk 2 db + half,
  // with the chunk permutation split into its half and db bits; the 16
  // offsets (and the 4 of the K reads) are formed once per lane, so a read
  // costs one add of the stage base
  int v_off[4][kDB];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = slot_key(g, 8 * q + m8);
    const int sw = v_swz<D8>(row);
#pragma unroll
    for (int db = 0; db < kDB; ++db)
      v_off[q][db] = row * D8 + 8 * par + 16 * (half ^ (sw & 1)) + ((32 * db) ^ (32 * (sw >> 1)));
  }
  // K operand reads: 16-byte chunk 4 kc + 2 g + h of row r32, swizzled
  int k_off[kKC][2];
#pragma unroll
  for (int kc = 0; kc < kKC; ++kc)
#pragma unroll
    for (int h = 0; h < 2; ++h) k_off[kc][h] = k_row + 16 * ((4 * kc + 2 * g + h) ^ k_sw);

  const int kv_end = CAUSAL ? min(p.Sk, (qb + 1) * kBM8) : p.Sk;
  const int n = (kv_end + kBN8 - 1) / kBN8;
  int n_wave = CAUSAL ? max(1, min(n, (q_wave_lo + kQW8 + kBN8 - 1) / kBN8)) : n;
  if (CAUSAL) asm volatile("" : "+s"(n_wave));

  f32x16 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x16{};
  f32x16 s[kKB];
  i32x8 pk[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) pk[ks] = i32x8{};
  float m_ref = kNegInf;
  float l_part[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  // LDS ring: K stages 0, 1 then V stages 0, 1 (MXFP4 K stages are half a
  // tile plus the scale dwords)
  constexpr int kStageK = FP4QK ? kStageK4 : kTileD;
  auto k_stage = [&](int u) __attribute__((always_inline)) -> char* { return smem + (u & 1) * kStageK; };
  auto v_stage = [&](int u) __attribute__((always_inline)) -> char* {
    return smem + 2 * kStageK + (u & 1) * kTileD;
  };
  // MXFP4 K operand: row 32 kb + r32, bytes 32 kc + 16 g .. +15 (chunk 2 kc + g)
  int k4_off[2];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) k4_off[kc] = r32 * kRow4 + 16 * ((2 * kc + g) ^ swz4(r32));

  // ---- matrix phase: O^T += V^T P^T of tile uv, then S^T = K Q^T of tile uk
  auto matrix_stream_body = [&](int uk, int uv, auto with_pv, auto with_s) __attribute__((always_inline)) {
    constexpr bool PV = decltype(with_pv)::value;
    constexpr bool SK = decltype(with_s)::value;
    constexpr int j0 = PV ? 0 : kNV;
    constexpr int j1 = SK ? kNV + kNK : kNV;
    const char* vst = v_stage(uv);
    const char* kst = k_stage(uk);
    // j < kNV: (ks, db) = (j / kDB, j % kDB); else (kb, kc) = (i % kKB, i / kKB), i = j - kNV
    auto operand = [&](int j) __attribute__((always_inline)) -> i32x8 {
      if (j < kNV) {
        const int ks = j / kDB, db = j % kDB;
        i32x8 r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const char* a = vst + ks * 64 * D8 + v_off[q][db];
          const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(lds_addr(a)));
          r[2 * q] = t[0];
          r[2 * q + 1] = t[1];
        }
        return r;
      }
      const int i = j - kNV;
      const int kb = i % kKB, kc = i / kKB;
      i32x8 r;
      if constexpr (FP4QK) {
        // 16 bytes (32 elements) per lane; the upper half of the ring entry is unused
        r.lo = *reinterpret_cast<const i32x4*>(kst + kb * 32 * kRow4 + k4_off[kc]);
      } else {
        const char* row = kst + kb * 32 * D8;
        r.lo = *reinterpret_cast<const i32x4*>(row + k_off[kc][0]);
        r.hi = *reinterpret_cast<const i32x4*>(row + k_off[kc][1]);
      }
      return r;
    };
    // MXFP4: the scale bytes of the K rows of each 32-key block (byte kc = the
    // lane's block of k-step kc)
    uint32_t k_sc[kKB];
    if constexpr (FP4QK && SK) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
        k_sc[kb] = scale_pair(*reinterpret_cast<const uint32_t*>(kst + kTileK4 + (32 * kb + r32) * 4), g);
    }
    i32x8 ring[kAhead8];
#pragma unroll
    for (int j = j0; j < j0 + kAhead8 && j < j1; ++j) ring[(j - j0) % kAhead8] = operand(j);
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const i32x8 a = ring[(j - j0) % kAhead8];
      if (j + kAhead8 < j1) ring[(j - j0) % kAhead8] = operand(j + kAhead8);
      if (j < kNV) {
        mfma8_acc(o[j % kDB], a, pk[j / kDB]);
      } else {
        const int i = j - kNV;   // the first k-step starts each accumulator
        if constexpr (FP4QK) {
          if (i < kKB)
            mfma4_init(s[i % kKB], a.lo, qf4[0], k_sc[i % kKB], q_sc);
          else
            mfma4_acc1(s[i % kKB], a.lo, qf4[1], k_sc[i % kKB], q_sc);
        } else {
          if (i < kKB)
            mfma8_init(s[i % kKB], a, qf[i / kKB]);
          else
            mfma8_acc(s[i % kKB], a, qf[i / kKB]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PV) {
      if constexpr (kDB == 4) drain8(o[0], o[1], o[2], o[3]);
      else drain8(o[0], o[1]);
    }
    if (SK) drain8(s[0], s[1], s[2], s[3]);
  };
  auto matrix_stream = [&](int uk, int uv, auto with_pv, auto with_s) __attribute__((always_inline)) {
    matrix_stream_body(uk, uv, with_pv, with_s);
  };
  auto matrix_s = [&](int t) __attribute__((always_inline)) {
    matrix_stream(t, 0, std::false_type{}, std::true_type{});
  };
  auto matrix_full = [&](int t) __attribute__((always_inline)) {
    matrix_stream(t, t - 1, std::true_type{}, std::true_type{});
  };
  auto matrix_pv = [&](int t) __attribute__((always_inline)) {
    matrix_stream(0, t - 1, std::true_type{}, std::false_type{});
  };

  // ---- vector phase: softmax of tile t, P rounded to e4m3
  auto vector = [&](int t) __attribute__((always_inline)) {
    if (t >= n_wave) return;
    // with e4m3 products the softmax's VALU work is the longer phase, so it
    // (not the matrix phase, as in the bf16 kernel) gets the raised priority
    __builtin_amdgcn_s_setprio(2);
    const int k0 = t * kBN8;
    const bool need_mask = (k0 + kBN8 > p.Sk) || (CAUSAL && k0 + kBN8 - 1 > q_wave_lo);
    if (need_mask) {
      const int last = CAUSAL ? min(p.Sk - 1, q_lane) : p.Sk - 1;
      softmax_mask_prefix<kKB>(s, last - k0 - 4 * g);
    }
    const float mx = softmax_row_max<kKB>(s);
    // the tile's score factor (BS: times its K block's factor)
    float c_t = s_log2, log2_r = 0.0f;
    if constexpr (BS) {
      if ((t & 63) == 0 && t > 0) fill_window(t);
      c_t = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c_win), t & 63));
      log2_r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lr_win), t & 63));
    }
    softmax_conditional_rescale(m_ref, mx * c_t, p.tau, [&](float alpha) {
#pragma unroll
      for (int c = 0; c < 4; ++c) l_part[c] *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db) o[db] *= alpha;
    });
    if constexpr (BS) {
      // P' = r P = 2^(s c - (m_ref - log2 r)), r = V factor / the largest (<= 1);
      // the partial sums go back by 2^-log2 r, the same factor P' carries
      float l_tile[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      softmax_exp_rowsum<kKB, 0>(s, c_t, m_ref - log2_r, l_tile);
      const float inv_r = __builtin_amdgcn_exp2f(-log2_r);
#pragma unroll
      for (int c = 0; c < 4; ++c) l_part[c] = __builtin_fmaf(l_tile[c], inv_r, l_part[c]);
    } else {
      softmax_exp_rowsum<kKB, 0>(s, c_t, m_ref, l_part);
    }
    // P^T operand of 64-key step ks: bytes j = 0..31 are s[2 ks + j / 16][j % 16]
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = 2 * ks + w / 4, i0 = 4 * (w % 4);
        // the first conversion keeps the upper half of its destination, which
        // the second one overwrites: pass the stale value rather than a zero
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][i0], s[kb][i0 + 1], pk[ks][w], false);
        d = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][i0 + 2], s[kb][i0 + 3], d, true);
        pk[ks][w] = d;
      }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- tile IO: interval 2u-1 issues K_u and V_{u-1}; the end of every even
  // interval waits for them (the schedule of the bf16 256-row form)
  auto fetch = [&](int u) __attribute__((always_inline)) {
    if (u < n) {
      if constexpr (FP4QK) dma_tile4(rk, rks, u * kBN8, k_stage(u), wave, lane);
      else dma_tile8<D8, false>(rk, u * kBN8, k_stage(u), wave, lane);
    }
    if (u >= 1 && u <= n) dma_tile8<D8, true>(rv, (u - 1) * kBN8, v_stage(u - 1), wave, lane);
  };
  auto commit = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  fetch(0);
  commit();
  barrier();
  if (group == 0) {
    fetch(1);
    matrix_s(0);
    barrier();
    vector(0);
    commit();
    barrier();
    for (int t = 1; t < n_wave; ++t) {
      fetch(t + 1);
      matrix_full(t);
      barrier();
      vector(t);
      commit();
      barrier();
    }
    // the last P V (tile n_wave - 1) has one call site, so the accumulators
    // are never merged across branches (the products are asm the compiler
    // cannot see the latency of: a merge copy right after one would read a
    // result not yet written); with n_wave = n, fetch(n + 1) loads nothing
    fetch(n_wave + 1);
    matrix_pv(n_wave);
    barrier();
    if (n_wave < n) {
      commit();
      barrier();
      for (int t = n_wave + 1; t < n; ++t) {
        fetch(t + 1);
        barrier();
        commit();
        barrier();
      }
      barrier();
    }
    barrier();
  } else {
    fetch(1);
    barrier();
    matrix_s(0);
    commit();
    barrier();
    fetch(2);
    vector(0);
    barrier();
    for (int t = 1; t < n_wave; ++t) {
      matrix_full(t);
      commit();
      barrier();
      fetch(t + 2);
      vector(t);
      barrier();
    }
    matrix_pv(n_wave);
    commit();
    barrier();
    if (n_wave < n) {
      fetch(n_wave + 2);
      barrier();
      for (int t = n_wave + 1; t < n; ++t) {
        commit();
        barrier();
        fetch(t + 2);
        barrier();
      }
      barrier();
    }
  }

  // ---- epilogue: O = v_descale O / l as bf16 rows, LSE = (m_ref + log2 l) ln 2
  const float l = pair_sum((l_part[0] + l_part[1]) + (l_part[2] + l_part[3]));
  const float inv_l = l > 0.0f ? v_descale / l : 0.0f;
  RowStore<D8>::store(smem + wave * RowStore<D8>::kBytes, o, inv_l, p.o + (size_t)bh * p.Sq * D8, q_wave_lo,
                       p.Sq, lane);
  if (q_lane < p.Sq && g == 0) p.lse[(size_t)bh * p.Sq + q_lane] = (m_ref + __builtin_log2f(l)) * kLn2;
}

// One query block per workgroup, heaviest causal blocks first; or, paired,
// workgroup (r, bh) runs rank r and then rank n_qblocks - 1 - r of the same
// head (equal causal work per workgroup, no new workgroup between the two
// blocks).  Between them every wave's loads, stores and LDS reads have
// completed.
template <bool CAUSAL, bool FP4QK = false, bool BS = false, int D8 = 128>
__global__ __launch_bounds__(kThreads8, 1) void fwd8_kernel(Fwd8Params p) {
  const int r = blockIdx.x / p.BH, bh = blockIdx.x % p.BH;
  int n_it = p.paired ? 2 : 1;
  asm volatile("" : "+s"(n_it));
#pragma unroll 1
  for (int it = 0; it < n_it; ++it) {
    if (it > 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    fwd8_block<CAUSAL, FP4QK, BS, D8>(p, it == 0 ? r : p.n_qblocks - 1 - r, bh);
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdFp8Args& a, hipStream_t stream) {
  Fwd8Params prm;
  prm.q = static_cast<const uint8_t*>(a.q);
  prm.k = static_cast<const uint8_t*>(a.k);
  prm.v = static_cast<const uint8_t*>(a.v);
  prm.o = static_cast<bf16*>(a.o);
  prm.lse = a.lse;
  prm.BH = a.B * a.H;
  prm.Sq = a.Sq;
  prm.Sk = a.Sk;
  prm.n_qblocks = (a.Sq + kBM8 - 1) / kBM8;
  prm.s_log2 = a.scale * a.q_descale * a.k_descale * kLog2e;
  prm.v_descale = a.v_descale;
  prm.hd = a.head_descales;
  prm.tau = a.tau;
  prm.qbs = a.q_blocks;
  prm.kbs = a.k_blocks;
  prm.vbs = a.v_blocks;
  prm.nqb = (a.Sq + kFp8ScaleBlock - 1) / kFp8ScaleBlock;
  prm.nkb = (a.Sk + kFp8ScaleBlock - 1) / kFp8ScaleBlock;
  const bool bs = a.q_blocks != nullptr;
  const bool d64 = a.d == 64;
  if (bs) {   // the block factors replace the per-tensor and per-slice ones
    prm.s_log2 = a.scale * kLog2e;
    prm.v_descale = 1.0f;
    prm.hd = nullptr;
  }
  prm.paired = (a.causal && prm.n_qblocks % 2 == 0) ? 1 : 0;
  const dim3 grid((unsigned)((prm.paired ? prm.n_qblocks / 2 : prm.n_qblocks) * prm.BH));
  auto run = [&](auto kern) -> hipError_t {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds8);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads8), kLds8, stream, prm);
    return hipGetLastError();
  };
  if (d64) {
    if (bs) return a.causal ? run(fwd8_kernel<true, false, true, 64>) : run(fwd8_kernel<false, false, true, 64>);
    return a.causal ? run(fwd8_kernel<true, false, false, 64>) : run(fwd8_kernel<false, false, false, 64>);
  }
  if (bs) return a.causal ? run(fwd8_kernel<true, false, true>) : run(fwd8_kernel<false, false, true>);
  return a.causal ? run(fwd8_kernel<true>) : run(fwd8_kernel<false>);
}

hipError_t launch_fwd_mxfp4(const FwdFp8Args& a, hipStream_t stream) {
  Fwd8Params prm;
  prm.q = static_cast<const uint8_t*>(a.q);
  prm.k = static_cast<const uint8_t*>(a.k);
  prm.v = static_cast<const uint8_t*>(a.v);
  prm.qsc = static_cast<const uint8_t*>(a.q_scales);
  prm.ksc = static_cast<const uint8_t*>(a.k_scales);
  prm.o = static_cast<bf16*>(a.o);
  prm.lse = a.lse;
  prm.BH = a.B * a.H;
  prm.Sq = a.Sq;
  prm.Sk = a.Sk;
  prm.n_qblocks = (a.Sq + kBM8 - 1) / kBM8;
  prm.s_log2 = a.scale * kLog2e;
  prm.v_descale = a.v_descale;
  prm.hd = nullptr;
  prm.tau = a.tau;
  prm.qbs = prm.kbs = prm.vbs = nullptr;
  prm.nqb = prm.nkb = 0;
  prm.paired = (a.causal && prm.n_qblocks % 2 == 0) ? 1 : 0;
  const dim3 grid((unsigned)((prm.paired ? prm.n_qblocks / 2 : prm.n_qblocks) * prm.BH));
  auto run = [&](auto kern) -> hipError_t {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds8);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads8), kLds8, stream, prm);
    return hipGetLastError();
  };
  return a.causal ? run(fwd8_kernel<true, true>) : run(fwd8_kernel<false, true>);
}

}  // namespace fa
