// Fused exact-attention forward for gfx950.
//
// Method (FlashAttention-4 paper as summarised on "FlashAttention-4: Algorithm
// and Kernel Pipelining Co-Design for Asymmetric Hardware Scaling", Method):
// keys and values are streamed tile by tile; each query row keeps a running
// output, a running row sum and a reference max; the correction of the
// running output is applied only when the row max has grown by more than tau
// (log2 units) over the reference (paper §3.1.4, Eq. 6), gated per wavefront;
// a fixed share of the exponentials is computed by the software 2^x (paper
// §3.1.3); the output is divided by the row sum once at the end, which makes
// the result exact.
//
// CDNA4 mapping (ours, not the pages'):
//   * workgroup = 8 wavefronts x 32 query rows = 256 rows, one per CU; grid
//     over (query block, head, batch), heaviest causal blocks first.  A
//     causal grid of fewer than two such blocks per CU is split instead:
//     128-row workgroups whose two wave groups take alternate key tiles of
//     the same rows and merge their partial (O, row sum, max) at the end, so
//     heavy and light blocks can share the CUs;
//   * ping-pong: waves 0-3 and 4-7 form two groups with one wave of each on
//     every SIMD; the groups alternate between a matrix phase (O += V P of
//     the previous tile, then S of the next tile) and a vector phase (the
//     softmax of that tile), one workgroup barrier per phase, so one SIMD's
//     matrix core works for one wave while the other wave runs its softmax
//     (the role split that the pages give to separate warpgroups);
//   * S is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     Q^T is the B operand kept in registers, K the A operand from LDS; each
//     lane owns 16 scores of ONE query per 32-key block, so the row max / sum
//     need one v_permlane32_swap between the wave halves;
//   * O^T = V^T P^T: the S^T accumulator, rounded to bf16, is already the B
//     operand (keys of each 16-key group in a fixed permuted order); the V^T
//     A operand is read from row-major V in LDS with ds_read_b64_tr_b16;
//   * K / V tiles with the chunk permutation of fa_tiles.hpp (bank-conflict-
//     free operand reads): the 256-row form streams 128-key tiles through a
//     2-stage K ring and a 2-stage V ring, the split form 64-key tiles
//     through a 5-stage K+V ring, both loaded memory-to-LDS two intervals
//     ahead of their first read; buffer descriptors bound every head, so rows
//     past the end read zeros;
//   * the bf16 output leaves through a per-wave LDS area as whole rows.

#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_tiles.hpp"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;               // query rows per wavefront
constexpr int kBM = kWaves * kQW;     // query rows per workgroup
// keys per tile: 128 in the 256-row form (two 2-stage rings, K and V), 64 in
// the split form (one 5-stage ring of K+V stages)
constexpr int kBNFull = 128;
constexpr int kBNSplit = 64;
constexpr int kStages = 5;            // split form (5 x 32 KB = all 160 KB of LDS at d = 128)

struct FwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;           // bf16 output, or
  float* o32;        // float32 output when non-null
  float* lse;
  int BH;            // B * H
  int Sq, Sk;        // rows per head of Q / O and of K / V
  int k_begin;       // the keys attended to: k_begin .. k_begin + k_len - 1
  int k_len;
  int q_off;         // global index of query row 0 (causal: key j visible iff k_begin + j <= q_off + i)
  int n_qblocks;
  int paired;        // causal, n_qblocks even: workgroup (r, bh) runs ranks r and n_qblocks - 1 - r
  float scale_log2;  // scale * log2(e)
  float tau;
  unsigned* events;  // counting instantiation: corrections per (b, h, 32-row slot), added to
};

// LDS of the 256-row form: K ring of 2 stages, then V ring of 2 stages, each
// stage one 128-key tile: 4 * 128 * 2D bytes (128 KiB at D = 128).  Split
// form: 5 stages of (K tile, V tile) of 64 keys (160 KiB at D = 128).
template <int D, bool SPLIT>
struct FwdLayout {
  static constexpr int kBN = SPLIT ? kBNSplit : kBNFull;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kBN * kRowBytes;
  static constexpr int kLdsBytes = SPLIT ? kStages * 2 * kTileBytes : 4 * kTileBytes;
  __device__ __forceinline__ static char* k_stage(char* smem, int u) {
    return SPLIT ? smem + (u % kStages) * 2 * kTileBytes : smem + (u & 1) * kTileBytes;
  }
  __device__ __forceinline__ static char* v_stage(char* smem, int u) {
    return SPLIT ? smem + (u % kStages) * 2 * kTileBytes + kTileBytes : smem + (2 + (u & 1)) * kTileBytes;
  }
};

constexpr int kAhead = 4;   // MFMA operand fragments in flight per wave

// SPLIT (causal launches with few query blocks): a workgroup covers 128 rows
// instead of 256; both wave groups hold the same rows, group g takes the key
// tiles 2t + g, and group 1 hands its partial row state to group 0 at the
// end.  Twice as many workgroups of half the size let the scheduler pair
// heavy causal blocks with light ones when one 256-row block per CU would
// leave the chip waiting on the heaviest.
// COUNT: the instrumented instantiation adds, per (b, h) and 32-row
// wavefront slot (rows 32 i .. 32 i + 31 of the head), the number of
// (wavefront, tile) steps after the wavefront's first tile in which the
// correction branch was taken to p.events[(b H + h) n_slots + i] (in the
// split form both wave groups of those rows add to the slot).
template <int D, bool CAUSAL, int EMU, bool SPLIT, bool COUNT>
__device__ __forceinline__ void fwd_block(const FwdParams& p, const int rank, const int bh) {
  using L = FwdLayout<D, SPLIT>;
  constexpr int kBN = L::kBN;
  constexpr int kKB = kBN / 32;   // 32-key blocks per tile
  constexpr int kKS = kBN / 16;   // 16-key steps of P V
  constexpr int kDB = D / 32;     // 32-dim blocks of the output
  constexpr int kKC = D / 16;     // 16-dim steps of Q K^T
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

  // rank 0 is the heaviest causal query block
  const int qb = CAUSAL ? (p.n_qblocks - 1 - rank) : rank;

  // key indices below are local to the range (key j is global key k_begin + j)
  const unsigned head_q = (unsigned)p.Sq * L::kRowBytes;
  const unsigned head_k = (unsigned)p.k_len * L::kRowBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + ((size_t)bh * p.Sk + p.k_begin) * D, head_k);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + ((size_t)bh * p.Sk + p.k_begin) * D, head_k);

  constexpr int kRows = SPLIT ? kBM / 2 : kBM;   // query rows per workgroup
  const int q_wave_lo = qb * kRows + (SPLIT ? (wave & 3) : wave) * kQW;
  const int q_lane = q_wave_lo + r32;
  const int k_lane = row_lane_offset<D>(lane);
  const int v_lane = tr_lane_offset<D>(lane);

  // Q^T operand: lane holds Q[q_lane][16 kc + 8 g .. +8] (zeros past the end)
  bf16x8 qf[kKC];
#pragma unroll
  for (int kc = 0; kc < kKC; ++kc)
    qf[kc] = __builtin_bit_cast(bf16x8, load16(rq, (unsigned)q_lane * L::kRowBytes + (kc * 16 + 8 * g) * 2));

  // causal, in local key coordinates: row i sees keys j <= i + q_diag
  const int q_diag = p.q_off - p.k_begin;
  const int kv_end = CAUSAL ? min(p.k_len, q_diag + (qb + 1) * kRows) : p.k_len;
  if (kv_end <= 0) {
    // no key is visible to any row of the block (key range after its rows)
    if (!(SPLIT && group == 1) && q_lane < p.Sq) {
      if (p.o32) {
        float* orow = p.o32 + ((size_t)bh * p.Sq + q_lane) * D;
#pragma unroll
        for (int c = 0; c < D / 2; c += 4) *reinterpret_cast<f32x4*>(orow + c + (D / 2) * g) = f32x4{};
      } else {
        bf16* orow = p.o + ((size_t)bh * p.Sq + q_lane) * D;
#pragma unroll
        for (int c = 0; c < D / 2; c += 8) *reinterpret_cast<u32x4*>(orow + c + (D / 2) * g) = u32x4{};
      }
      if (g == 0) p.lse[(size_t)bh * p.Sq + q_lane] = kNegInf;
    }
    return;
  }
  const int n = (kv_end + kBN - 1) / kBN;
  // tiles this wave needs: causal stops at the wave's last row; a wave whose
  // rows see no key of the range still runs tile 0, fully masked
  int n_wave = CAUSAL ? max(1, min(n, (q_diag + q_wave_lo + kQW + kBN - 1) / kBN)) : n;
  // as for n_mine below: knowing the bound, the optimiser reshapes the tile
  // loops in a way that makes the allocator spill
  if (CAUSAL) asm volatile("" : "+s"(n_wave));
  // SPLIT: group g takes tiles 2t + g, all of them up to n: a causal tile
  // past the wave's rows is fully masked (P = 0, the reference max stays).
  // The waves move in step through the barriers and the last rows' waves
  // set the pace, so such tiles cost no time, while a per-wave count would
  // put a branch around the accumulating code, which the allocator answers
  // with spills.  Group 1 with no tile (n = 1) still runs tile 1, whose keys
  // all lie past Sk or past its rows.
  int n_mine = SPLIT ? max(1, (n - group + 1) >> 1) : n_wave;
  // hide the bound from the optimiser: knowing n_mine >= 1 it restructures
  // the tile loop in a way that makes the allocator spill
  if (SPLIT) asm volatile("" : "+s"(n_mine));

  f32x16 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x16{};
  f32x16 s[kKB];
  bf16x8 pk[kKS];
  float m_ref = kNegInf;
  float l_part[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // 4 partial row sums of the float32 P (for the LSE)
  // Row sums of the bf16 weights P V multiplies (for O), on the matrix pipe:
  // a 16x16x32 product of a 0/1 selector with the packed P^T of a 16-key step
  // adds the step's 16 weights of query c to C[0][c] and of query c + 16 to
  // C[1][c] (lane c < 16 holds both).  O divided by this sum is a weighted
  // mean of V rows, so a row that one key dominates gets that key's V row
  // unchanged; a division by the float32 sum would carry the bf16 rounding of
  // the dominant weight into O.
  f32x4 lh4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const bf16x8 lh_sel = row_sum_selector(lane);
  int n_events = 0;                             // COUNT only (wave-uniform)

  // ---- matrix phase: O += V_{t-1} P_{t-1}, then S_t = K_t Q^T, as one stream
  // of MFMAs whose LDS operands are read kAhead MFMAs ahead through a small
  // register ring; scheduling fences keep the compiler from hoisting all of
  // them (which would not fit the register budget of two waves per SIMD).
  constexpr int kNV = kKS * kDB;    // P V products
  constexpr int kNK = kKB * kKC;    // K Q^T products
  // uk: the tile whose S is computed; uv: the tile whose P V is added
  auto matrix_stream_body = [&](int uk, int uv, auto with_pv, auto with_s) __attribute__((always_inline)) {
    constexpr bool PV = decltype(with_pv)::value;
    constexpr bool SK = decltype(with_s)::value;
    constexpr int j0 = PV ? 0 : kNV;
    constexpr int j1 = SK ? kNV + kNK : kNV;
    const char* vst = L::v_stage(smem, uv);
    const char* kst = L::k_stage(smem, uk);
    // j < kNV: (ks, db) = (j / kDB, j % kDB); j >= kNV: (kc, kb) = (i / kKB, i % kKB), i = j - kNV
    auto operand = [&](int j) __attribute__((always_inline)) -> bf16x8 {
      if (j < kNV) return read_cols<D>(vst, v_lane, j / kDB, j % kDB);
      const int i = j - kNV;
      return read_rows<D>(kst, k_lane, i % kKB, i / kKB);
    };
    if (SK) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) s[kb] = f32x16{};
    }
    bf16x8 ring[kAhead];
#pragma unroll
    for (int j = j0; j < j0 + kAhead && j < j1; ++j) ring[(j - j0) % kAhead] = operand(j);
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const bf16x8 a = ring[(j - j0) % kAhead];
      if (j + kAhead < j1) ring[(j - j0) % kAhead] = operand(j + kAhead);
      if (j < kNV) {
        o[j % kDB] = mfma32x32x16(a, pk[j / kDB], o[j % kDB]);
        // the row sum of exactly the bf16 weights P V multiplies, on VALU
        // slots the matrix phase leaves idle: O divided by it is a weighted
        // mean of V rows, so a row that one key dominates gets that key's V
        // row unchanged (a division by the float32 sum would carry the bf16
        // rounding of that key's weight)
        if (j % kDB == kDB - 1) lh4 = mfma16x16x32(lh_sel, pk[j / kDB], lh4);
      } else {
        const int i = j - kNV;
        s[i % kKB] = mfma32x32x16(a, qf[i / kKB], s[i % kKB]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The matrix phase runs at raised wave priority so its MFMAs issue ahead of
  // the vector-phase wave sharing the SIMD.
  auto matrix_stream = [&](int uk, int uv, auto with_pv, auto with_s) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
    matrix_stream_body(uk, uv, with_pv, with_s);
    __builtin_amdgcn_s_setprio(0);
  };
  // tiles of the group: consecutive (t) or every other one (SPLIT: 2t + group)
  auto tile_of = [&](int t) __attribute__((always_inline)) -> int { return SPLIT ? 2 * t + group : t; };
  auto matrix_s = [&](int t) __attribute__((always_inline)) {
    matrix_stream(tile_of(t), 0, std::false_type{}, std::true_type{});
  };
  auto matrix_full = [&](int t) __attribute__((always_inline)) {
    matrix_stream(tile_of(t), tile_of(t - 1), std::true_type{}, std::true_type{});
  };
  auto matrix_pv = [&](int t) __attribute__((always_inline)) {
    matrix_stream(0, tile_of(t - 1), std::true_type{}, std::false_type{});
  };

  // ---- vector phase: softmax of tile t
  auto vector = [&](int t) __attribute__((always_inline)) {
    if (t >= n_mine) return;
    const int k0 = tile_of(t) * kBN;
    const bool need_mask = (k0 + kBN > p.k_len) || (CAUSAL && k0 + kBN - 1 > q_diag + q_wave_lo);
    if (need_mask) {
      // key (kb, i) of this lane is k0 + 32 kb + 8 (i / 4) + 4 g + i % 4; it
      // is kept iff below k_len (and, causal, at most the row's diagonal)
      const int last = CAUSAL ? min(p.k_len - 1, q_diag + q_lane) : p.k_len - 1;
      softmax_mask_prefix<kKB>(s, last - k0 - 4 * g);
    }
    const float mx = softmax_row_max<kKB>(s);
    const bool corrected = softmax_conditional_rescale(m_ref, mx * p.scale_log2, p.tau, [&](float alpha) {
#pragma unroll
      for (int c = 0; c < 4; ++c) l_part[c] *= alpha;
      // the selector sums hold queries lane % 16 and lane % 16 + 16
      lh4[0] *= __shfl(alpha, lane & 15);
      lh4[1] *= __shfl(alpha, (lane & 15) + 16);
#pragma unroll
      for (int db = 0; db < kDB; ++db) o[db] *= alpha;
    });
    if constexpr (COUNT) n_events += (corrected && t > 0) ? 1 : 0;
    (void)corrected;
    softmax_exp_rowsum<kKB, EMU>(s, p.scale_log2, m_ref, l_part);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const int kb = ks >> 1, h = (ks & 1) * 8;
      pk[ks] = pack_bf16x8(s[kb][h + 0], s[kb][h + 1], s[kb][h + 2], s[kb][h + 3], s[kb][h + 4], s[kb][h + 5],
                           s[kb][h + 6], s[kb][h + 7]);
    }
  };

  // Tile IO.  The 256-row form loads tiles straight into LDS (memory-to-LDS
  // loads, no registers).  Tile u's K is read in intervals 2u+1 and 2u+2 (the
  // S products of the two groups) and its V in 2u+3 and 2u+4 (their P V
  // products).  With two stages per ring, K_u replaces K_{u-2} (last read in
  // interval 2u-2) and V_u replaces V_{u-2} (last read in 2u), so interval
  // 2u-1 issues K_u and V_{u-1} (fetch(u)) and the end of interval 2u waits
  // for them (commit): every load has two intervals to arrive.  The split
  // form loads tile u (K and V, one 5-stage ring) memory-to-LDS at the start
  // of interval u-1, into the stage of tile u-5, whose last read was in
  // interval u-2, and waits for it at the end of interval u: two intervals
  // for every load too (staged through registers with four stages, the load
  // had one).  It fetches unconditionally: past the last tile that costs a
  // little bandwidth (rows past the head read as zeros) and keeps the
  // per-wave load count, which the waits count, the same every interval.
  using DMA = TileDMA<D, kBN, kWaves>;
  constexpr int kSplitLoads = 2 * DMA::kLoads;   // per wave and tile (K, V)
  auto fetch = [&](int u) __attribute__((always_inline)) {
    if constexpr (SPLIT) {
      DMA::load(rk, u * kBN, L::k_stage(smem, u), wave, lane);
      DMA::load(rv, u * kBN, L::v_stage(smem, u), wave, lane);
    } else {
      if (u < n) DMA::load(rk, u * kBN, L::k_stage(smem, u), wave, lane);
      if (u >= 1 && u <= n) DMA::load(rv, (u - 1) * kBN, L::v_stage(smem, u - 1), wave, lane);
    }
  };
  // 256-row form: every load issued so far; split form: all but the last
  // tile's (the one fetched in this interval)
  auto commit = [&](int) __attribute__((always_inline)) {
    if constexpr (SPLIT) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSplitLoads) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  if constexpr (SPLIT) {
    // Interval k = 1 .. max(n, 2) + 2, one workgroup barrier after each.  Every wave
    // opens interval k by loading tile k+1 into stage (k+1) % 5 and closes it
    // by waiting for tile k (all but tile k+1's loads), so tile u is readable
    // from interval u+1.  Group g takes the tiles u = 2t + g: matrix(t) in
    // interval 2t+1+g (S of tile u, P V of tile u-2) and vector(t) one
    // interval later.  The last read of tile u (its V) falls in interval
    // u+3, before tile u+5's load in interval u+4.
    fetch(0);
    fetch(1);
    commit(0);
    barrier();
    int k = 1;
    auto open = [&]() __attribute__((always_inline)) { fetch(k + 1); };
    auto close = [&]() __attribute__((always_inline)) {
      commit(k);
      barrier();
      ++k;
    };
    if (group == 1) {
      open();
      close();
    }
    open();
    matrix_s(0);
    close();
    open();
    vector(0);
    close();
    for (int t = 1; t < n_mine; ++t) {
      open();
      matrix_full(t);
      close();
      open();
      vector(t);
      close();
    }
    open();
    matrix_pv(n_mine);
    close();
    while (k <= max(n, 2) + 2) {
      open();
      close();
    }
  } else {
    // Interval k = 1 .. 2n+2, one workgroup barrier after each:
    //   group 0: interval 2t+1 matrix(t), 2t+2 vector(t); 2n+1 matrix(n); 2n+2 idle
    //   group 1: interval 1 idle; 2t+2 matrix(t), 2t+3 vector(t); 2n+2 matrix(n)
    // matrix(t) = O += V_{t-1} P_{t-1} (t > 0) and S_t = K_t Q^T (t < n_wave);
    // vector(t) = softmax of S_t.  A causal wave has nothing to do after tile
    // n_wave - 1 but keeps taking part in the barriers and the loads.  Every
    // wave issues its share of fetch(u) in interval 2u-1 and commits at the
    // end of every even interval.  Each variant of the matrix phase has one
    // call site (the last P V is matrix_pv(n_wave), n_wave = n when the wave
    // has no tile left), so the compiler never merges two copies of a phase
    // at a branch join (which cost registers and copies).  Prologue: K_0 is
    // loaded and readable in interval 1.
    fetch(0);
    commit(0);
    barrier();
    if (group == 0) {
      fetch(1);
      matrix_s(0);
      barrier();
      vector(0);
      commit(0);
      barrier();
      for (int t = 1; t < n_wave; ++t) {
        fetch(t + 1);
        matrix_full(t);
        barrier();
        vector(t);
        commit(0);
        barrier();
      }
      // one call site of the last P V (n_wave = n when nothing is left)
      if (n_wave < n) fetch(n_wave + 1);
      matrix_pv(n_wave);
      barrier();
      if (n_wave < n) {
        commit(0);
        barrier();
        for (int t = n_wave + 1; t < n; ++t) {
          fetch(t + 1);
          barrier();
          commit(0);
          barrier();
        }
        barrier();
      }
      barrier();
    } else {
      fetch(1);
      barrier();
      matrix_s(0);
      commit(0);
      barrier();
      fetch(2);
      vector(0);
      barrier();
      for (int t = 1; t < n_wave; ++t) {
        matrix_full(t);
        commit(0);
        barrier();
        fetch(t + 2);
        vector(t);
        barrier();
      }
      matrix_pv(n_wave);
      if (n_wave < n) {
        commit(0);
        barrier();
        fetch(n_wave + 2);
        barrier();
        for (int t = n_wave + 1; t < n; ++t) {
          commit(0);
          barrier();
          fetch(t + 2);
          barrier();
        }
      }
      barrier();
    }
  }
  if constexpr (COUNT) {
    // one vector atomic per wavefront (lane 0 holds the address)
    if (lane == 0 && n_events > 0 && q_wave_lo < p.Sq)
      atomicAdd(p.events + (size_t)bh * ((p.Sq + kQW - 1) / kQW) + q_wave_lo / kQW, (unsigned)n_events);
  }
  float l_lane = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
  // this lane's query r32 from lane r32 % 16 (row 0: queries 0-15, row 1: 16-31)
  float lh_lane;
  {
    const float x0 = __shfl(lh4[0], r32 & 15), x1 = __shfl(lh4[1], r32 & 15);
    lh_lane = r32 < 16 ? x0 : x1;
  }
  if constexpr (SPLIT) {
    // group 1 hands (O, row sums, reference max) of each lane to the lane of
    // group 0 that holds the same row and columns, in the ring: once every
    // wave's last tile load (issued in the last interval, past the last
    // tile) has landed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();
    constexpr int kXO = kDB * 4 * 256 * 16;   // O: [db * 4 + i4][256 lanes] f32x4
    static_assert(kXO + 3 * 256 * 4 <= L::kLdsBytes, "merge area exceeds the LDS ring");
    const int tl = (wave & 3) * 64 + lane;
    f32x4* xo = reinterpret_cast<f32x4*>(smem);
    float* xs = reinterpret_cast<float*>(smem + kXO);
    if (group == 1) {
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          xo[(db * 4 + i4) * 256 + tl] = f32x4{o[db][4 * i4 + 0], o[db][4 * i4 + 1], o[db][4 * i4 + 2],
                                               o[db][4 * i4 + 3]};
      xs[tl] = m_ref;
      xs[256 + tl] = l_lane;
      xs[512 + tl] = lh_lane;
    }
    barrier();
    if (group == 1) return;
    const float m1 = xs[tl];
    const float m = __builtin_fmaxf(m_ref, m1);
    // a group that saw no key of this row has m = -inf and weight 0
    const float a0 = (m_ref == kNegInf) ? 0.0f : exp2_hw(m_ref - m);
    const float a1 = (m1 == kNegInf) ? 0.0f : exp2_hw(m1 - m);
    l_lane = l_lane * a0 + xs[256 + tl] * a1;
    lh_lane = lh_lane * a0 + xs[512 + tl] * a1;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 x = xo[(db * 4 + i4) * 256 + tl];
#pragma unroll
        for (int c = 0; c < 4; ++c) o[db][4 * i4 + c] = o[db][4 * i4 + c] * a0 + x[c] * a1;
      }
    m_ref = m;
  }

  // ---- epilogue: O = O / lh (bf16 or float32; lh sums the bf16 weights P V
  // used), LSE = (m_ref + log2 l) ln 2 (l sums the float32 P); a row that saw
  // no key (only possible for a key range) gets O = 0 and LSE = -inf, the
  // identity of the merge of partial results
  const float l = pair_sum(l_lane);
  const float lh = lh_lane;   // already the whole row's sum (both lane halves)
  const bool empty = !(l > 0.0f);
  const float inv_l = empty ? 0.0f : 1.0f / lh;
  if (!p.o32) {
    // bf16 output, stored as whole rows through a per-wave LDS area in the
    // ring, idle after the last barrier (every tile read and load has
    // completed); in the split form the areas follow the merge area, which
    // the other waves of group 0 may still be reading
    using RS = RowStore<D>;
    constexpr int kStageBase = SPLIT ? kDB * 4 * 256 * 16 + 3 * 256 * 4 : 0;
    constexpr int kStagingWaves = SPLIT ? kWaves / 2 : kWaves;
    static_assert(kStageBase + kStagingWaves * RS::kBytes <= L::kLdsBytes, "output staging exceeds the LDS ring");
    RS::store(smem + kStageBase + (SPLIT ? (wave & 3) : wave) * RS::kBytes, o, inv_l, p.o + (size_t)bh * p.Sq * D,
              q_wave_lo, p.Sq, lane);
    if (q_lane < p.Sq && g == 0)
      p.lse[(size_t)bh * p.Sq + q_lane] = empty ? kNegInf : (m_ref + __builtin_log2f(l)) * kLn2;
  } else if (q_lane < p.Sq) {
    // float32 output (key-range parts): 16-byte pieces, stored directly
    float* orow = p.o32 + ((size_t)bh * p.Sq + q_lane) * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4 + 4 * g) =
            f32x4{o[db][4 * i4 + 0] * inv_l, o[db][4 * i4 + 1] * inv_l, o[db][4 * i4 + 2] * inv_l,
                  o[db][4 * i4 + 3] * inv_l};
    if (g == 0) p.lse[(size_t)bh * p.Sq + q_lane] = empty ? kNegInf : (m_ref + __builtin_log2f(l)) * kLn2;
  }
}

// One query block per workgroup, heaviest causal blocks first (consecutive
// workgroups take different heads of the same block rank); or, paired,
// workgroup (r, bh) runs rank r and then rank n_qblocks - 1 - r of the same
// head: every workgroup has the same causal work and the CU starts no new
// workgroup between the two blocks.  Between them every wave's loads,
// stores and LDS reads have completed (the second block's prologue loads
// into the LDS the first one's epilogue staged its output in).
template <int D, bool CAUSAL, int EMU, bool SPLIT, bool COUNT = false>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdParams p) {
  const int r = blockIdx.x / p.BH, bh = blockIdx.x % p.BH;
  int n_it = p.paired ? 2 : 1;
  asm volatile("" : "+s"(n_it));
#pragma unroll 1
  for (int it = 0; it < n_it; ++it) {
    if (it > 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    fwd_block<D, CAUSAL, EMU, SPLIT, COUNT>(p, it == 0 ? r : p.n_qblocks - 1 - r, bh);
  }
}

// Software-exponential counts per 32 scores of a lane (64 keys) that are
// instantiated.
constexpr int kEmuCounts[] = {0, 3, 8, 16, 32};

template <int D, bool CAUSAL, int EMU, bool SPLIT, bool COUNT = false>
hipError_t launch_one(const FwdParams& prm, dim3 grid, hipStream_t stream) {
  auto kern = fwd_kernel<D, CAUSAL, EMU, SPLIT, COUNT>;
  const int lds = FwdLayout<D, SPLIT>::kLdsBytes;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, prm);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_d_causal(const FwdParams& prm, int emu, dim3 grid, hipStream_t stream) {
  if (prm.events) return launch_one<D, CAUSAL, 0, SPLIT, true>(prm, grid, stream);
  switch (emu) {
    case 0: return launch_one<D, CAUSAL, 0, SPLIT>(prm, grid, stream);
    case 3: return launch_one<D, CAUSAL, 3, SPLIT>(prm, grid, stream);
    case 8: return launch_one<D, CAUSAL, 8, SPLIT>(prm, grid, stream);
    case 16: return launch_one<D, CAUSAL, 16, SPLIT>(prm, grid, stream);
    case 32: return launch_one<D, CAUSAL, 32, SPLIT>(prm, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// Causal launches split a query block over both wave groups when the grid
// of 256-row blocks would give fewer than two workgroups per CU: a workgroup
// fills a CU, so with one wave of workgroups the heaviest block sets the
// time, while 128-row blocks of half the cost can be paired heavy with light.
constexpr int kSplitBelowBlocks = 512;

}  // namespace

// the software share is placed per 64 keys (32 scores of a lane) in both forms
int fwd_exps_per_lane_tile(int /*d*/) { return 32; }

int fwd_nearest_emu_count(int d, float emu_frac) {
  const float want = emu_frac * (float)fwd_exps_per_lane_tile(d);
  int best = kEmuCounts[0];
  for (int c : kEmuCounts) {
    if (__builtin_fabsf((float)c - want) < __builtin_fabsf((float)best - want)) best = c;
  }
  return best;
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  FwdParams prm;
  prm.q = static_cast<const bf16*>(a.q);
  prm.k = static_cast<const bf16*>(a.k);
  prm.v = static_cast<const bf16*>(a.v);
  prm.o = static_cast<bf16*>(a.o);
  prm.o32 = a.o32;
  prm.lse = a.lse;
  prm.BH = a.B * a.H;
  prm.Sq = a.Sq;
  prm.Sk = a.Sk;
  prm.k_begin = a.k_begin;
  prm.k_len = a.k_end - a.k_begin;
  prm.q_off = a.q_off;
  prm.scale_log2 = a.scale * kLog2e;
  prm.tau = a.tau;
  prm.events = a.events;
  if (a.events && a.emu_count != 0) return hipErrorInvalidValue;   // counted with hardware exponentials only
  const long long full_blocks = (long long)((a.Sq + kBM - 1) / kBM) * prm.BH;
  const bool split = a.causal && full_blocks < kSplitBelowBlocks;
  const int rows = split ? kBM / 2 : kBM;
  prm.n_qblocks = (a.Sq + rows - 1) / rows;
  prm.paired = (a.causal && prm.n_qblocks % 2 == 0) ? 1 : 0;
  const dim3 grid((unsigned)((prm.paired ? prm.n_qblocks / 2 : prm.n_qblocks) * prm.BH));
  if (a.d == 64) {
    if (!a.causal) return launch_d_causal<64, false, false>(prm, a.emu_count, grid, stream);
    return split ? launch_d_causal<64, true, true>(prm, a.emu_count, grid, stream)
                 : launch_d_causal<64, true, false>(prm, a.emu_count, grid, stream);
  }
  if (!a.causal) return launch_d_causal<128, false, false>(prm, a.emu_count, grid, stream);
  return split ? launch_d_causal<128, true, true>(prm, a.emu_count, grid, stream)
               : launch_d_causal<128, true, false>(prm, a.emu_count, grid, stream);
}

// ---------------------------------------------------------------- exp2 probe
namespace {
__global__ void exp2_probe_kernel(const float* x, float* y_hw, float* y_emu, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const float v = x[i];
    y_hw[i] = exp2_hw(v);
    y_emu[i] = exp2_sw(v);
  }
}
}  // namespace

hipError_t launch_exp2_probe(const float* x, float* y_hw, float* y_emu, long long n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(exp2_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y_hw, y_emu, n);
  return hipGetLastError();
}

}  // namespace fa
