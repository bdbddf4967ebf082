// Fused exact-attention backward for gfx950.
//
// Method.  The gradients of O = softmax(scale Q K^T) V with P recomputed from
// the forward's log-sum-exp (FA4 paper §3.2 as summarised on "FlashAttention-4:
// Algorithm and Kernel Pipelining Co-Design for Asymmetric Hardware Scaling"):
//   S = Q K^T,  P = exp(scale S - LSE),  dP = dO V^T,  dS = P (dP - D),
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K,
// with D_i = sum_c dO_ic O_ic.
//
// CDNA4 design (ours).  The paper adds every key block's dQ contribution with
// atomics (and orders them behind a lock in its deterministic mode).  On
// MI355X the float32 atomic adds of that pattern run at ~1.3 TB/s (measured,
// probes/dq_atomics.hip), and ordering them serialises the key blocks of a
// head.  Here the backward is split by output instead, so every output
// element is written exactly once:
//   bwd_prep_kernel   D_i (inside bwd_dq_kernel when both run in one call);
//   bwd_dq_kernel     a workgroup owns 128 query rows and streams K / V tiles:
//                     S^T = K Q^T, dP^T = V dO^T (one query per lane, so LSE_i
//                     and D_i are per-lane scalars), dS^T, dQ^T += K^T dS^T;
//   bwd_dkdv_kernel   a workgroup owns 128 key rows and streams Q / dO tiles:
//                     S = Q K^T, dP = dO V^T (one key per lane), P, dS,
//                     dV^T += dO^T P, dK^T += Q^T dS.
// That is seven products per tile pair instead of five, no atomics, no
// workspace beyond the row terms D and LSE log2(e), and results that are
// bit-identical run to run in both modes (the deterministic flag costs
// nothing).  Tiles use the layout of
// fa_tiles.hpp, so Q, dO, K and V are each read both row-wise and transposed
// from one LDS copy.
//
// Five-product form (fa_bwd_ds): the paper's five products per tile pair
// without its dQ atomics.  bwd_dkdv_kernel, which rounds dS to bf16 for its
// dK product anyway, also stores it to a dS^T buffer in the workspace, and
// bwd_dq_ds_kernel forms dQ = scale dS K from that buffer and K: S and dP
// are formed once, at the price of writing and reading dS (2 bytes per
// visited pair) through HBM.  Also free of atomics and bit-identical run to
// run.

#include <mutex>
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_tiles.hpp"

namespace fa {
namespace {

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const float* lse;
  const bf16* dout;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* dvec;   // D_i, [B, H, Sq]
  float* lse2;   // LSE_i * log2(e), [B, H, Sq]
  bf16* ds;      // five-product form: dS^T slabs, [B H, ds_nqb, ds_rows, 128]
  int ds_nqb;    // blocks of 128 query rows, ceil(Sq / 128)
  int ds_rows;   // key rows per slab, Sk rounded up to 128
  int BH, Sq, Sk;
  int fuse_prep; // the dQ kernel forms D_i and LSE_i log2(e) itself and stores them
  float scale;
  float scale_log2;
};

// dS^T buffer of the five-product form.  Per (b, h) and block of 128 query
// rows ("positions", one dQ workgroup each) a slab of ds_rows / 64 key tiles
// of 16 KB: in tile kt, group pg of 16 positions and key k (kt = k / 64)
// hold positions 16 pg .. +16 of key k as one 32-byte record at byte
// (kt * 8 + pg) * 2048 + (k % 64) * 32, so the dQ kernel reads each tile as
// one contiguous block.  Position 16 x + 8 g + j of a block holds query row
// 16 x + 8 (j / 4) + 4 g + j % 4 (bits 2 and 3 of the row index exchanged):
// the order in which a lane of the dK/dV kernel holds dS, so one of its
// 16-byte stores of a 16-row step covers half a record and a wave's store
// (32 keys) 1 KB of consecutive records.
constexpr int kDsPositions = 128;
constexpr int kDsGroup = 16;                                // positions per record
constexpr int kDsRecord = kDsGroup * 2;                     // bytes per record
constexpr int kDsTileKeys = 64;                             // keys per slab tile
constexpr int kDsTileBytes = kDsTileKeys * kDsRecord * (kDsPositions / kDsGroup);   // 16 KB

// ------------------------------------------------------------------- prep
// D_i and LSE_i log2(e) of every query row into the workspace.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p, long long rows) {
  // D_i = sum_c dO_ic O_ic: D/8 lanes per row, 16 bytes each
  constexpr int kTPR = D / 8;
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nthreads = (long long)gridDim.x * blockDim.x;
  for (long long t = gtid; t < rows * kTPR; t += nthreads) {
    const long long row = t / kTPR;
    const int c = (int)(t % kTPR) * 8;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p.o + row * D + c);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(p.dout + row * D + c);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s = __builtin_fmaf((float)a[j], (float)b[j], s);
#pragma unroll
    for (int off = kTPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if ((t % kTPR) == 0) {
      p.dvec[row] = s;
      p.lse2[row] = p.lse[row] * kLog2e;
    }
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ==================================================================== dQ
// 4 wavefronts x 32 query rows = 128 rows per workgroup (one wave per SIMD);
// key tiles of 64 rows, walked from the diagonal down (the two tiles that
// can need a mask come first).  Work is pipelined by 32-key half tiles u:
//   [S^T, dP^T of u  |  P, dS of u-1 (VALU)]  [dQ^T += K^T dS^T of u-1]
// so a tile is [S,dP b0 | P,dS of the previous tile's b1] [dQ prev b1]
// [S,dP b1 | P,dS b0] [dQ b0], one fixed sequence of MFMAs whose LDS operands
// stream through a register ring running on across tiles.  K / V tiles
// arrive memory-to-LDS in a 4-stage ring issued three tiles ahead (a tile's
// K is still read during the next tile), one barrier per tile.
namespace dqk {
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;
constexpr int kBM = kWaves * kQW;
constexpr int kBN = 64;
constexpr int kStages = 4;
constexpr int kRing = 8;
template <int D>
struct Layout {
  static constexpr int kTileBytes = kBN * TileGeom<D>::kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;   // K then V
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kLoadsPerTile = 2 * TileDMA<D, kBN, kWaves>::kLoads;   // per wave
};
}  // namespace dqk

template <int D, bool CAUSAL>
__global__ __launch_bounds__(dqk::kThreads, 1) void bwd_dq_kernel(BwdParams p) {
  using namespace dqk;
  using L = Layout<D>;
  using G = TileGeom<D>;
  constexpr int kKC = D / 16;           // 16-dim steps of S^T and dP^T
  constexpr int kDB = D / 32;           // 32-dim blocks of dQ^T
  constexpr int kNS = 2 * kKC;          // S^T and dP^T products of a half tile
  constexpr int kNQ = 2 * kDB;          // dQ^T products of a half tile
  constexpr int kU = kNS + kNQ;         // steps of a half tile
  constexpr int kSteps = 2 * kU;
  constexpr int kBar = kSteps - kRing;  // barrier position (before this step)
  constexpr int kPPS = 16 / kNS;        // P / dS elements per step
  constexpr int kPer = L::kLoadsPerTile;
  static_assert(kSteps % kRing == 0, "ring must divide the step count");
  static_assert(kRing <= kNS, "the ring's look-ahead into the next tile stays in its first S / dP block");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int n_qb = (p.Sq + kBM - 1) / kBM;
  const int qb = CAUSAL ? n_qb - 1 - (int)(blockIdx.x / p.BH) : (int)(blockIdx.x / p.BH);   // heavy first
  const int bh = blockIdx.x % p.BH;
  const int q0 = qb * kBM;
  const int qi = q0 + wave * kQW + r32;   // the lane's query row
  const bool q_ok = qi < p.Sq;

  const unsigned head_q = (unsigned)p.Sq * G::kRowBytes;
  const unsigned head_k = (unsigned)p.Sk * G::kRowBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (size_t)bh * p.Sk * D, head_k);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (size_t)bh * p.Sk * D, head_k);

  const int row_lane = row_lane_offset<D>(lane);
  const int tr_lane = tr_lane_offset<D>(lane);

  // B operands: the lane's Q and dO rows, dims 16 kc + 8 g .. +8 (AGPRs)
  const bool fuse = p.fuse_prep != 0;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + (size_t)bh * p.Sq * D, head_q);
  bf16x8 qf[kKC], of[kKC];
  float dchunk[kKC];   // sum over the 8 dims 16 kc + 8 g .. of dO O (fused prep only)
#pragma unroll
  for (int kc = 0; kc < kKC; ++kc) {
    const unsigned off = (unsigned)qi * G::kRowBytes + (kc * 16 + 8 * g) * 2;
    qf[kc] = __builtin_bit_cast(bf16x8, load16(rq, off));
    of[kc] = __builtin_bit_cast(bf16x8, load16(rdo, off));
    dchunk[kc] = 0.0f;
    if (fuse) {
      const bf16x8 oc = __builtin_bit_cast(bf16x8, load16(ro, off));
#pragma unroll
      for (int j = 0; j < 8; ++j) dchunk[kc] = __builtin_fmaf((float)oc[j], (float)of[kc][j], dchunk[kc]);
    }
    asm volatile("s_nop 1" : "+a"(qf[kc]), "+a"(of[kc]));
  }
  // the lane's row terms (rows past the end: any finite value; never stored)
  const size_t ri = (size_t)bh * p.Sq + (q_ok ? qi : 0);
  float lse2, dval;
  if (fuse) {
    // D_i in the association of bwd_prep_kernel's butterfly (16 lanes of 8
    // dims at D = 128, 8 at D = 64; its lane 0 ends with the even 8-dim
    // chunks plus the odd ones), so the value is bit-identical: here chunk
    // 2 kc + g sits in lane g of the pair
    static_assert(kKC == 8 || kKC == 4, "D = 128 or 64");
    float w;
    if constexpr (kKC == 8)
      w = ((dchunk[0] + dchunk[4]) + (dchunk[2] + dchunk[6])) + ((dchunk[1] + dchunk[5]) + (dchunk[3] + dchunk[7]));
    else
      w = (dchunk[0] + dchunk[2]) + (dchunk[1] + dchunk[3]);
    dval = w + __shfl_xor(w, 32);
    lse2 = p.lse[ri] * kLog2e;
    if (q_ok && g == 0) {
      p.dvec[ri] = dval;
      p.lse2[ri] = lse2;
    }
  } else {
    lse2 = p.lse2[ri];
    dval = p.dvec[ri];
  }

  f32x16 dq[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    dq[db] = f32x16{};
    asm volatile("s_nop 1" : "+a"(dq[db]));
  }

  // key tiles: n of them, relative tile t is key tile n - 1 - t
  const int n_kt_all = (p.Sk + kBN - 1) / kBN;
  const int n_kt_causal = (q0 + kBM + kBN - 1) / kBN;
  const int n = CAUSAL ? (n_kt_causal < n_kt_all ? n_kt_causal : n_kt_all) : n_kt_all;

  auto issue = [&](int t, auto stage_tag) __attribute__((always_inline)) {
    char* st = smem + decltype(stage_tag)::value * L::kStageBytes;
    const int k0 = (n - 1 - t) * kBN;
    TileDMA<D, kBN, kWaves>::load(rk, k0, st, wave, lane);
    TileDMA<D, kBN, kWaves>::load(rv, k0, st + L::kTileBytes, wave, lane);
  };

  // operand j of a tile: [rows of K, V block 0][cols of the previous tile's
  // K, steps 2, 3][rows of K, V block 1][cols of this tile's K, steps 0, 1]
  auto op = [&](const char* cur, const char* prev, int j) __attribute__((always_inline)) -> bf16x8 {
    const int u = j / kU, jj = j % kU;
    if (jj < kNS) {
      const char* tile = (jj & 1) ? cur + L::kTileBytes : cur;
      return read_rows<D>(tile, row_lane, u, jj >> 1);
    }
    const int qj = jj - kNS;
    const int ks = 2 * (1 - u) + qj / kDB, db = qj % kDB;
    return read_cols<D>(u == 0 ? prev : cur, tr_lane, ks, db);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  static_assert(kStages == 4, "stage constants below assume four stages");

  // ---- prologue: tiles 0, 1, 2 in flight; wait for tile 0
  issue(0, S0{});
  if (n > 1) issue(1, S1{});
  if (n > 2) issue(2, S2{});
  if (n > 2) wait_vmcnt<2 * kPer>();
  else if (n > 1) wait_vmcnt<kPer>();
  else wait_vmcnt<0>();
  lds_barrier();
  bf16x8 ring[kRing];
#pragma unroll
  for (int j = 0; j < kRing; ++j) ring[j] = op(smem, smem, j);

  f32x16 s[2], dp[2];
  bf16x8 bs[4];      // bf16 dS^T of the four 16-key steps (B operands)
  float de[16];      // dS of the half tile in progress

  // P, dS of half tile b of the tile starting at key k0: element i holds key
  // k0 + 32 b + 8 (i / 4) + 4 g + i % 4 of the lane's query
  auto pds_elem = [&](int b, int i, int lim, auto mask_tag) __attribute__((always_inline)) {
    float x = __builtin_fmaf(s[b][i], p.scale_log2, -lse2);
    if (decltype(mask_tag)::value && 8 * (i >> 2) + (i & 3) > lim) x = kNegInf;
    const float pv = exp2_hw(x);
    de[i] = pv * (dp[b][i] - dval);
    if ((i & 7) == 7) {
      const int h = i - 7;
      bs[2 * b + (i >> 3)] = pack_bf16x8(de[h], de[h + 1], de[h + 2], de[h + 3], de[h + 4], de[h + 5], de[h + 6],
                                         de[h + 7]);
      asm volatile("" ::"v"(bs[2 * b + (i >> 3)]));
    }
  };
  // largest in-block key offset 8 (i / 4) + i % 4 that is visible to the lane
  auto mask_lim = [&](int k0, int b) __attribute__((always_inline)) -> int {
    const int last = CAUSAL ? (qi < p.Sk - 1 ? qi : p.Sk - 1) : p.Sk - 1;
    return last - k0 - 32 * b - 4 * g;
  };

  // One tile.  FIRST: no previous half tile (its dQ products are skipped);
  // MASK: mask this tile's elements; PMASK: the previous tile's.
  auto tile = [&](int t, auto first_tag, auto mask_tag, auto pmask_tag, auto stage_tag)
                  __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_tag)::value;
    constexpr int kS = decltype(stage_tag)::value;   // == t % kStages
    const char* cur = smem + kS * L::kStageBytes;
    const char* prev = smem + ((kS + kStages - 1) % kStages) * L::kStageBytes;
    const char* nxt = smem + ((kS + 1) % kStages) * L::kStageBytes;
    const int k0 = (n - 1 - t) * kBN;
    const int lim0 = mask_lim(k0, 0);
    const int plim1 = mask_lim(k0 + kBN, 1);

    static_for<kSteps>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = J;
      constexpr int u = j / kU, jj = j % kU;
      if constexpr (j == kBar) {
        // every operand of the previous tile has been read; publish tile t + 1
        if (t + 2 < n) wait_vmcnt<kPer>();
        else wait_vmcnt<0>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (t + 3 < n) issue(t + 3, std::integral_constant<int, (kS + 3) % kStages>{});
      }
      const bf16x8 a = ring[j % kRing];
      if constexpr (j + kRing < kSteps) ring[j % kRing] = op(cur, FIRST && j + kRing < kU ? cur : prev, j + kRing);
      else ring[j % kRing] = op(nxt, cur, j + kRing - kSteps);
      if constexpr (jj < kNS) {
        // S^T (even), dP^T (odd) of half tile u, in VGPRs
        if constexpr (jj < 2) {
          if constexpr (jj & 1) MfmaAsm<'v', 'a'>::init_v(dp[u], a, of[jj >> 1]);
          else MfmaAsm<'v', 'a'>::init_v(s[u], a, qf[jj >> 1]);
        } else {
          if constexpr (jj & 1) MfmaAsm<'v', 'a'>::acc_v(dp[u], a, of[jj >> 1]);
          else MfmaAsm<'v', 'a'>::acc_v(s[u], a, qf[jj >> 1]);
        }
      } else if constexpr (!(FIRST && u == 0)) {
        // dQ^T of the previous half tile: steps 2, 3 (u = 0, previous tile) or 0, 1
        constexpr int qj = jj - kNS;
        constexpr int ks = 2 * (1 - u) + qj / kDB, db = qj % kDB;
        MfmaAsm<'v', 'v'>::acc_a(dq[db], a, bs[ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // VALU during the S / dP products: P, dS of the previous half tile
      if constexpr (jj < kNS && !(FIRST && u == 0)) {
        constexpr int pb = 1 - u;   // its accumulators: block 1 (previous tile) or 0
        if constexpr (jj == 0) mfma_drain_v2(s[pb], dp[pb]);
        static_for<kPPS>([&](auto V) __attribute__((always_inline)) {
          constexpr int i = jj * kPPS + V;
          if constexpr (u == 0) pds_elem(pb, i, plim1, pmask_tag);
          else pds_elem(pb, i, lim0, mask_tag);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  using T = std::true_type;
  using F = std::false_type;
  using M = std::true_type;   // the two tiles next to the diagonal (or the ragged end) are masked
  tile(0, T{}, M{}, F{}, S0{});
  if (n > 1) tile(1, F{}, M{}, M{}, S1{});
  int t = 2;
  if (t < n) {
    tile(t, F{}, F{}, M{}, S2{});   // its previous tile (1) was masked
    ++t;
    while (t < n) {
      tile(t, F{}, F{}, F{}, S3{});
      if (++t >= n) break;
      tile(t, F{}, F{}, F{}, S0{});
      if (++t >= n) break;
      tile(t, F{}, F{}, F{}, S1{});
      if (++t >= n) break;
      tile(t, F{}, F{}, F{}, S2{});
      ++t;
    }
  }

  // ---- tail: P, dS and dQ^T of the last tile's half tile 1
  {
    const int tl = n - 1;
    const char* last = smem + (tl % kStages) * L::kStageBytes;
    const int k0 = (n - 1 - tl) * kBN;
    const int plim = mask_lim(k0, 1);
    mfma_drain_v2(s[1], dp[1]);
    if (tl < 2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) pds_elem(1, i, plim, T{});
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) pds_elem(1, i, plim, F{});
    }
    asm volatile("s_nop 1" : "+v"(bs[2]), "+v"(bs[3]));   // VALU writes -> MFMA reads
#pragma unroll
    for (int qj = 0; qj < kNQ; ++qj) {
      const int ks = 2 + qj / kDB, db = qj % kDB;
      MfmaAsm<'v', 'v'>::acc_a(dq[db], read_cols<D>(last, tr_lane, ks, db), bs[ks]);
    }
  }

  // ---- dQ = scale (dQ^T)^T -> bf16 (lane = query, 4 consecutive dims per group)
#pragma unroll
  for (int db = 0; db < kDB; ++db) mfma_drain_a(dq[db]);
  // whole-row stores through LDS, once every wave has read its last tile
  static_assert(kWaves * RowStore<D>::kBytes <= L::kLdsBytes, "output staging exceeds the LDS ring");
  dma_barrier();
  RowStore<D>::store(smem + wave * RowStore<D>::kBytes, dq, p.scale, p.dq + (size_t)bh * p.Sq * D,
                     q0 + wave * kQW, p.Sq, lane);
}

// =================================================================== dK dV
// 8 wavefronts, two on every SIMD, for 128 keys (four blocks of 32 keys);
// query tiles of 64 rows.  The two waves of a SIMD share a 32-key block and
// split each tile's work between them:
//   S wave  (wave w < 4):  S = Q K^T, P = 2^(scale log2(e) S - LSE log2(e))
//                          (causal mask applied), dV^T += dO^T P;
//   dP wave (wave w + 4):  dP = dO V^T, dS = P (dP - D) with P taken from
//                          the S wave through LDS in float32, dK^T += Q^T dS.
// They take turns on the matrix unit, one tile pipelined over two phases:
//   phase A(k)  S wave: dV^T += dO(k)^T P(k), S(k+1) = Q(k+1) K^T   (MFMA)
//               dP wave: dS(k) from P(k), dP(k)                     (VALU)
//   phase B(k)  dP wave: dK^T += Q(k)^T dS(k), dP(k+1) = dO(k+1) V^T (MFMA)
//               S wave: P(k+1) from S(k+1), written to LDS          (VALU)
// so in every phase one wave of a SIMD issues only products (operands
// streamed from LDS through a register ring that runs on across phases) and
// the other only element work, with a barrier between phases.  A prelude
// forms S(0), P(0) and dP(0); the last interval forms S(n), P(n), dP(n) of
// a tile that does not exist (LDS contents never used, every address in the
// allocation) so that all intervals run the same code.
// Tiles arrive memory-to-LDS in a 3-stage ring (tiles k and k + 1 are read
// during interval k): the loads of tile k + 2 are issued at the start of
// A(k) and published at the barrier after B(k).
namespace kvk {
constexpr int kPairs = 4;                // 32-key blocks per workgroup
constexpr int kWaves = 2 * kPairs;
constexpr int kThreads = kWaves * 64;
constexpr int kKW = 32;
constexpr int kBK = kPairs * kKW;
constexpr int kBQ = 64;
constexpr int kStages = 3;
// LDS by kind: the Q tiles of the stages, then the dO tiles, so that every
// operand read of a wave (Q and dO only) is a lane address plus an
// immediate offset below 64 KB from its kind's base; then per stage the
// tile's 64 rows of LSE log2(e) and of D; then P of each pair, float32 in
// the S wave's accumulator order: block b, elements 4 i4 .. 4 i4 + 3 of
// lane l at ((4 b + i4) 64 + l) 16.
template <int D>
struct Layout {
  static constexpr int kTileBytes = kBQ * TileGeom<D>::kRowBytes;
  static constexpr int kQOff = 0;
  static constexpr int kDoOff = (kStages * kTileBytes + 16383) / 16384 * 16384;
  static constexpr int kRowsOff = kDoOff + kStages * kTileBytes;
  static constexpr int kRowsBytes = 2 * kBQ * 4;   // per stage
  static constexpr int kPOff = kRowsOff + kStages * kRowsBytes;
  static constexpr int kPPairBytes = kKW * kBQ * 4;
  static constexpr int kLdsBytes = kPOff + kPairs * kPPairBytes;
  // the dP waves load the tiles: kTileLoads per wave and tile, plus one
  // row-term load for the waves of pairs 0 (LSE) and 1 (D)
  static constexpr int kTileLoads = 2 * TileDMA<D, kBQ, kPairs>::kLoads;
  // a kind's base shares no bit with a lane offset within a tile (nor with
  // the constants those are XORed with), and its tiles span under 64 KB
  static_assert(kQOff == 0 && kDoOff % 16384 == 0 && kTileBytes <= 16384, "tile kinds' bases");
  static_assert(kStages * kTileBytes <= 65536, "a kind's tiles span more than 64 KB");
};
}  // namespace kvk

// DS: also store the tile's bf16 dS (the five-product form).
template <int D, bool CAUSAL, bool DS = false>
__global__ __launch_bounds__(kvk::kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  using namespace kvk;
  using L = Layout<D>;
  using G = TileGeom<D>;
  constexpr int kKC = D / 16;          // 16-dim steps of S and dP per 32-row block
  constexpr int kDB = D / 32;          // 32-dim blocks of dK^T / dV^T
  constexpr int kHalf = 2 * kKC;       // products of S (dP) per tile = of dV (dK) = D / 8
  constexpr int kPhase = 2 * kHalf;    // products per matrix phase
  constexpr int kRing = 8;             // LDS operands in flight
  static_assert(4 * kDB == kHalf, "dV / dK products per tile");
  static_assert(kRing <= kHalf, "the ring reaches at most into the next phase's first half");
  static_assert(kHalf % kRing == 0, "phases hold whole rings");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (kPairs - 1);
  const bool s_wave = wave < kPairs;   // wave-uniform
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int kb = blockIdx.x / p.BH;   // small key blocks (most work when causal) first
  const int bh = blockIdx.x % p.BH;
  const int k0 = kb * kBK;
  const int key = k0 + pair * kKW + r32;

  const unsigned head_q = (unsigned)p.Sq * G::kRowBytes;
  const unsigned head_k = (unsigned)p.Sk * G::kRowBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + (size_t)bh * p.Sq * D, head_q);
  // the row term a dP wave loads: LSE log2(e) (pair 0) or D (pair 1)
  const __amdgpu_buffer_rsrc_t rrow =
      make_rsrc((pair == 0 ? p.lse2 : p.dvec) + (size_t)bh * p.Sq, (unsigned)p.Sq * 4u);

  const int row_lane = row_lane_offset<D>(lane);
  const int tr_lane = tr_lane_offset<D>(lane);
  char* const pbuf = smem + L::kPOff + pair * L::kPPairBytes + lane * 16;   // + (4 b + i4) 1024

  // Tiles qt_lo .. n_qt-1.  qt_lo < n_qt always holds: causal requires
  // Sq == Sk and k0 < Sk, so k0 / kBQ <= (Sq - 1) / kBQ.
  const int n_qt = (p.Sq + kBQ - 1) / kBQ;
  const int qt_lo = CAUSAL ? k0 / kBQ : 0;
  const int n = n_qt - qt_lo;

  // the Q tile, the dO tile and the row terms (LSE log2(e), then D) of stage s
  auto qtile = [&](int s) __attribute__((always_inline)) -> char* { return smem + L::kQOff + s * L::kTileBytes; };
  auto otile = [&](int s) __attribute__((always_inline)) -> char* { return smem + L::kDoOff + s * L::kTileBytes; };
  auto rows = [&](int s) __attribute__((always_inline)) -> float* {
    return reinterpret_cast<float*>(smem + L::kRowsOff + s * L::kRowsBytes);
  };
  // the loads of relative tile t into stage S, issued by the dP waves only:
  // each its share of the Q and dO tiles, pairs 0 and 1 a row term
  auto issue = [&](int t, auto stage_tag) __attribute__((always_inline)) {
    constexpr int st = decltype(stage_tag)::value;
    const int q0 = (qt_lo + t) * kBQ;
    TileDMA<D, kBQ, kPairs>::load(rq, q0, qtile(st), pair, lane);
    TileDMA<D, kBQ, kPairs>::load(rdo, q0, otile(st), pair, lane);
    if (pair < 2) lds_dma4(rrow, (unsigned)(q0 + lane) * 4, rows(st) + pair * kBQ);
  };

  // B operands: the lane's K row (S wave) or V row (dP wave), dims
  // 16 kc + 8 g .. +8, loaded ahead of the tiles
  const __amdgpu_buffer_rsrc_t rkv = make_rsrc((s_wave ? p.k : p.v) + (size_t)bh * p.Sk * D, head_k);
  bf16x8 kvf[kKC];
#pragma unroll
  for (int kc = 0; kc < kKC; ++kc)
    kvf[kc] = __builtin_bit_cast(bf16x8, load16(rkv, (unsigned)key * G::kRowBytes + (kc * 16 + 8 * g) * 2));

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  static_assert(kStages == 3, "stage constants below assume three stages");
  static_assert(kBK / kBQ == 2, "two masked tiles per causal key block");

  // ---- prologue: tiles 0 and 1 in flight; wait for tile 0
  if (!s_wave) {
    issue(0, S0{});
    if (n > 1) {
      issue(1, S1{});
      if (pair < 2) wait_vmcnt<L::kTileLoads + 1>();
      else wait_vmcnt<L::kTileLoads>();
    } else {
      wait_vmcnt<0>();
    }
  }
  lds_barrier();

  // phase barriers.  After A: the dP wave has used P(k) (its uses come
  // before), so the S wave may overwrite it.  After B: P(k + 1) written
  // (the S wave waits for its LDS writes), tile k + 2 landed (the dP waves
  // wait for their loads; nothing later is in flight), tile k read by both.
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto barrier_tiles = [&](auto lds_writes) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(lds_writes)::value) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // The matrix phases: the prelude's kHalf products (S(0) or dP(0)), then
  // full phases of kHalf products of dV / dK for tile k and kHalf of S / dP
  // for tile k + 1.  The ring holds the operands of the next products; past
  // the phase's end they are the first products of the next phase (dV / dK
  // of the following tile, always published by then).
  using RS = RowStore<D>;
  static_assert(kWaves * RS::kBytes <= L::kLdsBytes, "output staging exceeds the LDS ring");

  if (s_wave) {
    // ================================================= S wave: S, P, dV
    const bf16x8* kf = kvf;
    f32x16 dv[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      dv[db] = f32x16{};
      asm volatile("s_nop 1" : "+v"(dv[db]));
    }
    // the products of a tile (row reads of Q for S; dO transposed for dV).
    // Each kind's base is folded into the lane offset (it shares no bit
    // with the lane offsets or the constants they are XORed with), hidden
    // from the compiler so that a read is one lane register plus the
    // stage's immediate offset.
    int rl = row_lane + L::kQOff, tl = tr_lane + L::kDoOff;
    asm volatile("" : "+v"(rl), "+v"(tl));
    auto op_s = [&](int st, int j) __attribute__((always_inline)) -> bf16x8 {
      return read_rows<D>(smem + st * L::kTileBytes, rl, j / kKC, j % kKC);
    };
    auto op_v = [&](int st, int j) __attribute__((always_inline)) -> bf16x8 {
      return read_cols<D>(smem + st * L::kTileBytes, tl, j / kDB, j % kDB);
    };
    bf16x8 ring[kRing];
    f32x16 s[2];
    bf16x8 bp[4];
    f32x4 lse[8];   // LSE log2(e) of the next P's rows, read ahead
#pragma unroll
    for (int j = 0; j < kRing; ++j) ring[j] = op_s(0, j);

    // a matrix phase: NV (0 or kHalf) products of dV for the tile in stage
    // CUR, then kHalf of S for the tile in stage NXT; operands past the end
    // are the next phase's first dV operands (tile in NXT).  Near its end
    // the rows' LSE of the tile in NXT is read for the P that follows.
    auto mphase = [&](auto nv_tag, auto cur_tag, auto nxt_tag) __attribute__((always_inline)) {
      constexpr int NV = decltype(nv_tag)::value;
      constexpr int kN = NV + kHalf;
      constexpr int cur = decltype(cur_tag)::value;
      constexpr int nxt = decltype(nxt_tag)::value;
      // operand o of this phase
      auto op = [&](int o) __attribute__((always_inline)) -> bf16x8 {
        return o < NV ? op_v(cur, o) : op_s(nxt, o - NV);
      };
      static_for<kN>([&](auto J) __attribute__((always_inline)) {
        constexpr int j = J;
        if constexpr (j == kN - kRing) {
          static_for<8>([&](auto X) __attribute__((always_inline)) {
            constexpr int x = X;   // elements 4 (x % 4) .. +3 of block x / 4
            lse[x] = *reinterpret_cast<const f32x4*>(rows(nxt) + 32 * (x / 4) + 8 * (x % 4) + 4 * g);
          });
        }
        const bf16x8 a = ring[j % kRing];
        constexpr int jn = j + kRing;
        if constexpr (jn < kN) ring[j % kRing] = op(jn);
        else if constexpr (jn - kN < kRing) ring[j % kRing] = op_v(nxt, jn - kN);
        if constexpr (j < NV) {
          MfmaAsm<'v', 'v'>::acc_v(dv[j % kDB], a, bp[j / kDB]);
        } else {
          constexpr int b = (j - NV) / kKC, kc = (j - NV) % kKC;
          if constexpr (kc == 0) MfmaAsm<'v', 'v'>::init_v(s[b], a, kf[0]);
          else MfmaAsm<'v', 'v'>::acc_v(s[b], a, kf[kc]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // P of relative tile t: float32 to LDS, bf16 into bp
    auto vphase = [&](int t, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // causal: element i of block b is masked iff key - q0 - 32 b - 4 g > 8 (i / 4) + i % 4
      const int delta0 = key - (qt_lo + t) * kBQ - 4 * g;
      mfma_drain_v2(s[0], s[1]);
      static_for<2>([&](auto B) __attribute__((always_inline)) {
        constexpr int b = B;
        float pe[16];
        static_for<4>([&](auto I4) __attribute__((always_inline)) {
          constexpr int i4 = I4;
          const f32x4 l4 = lse[4 * b + i4];
          static_for<4>([&](auto U) __attribute__((always_inline)) {
            constexpr int u = U, i = 4 * i4 + u;
            float x = __builtin_fmaf(s[b][i], p.scale_log2, -l4[u]);
            if (MASK && delta0 - 32 * b > 8 * i4 + u) x = kNegInf;
            pe[i] = exp2_hw(x);
          });
          *reinterpret_cast<f32x4*>(pbuf + (4 * b + i4) * 1024) =
              f32x4{pe[4 * i4], pe[4 * i4 + 1], pe[4 * i4 + 2], pe[4 * i4 + 3]};
          // each write in place, between its elements' arithmetic: the
          // compiler would gather them into bursts, which stall the other
          // wave's operand reads (measured: ~250 cycles more per tile)
          __builtin_amdgcn_sched_barrier(0);
        });
        bp[2 * b] = pack_bf16x8(pe[0], pe[1], pe[2], pe[3], pe[4], pe[5], pe[6], pe[7]);
        bp[2 * b + 1] = pack_bf16x8(pe[8], pe[9], pe[10], pe[11], pe[12], pe[13], pe[14], pe[15]);
      });
      // two wait states before a product reads them
      asm volatile("s_nop 1" ::"v"(bp[0]), "v"(bp[1]), "v"(bp[2]), "v"(bp[3]));
    };
    using Z = std::integral_constant<int, 0>;
    using H = std::integral_constant<int, kHalf>;
    // prelude: S(0) | P(0)
    mphase(Z{}, S0{}, S0{});
    barrier();
    vphase(0, std::integral_constant<bool, CAUSAL>{});
    barrier_tiles(std::true_type{});
    // interval k: A(k) = dV(k), S(k + 1) | B(k) = P(k + 1)
    auto interval = [&](int k, auto mask_tag, auto st_tag) __attribute__((always_inline)) {
      constexpr int c = decltype(st_tag)::value;
      using C1 = std::integral_constant<int, (c + 1) % kStages>;
      mphase(H{}, st_tag, C1{});
      barrier();
      vphase(k + 1, mask_tag);
      barrier_tiles(std::true_type{});
    };
    // P(1) is the last masked tile when causal
    interval(0, std::integral_constant<bool, CAUSAL>{}, S0{});
    int k = 1;
    while (k < n) {
      interval(k, std::false_type{}, S1{});
      if (++k >= n) break;
      interval(k, std::false_type{}, S2{});
      if (++k >= n) break;
      interval(k, std::false_type{}, S0{});
      ++k;
    }

    // ---- dV = (dV^T)^T -> bf16 (lane = key), whole-row stores through LDS
#pragma unroll
    for (int db = 0; db < kDB; ++db) mfma_drain_v(dv[db]);
    dma_barrier();
    RS::store(smem + wave * RS::kBytes, dv, 1.0f, p.dv + (size_t)bh * p.Sk * D, k0 + pair * kKW, p.Sk, lane);
  } else {
    // ================================================ dP wave: dP, dS, dK
    const bf16x8* vf = kvf;
    f32x16 dk[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      dk[db] = f32x16{};
      asm volatile("s_nop 1" : "+v"(dk[db]));
    }
    // DS: the lane's dS values of a 16-row step (rows 8 (j / 4) + 4 g + j % 4,
    // j < 8) are half g of its key's record in the step's position group of
    // the tile's 128-row query block: one 16-byte buffer store whose per-tile
    // part is a scalar offset
    const size_t ds_slab = (size_t)p.ds_rows * kDsPositions;
    const __amdgpu_buffer_rsrc_t rds = make_rsrc(DS ? p.ds + (size_t)bh * p.ds_nqb * ds_slab : nullptr,
                                                 DS ? (unsigned)(p.ds_nqb * ds_slab * 2) : 0u);
    const int ds_lane = (key % kDsTileKeys) * kDsRecord + 16 * g;
    const int ds_tile = (k0 + pair * kKW) / kDsTileKeys;   // wave-uniform

    // the products of a tile (row reads of dO for dP; Q transposed for dK),
    // the kinds' bases folded into the lane offsets as in the S wave
    int rl = row_lane + L::kDoOff, tl = tr_lane + L::kQOff;
    asm volatile("" : "+v"(rl), "+v"(tl));
    auto op_p = [&](int st, int j) __attribute__((always_inline)) -> bf16x8 {
      return read_rows<D>(smem + st * L::kTileBytes, rl, j / kKC, j % kKC);
    };
    auto op_k = [&](int st, int j) __attribute__((always_inline)) -> bf16x8 {
      return read_cols<D>(smem + st * L::kTileBytes, tl, j / kDB, j % kDB);
    };
    bf16x8 ring[kRing];
    f32x16 dp[2];
    bf16x8 bs[4];
    f32x4 dr[8];   // D of the next dS's rows, read ahead
#pragma unroll
    for (int j = 0; j < kRing; ++j) ring[j] = op_p(0, j);

    // a matrix phase: NK (0 or kHalf) products of dK for the tile in CUR,
    // then kHalf of dP for the tile in NXT; operands past the end are the
    // next phase's first dK operands (tile in NXT).  Near its end the rows'
    // D of the tile in NXT is read for the dS that follows.
    auto mphase = [&](auto nk_tag, auto cur_tag, auto nxt_tag) __attribute__((always_inline)) {
      constexpr int NK = decltype(nk_tag)::value;
      constexpr int kN = NK + kHalf;
      constexpr int cur = decltype(cur_tag)::value;
      constexpr int nxt = decltype(nxt_tag)::value;
      auto op = [&](int o) __attribute__((always_inline)) -> bf16x8 {
        return o < NK ? op_k(cur, o) : op_p(nxt, o - NK);
      };
      static_for<kN>([&](auto J) __attribute__((always_inline)) {
        constexpr int j = J;
        if constexpr (j == kN - kRing) {
          static_for<8>([&](auto X) __attribute__((always_inline)) {
            constexpr int x = X;
            dr[x] = *reinterpret_cast<const f32x4*>(rows(nxt) + kBQ + 32 * (x / 4) + 8 * (x % 4) + 4 * g);
          });
        }
        const bf16x8 a = ring[j % kRing];
        constexpr int jn = j + kRing;
        if constexpr (jn < kN) ring[j % kRing] = op(jn);
        else if constexpr (jn - kN < kRing) ring[j % kRing] = op_k(nxt, jn - kN);
        if constexpr (j < NK) {
          MfmaAsm<'v', 'v'>::acc_v(dk[j % kDB], a, bs[j / kDB]);
        } else {
          constexpr int b = (j - NK) / kKC, kc = (j - NK) % kKC;
          if constexpr (kc == 0) MfmaAsm<'v', 'v'>::init_v(dp[b], a, vf[0]);
          else MfmaAsm<'v', 'v'>::acc_v(dp[b], a, vf[kc]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // dS of tile k from P in LDS and dP: bf16 into bs (and, DS, to the dS^T
    // buffer).  P is read first, in two batches, then the loads of tile
    // k + 2 are issued (memory-to-LDS loads hold up the issuing wave for a
    // while, here overlapping the P reads)
    auto vphase = [&](int k, auto load_stage) __attribute__((always_inline)) {
      f32x4 pl[8];
      static_for<4>([&](auto X) __attribute__((always_inline)) {
        pl[X] = *reinterpret_cast<const f32x4*>(pbuf + X * 1024);
      });
      if (k + 2 < n) issue(k + 2, load_stage);
      mfma_drain_v2(dp[0], dp[1]);
      static_for<2>([&](auto B) __attribute__((always_inline)) {
        constexpr int b = B;
        if constexpr (b == 0) {
          static_for<4>([&](auto X) __attribute__((always_inline)) {
            pl[4 + X] = *reinterpret_cast<const f32x4*>(pbuf + (4 + X) * 1024);
          });
        }
        float de[16];
        static_for<4>([&](auto I4) __attribute__((always_inline)) {
          constexpr int i4 = I4;
          const f32x4 pv = pl[4 * b + i4];
          const f32x4 d4 = dr[4 * b + i4];
          static_for<4>([&](auto U) __attribute__((always_inline)) {
            constexpr int u = U, i = 4 * i4 + u;
            de[i] = pv[u] * (dp[b][i] - d4[u]);
          });
        });
        bs[2 * b] = pack_bf16x8(de[0], de[1], de[2], de[3], de[4], de[5], de[6], de[7]);
        bs[2 * b + 1] = pack_bf16x8(de[8], de[9], de[10], de[11], de[12], de[13], de[14], de[15]);
        if constexpr (DS) {
          // each block's two dS steps stored as soon as they are packed.
          // Non-temporal stores: dS is read once, by the other kernel, and
          // left in the L2 it would evict the Q / dO tiles every key block
          // of the head re-reads
          const int q0 = (qt_lo + k) * kBQ;
          constexpr int kNonTemporal = 2;   // cache-policy bit of the buffer store
          static_for<2>([&](auto X) __attribute__((always_inline)) {
            constexpr int x = 2 * b + X;
            const int pg = (q0 % kDsPositions) / kDsGroup + x;
            const int soff = (q0 / kDsPositions) * p.ds_rows * (kDsPositions * 2) +
                             (ds_tile * (kDsPositions / kDsGroup) + pg) * (kDsTileBytes / (kDsPositions / kDsGroup));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, bs[x]), rds, ds_lane, soff, kNonTemporal);
          });
        }
      });
      asm volatile("s_nop 1" ::"v"(bs[0]), "v"(bs[1]), "v"(bs[2]), "v"(bs[3]));
    };
    using Z = std::integral_constant<int, 0>;
    using H = std::integral_constant<int, kHalf>;
    // prelude: (idle) | dP(0)
    barrier();
    mphase(Z{}, S0{}, S0{});
    barrier_tiles(std::false_type{});
    // interval k: A(k) = dS(k) | B(k) = dK(k), dP(k + 1)
    auto interval = [&](int k, auto st_tag) __attribute__((always_inline)) {
      constexpr int c = decltype(st_tag)::value;
      using C1 = std::integral_constant<int, (c + 1) % kStages>;
      using C2 = std::integral_constant<int, (c + 2) % kStages>;
      vphase(k, C2{});
      barrier();
      mphase(H{}, st_tag, C1{});
      barrier_tiles(std::false_type{});
    };
    interval(0, S0{});
    int k = 1;
    while (k < n) {
      interval(k, S1{});
      if (++k >= n) break;
      interval(k, S2{});
      if (++k >= n) break;
      interval(k, S0{});
      ++k;
    }

    // ---- dK = scale (dK^T)^T -> bf16 (lane = key), whole-row stores through LDS
#pragma unroll
    for (int db = 0; db < kDB; ++db) mfma_drain_v(dk[db]);
    dma_barrier();
    RS::store(smem + wave * RS::kBytes, dk, p.scale, p.dk + (size_t)bh * p.Sk * D, k0 + pair * kKW, p.Sk, lane);
  }
}

// ============================================================ dQ from dS
// Five-product form: dQ = scale dS K from the dS^T buffer (layout above) and
// K.  A workgroup owns one slab (128 query rows) and streams 64-key tiles of
// K and of the slab, memory-to-LDS, through a ring of kStages stages issued
// kStages - 1 tiles ahead.  Eight waves, two per SIMD: wave w takes positions
// 32 (w % 4) .. +32 and the half h = w / 4 of the D dims; per tile
//   dQ^T (D/2 x 32) += K^T (dims of half h x 64 keys) . dS^T (64 keys x 32),
// both operands read transposed, so their k slots (keys) follow one order.
// (Two waves per SIMD: one issues its transposed LDS reads while the other
// waits on its own.)
// The K tile has the layout of fa_tiles.hpp.  The dS tile is the slab's 8
// groups x 64 records (2 KB per group); in odd groups record r holds key
// r ^ 4, so the two 16-lane halves of a transposed read pass (groups 2 w and
// 2 w + 1, same keys) meet opposite halves of the 64 banks.  A tile's loads
// are spread over its products (a memory-to-LDS load stalls the issuing
// wave for a while), and the K^T operands are read four products ahead (with
// one product's time between reads the kernel waited on LDS latency: MFMA
// busy 23 %, LDS active 15 %, and it ran as fast with no tile loads at all).
// The dS loads carry the non-temporal hint (dS is read once; K stays).
// Causal: the slab of block qb needs keys 0 .. 128 qb + 127 only (dS is zero
// past the diagonal, and those are exactly the tiles the dK/dV kernel
// wrote).  HBM-bound: dS is read once.
namespace dsk {
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kPosBlocks = 4;   // 32-position blocks of a slab
constexpr int kBN = 64;
constexpr int kStages = 4;
constexpr int kSlabTiles = kBN / kDsTileKeys;   // slab tiles per key tile
constexpr int kSBytes = kSlabTiles * kDsTileBytes;
constexpr int kSLoads = kSBytes / 1024 / kWaves;   // per wave
template <int D>
struct Layout {
  static constexpr int kKBytes = kBN * TileGeom<D>::kRowBytes;
  static constexpr int kStageBytes = kKBytes + kSBytes;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kKLoads = TileDMA<D, kBN, kWaves>::kLoads;
  static constexpr int kPer = kKLoads + kSLoads;
  static constexpr int kOutPitch = D * 2 + 16;   // output staging: bf16 rows padded by 16 bytes
};
}  // namespace dsk

template <int D, bool CAUSAL>
__global__ __launch_bounds__(dsk::kThreads, 1) void bwd_dq_ds_kernel(BwdParams p) {
  using namespace dsk;
  using L = Layout<D>;
  constexpr int kDBW = D / 64;                // 32-dim blocks per wave (half of D)
  constexpr int kPer = L::kPer;
  constexpr int kSteps = (kBN / 16) * kDBW;   // products per tile and wave
  constexpr int kAhead = 4;                   // K^T operands in flight
  static_assert(kPosBlocks * 32 == kDsPositions && kWaves == 2 * kPosBlocks, "two waves per position block");
  static_assert(kPer <= kSteps, "one load per product at most");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pw = wave % kPosBlocks, dh = wave / kPosBlocks;
  const int qb = p.ds_nqb - 1 - (int)blockIdx.x / p.BH;   // most key tiles first when causal
  const int bh = (int)blockIdx.x % p.BH;
  const int n_all = (p.Sk + kBN - 1) / kBN;
  const int n = CAUSAL ? min(n_all, (qb + 1) * (kDsPositions / kBN)) : n_all;

  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(p.k + (size_t)bh * p.Sk * D, (unsigned)p.Sk * TileGeom<D>::kRowBytes);
  const size_t slab = (size_t)p.ds_rows * kDsPositions;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.ds + ((size_t)bh * p.ds_nqb + qb) * slab, (unsigned)(slab * 2));
  // dims 32 (kDBW dh + j) .. +32 of the K^T operand: the transposed-read lane
  // offset XOR 64 (kDBW dh + j), the wave's part folded in once
  const int tr_k = tr_lane_offset<D>(lane) ^ (64 * kDBW * dh);
  // dS load i of this wave: 1 KB of LDS, blk = i kWaves + w: slab tile
  // kSlabTiles t + blk / 16, records 32 c .. +32 of its group pg (blk % 16 =
  // 2 pg + c); lane l fetches half l % 2 of record 32 c + l / 2.  The LDS
  // copy keeps the slab tiles' layout, one after the other.
  static_assert(kBN % kDsTileKeys == 0, "whole slab tiles per key tile");
  auto s_src = [&](int t, int i) __attribute__((always_inline)) -> unsigned {
    const int blk = i * kWaves + wave;
    const int st = kSlabTiles * t + blk / 16, b16 = blk % 16;
    const int pg = b16 >> 1;
    const int rec = ((b16 & 1) * 32 + (lane >> 1)) ^ (4 * (pg & 1));
    // a key past Sk (the zero-padded end of the last key block) gets an
    // offset past the buffer's end (2^31: beyond every slab, no 32-bit wrap),
    // so the load writes zeros: its dS, formed from zero K and V rows as
    // P = exp(-LSE) times (0 - D), need not be finite, and times its zero K
    // row would make dQ NaN
    if (st * kDsTileKeys + rec >= p.Sk) return 0x80000000u;
    return (unsigned)(st * kDsTileBytes + (pg * kDsTileKeys + rec) * kDsRecord + 16 * (lane & 1));
  };
  // B operand (dS^T, k = keys of step ks in accumulator order, n = position
  // 32 pw + lane % 32): two ds_read_b64_tr_b16 over 4 records x 16 positions of
  // group pg = 2 pw + h, h = (lane / 16) % 2; rows 16 ks + 4 g + s / 4 (and + 8)
  const int s16 = lane & 15, hh = (lane >> 4) & 1, gg = lane >> 5;
  const int tr_s = ((2 * pw + hh) * kDsTileKeys + 4 * (gg ^ hh) + (s16 >> 2)) * kDsRecord + 8 * (s16 & 3);
  auto read_s = [&](const char* stile, int ks) __attribute__((always_inline)) -> bf16x8 {
    constexpr int kStepsPerSlabTile = kDsTileKeys / 16;
    const char* base = stile + (ks / kStepsPerSlabTile) * kDsTileBytes + tr_s;
    const int kk = ks % kStepsPerSlabTile;
    const bf16x4_t lo = lds_read_tr16(base + 16 * kk * kDsRecord);
    const bf16x4_t hi = lds_read_tr16(base + (16 * kk + 8) * kDsRecord);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto load_one = [&](int t, int i) __attribute__((always_inline)) {
    char* st = smem + (t % kStages) * L::kStageBytes;
    if (i < L::kKLoads) {
      TileDMA<D, kBN, kWaves>::load_one(rk, t * kBN, st, wave, lane, i);
    } else {
      const int j = i - L::kKLoads;
      lds_dma16_stream(rs, s_src(t, j), st + L::kKBytes + (j * kWaves + wave) * 1024);
    }
  };

  f32x16 acc[kDBW];
#pragma unroll
  for (int j = 0; j < kDBW; ++j) acc[j] = f32x16{};

  constexpr int kLead = kStages - 1;   // tiles in flight ahead of the one in use
  static_for<kLead>([&](auto U) __attribute__((always_inline)) {
    if (U < n) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) load_one(U, i);
    }
  });
  for (int t = 0; t < n; ++t) {
    // tile t is complete once at most the loads of the (up to kLead - 1)
    // tiles issued after it are outstanding; the barrier also ends every
    // wave's reads of tile t - 1, whose stage tile t + kLead takes
    const int after = min(n - 1 - t, kLead - 1);
    static_for<kLead>([&](auto U) __attribute__((always_inline)) {
      if (after == U) wait_vmcnt<U * kPer>();
    });
    lds_barrier();
    const char* kt = smem + (t % kStages) * L::kStageBytes;
    const char* stile = kt + L::kKBytes;
    const bool more = t + kLead < n;
    // operands read kAhead products ahead (an LDS read takes several products'
    // time to return); the tile's four dS operands right after the barrier
    bf16x8 b[kBN / 16];
    bf16x8 a[kAhead];
    static_for<kBN / 16>([&](auto KS) __attribute__((always_inline)) { b[KS] = read_s(stile, KS); });
    static_for<kAhead>([&](auto J) __attribute__((always_inline)) {
      a[J] = read_cols<D>(kt, tr_k, J / kDBW, J % kDBW);
    });
    static_for<kSteps>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = J;
      constexpr int ks = j / kDBW, db = j % kDBW;
      const bf16x8 a_j = a[j % kAhead];
      if constexpr (j + kAhead < kSteps)
        a[j % kAhead] = read_cols<D>(kt, tr_k, (j + kAhead) / kDBW, (j + kAhead) % kDBW);
      constexpr int every = kSteps / kPer;
      if constexpr (j % every == 0 && j / every < kPer) {
        if (more) load_one(t + kLead, j / every);
      }
      acc[db] = mfma32x32x16(a_j, b[ks], acc[db]);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // dQ = scale (dQ^T)^T -> bf16.  In the MFMA C layout lane r + 32 g holds
  // position 32 pw + r' (r' = r with bits 2 and 3 exchanged: the row order of
  // the transposed dS^T reads) at dims 32 (kDBW dh + j) + 8 (i / 4) + 4 g + i % 4
  // of acc[j][i]; the slab's 128 x D rows are staged in LDS (8-byte writes,
  // rows padded so they meet every bank once per 16 rows), then stored 16
  // bytes per lane over whole rows, rows past Sq skipped
  static_assert(kDsPositions * L::kOutPitch <= L::kLdsBytes, "output staging exceeds the LDS ring");
  dma_barrier();
  {
    const int r = lane & 31, g = lane >> 5;
    char* srow = smem + (32 * pw + ((r & 19) | ((r & 4) << 1) | ((r & 8) >> 1))) * L::kOutPitch;
#pragma unroll
    for (int j = 0; j < kDBW; ++j)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v = {acc[j][4 * i4 + 0] * p.scale, acc[j][4 * i4 + 1] * p.scale, acc[j][4 * i4 + 2] * p.scale,
                         acc[j][4 * i4 + 3] * p.scale};
        *reinterpret_cast<bf16x4*>(srow + (32 * (kDBW * dh + j) + 8 * i4 + 4 * g) * 2) =
            __builtin_convertvector(v, bf16x4);
      }
  }
  lds_barrier();
  constexpr int kChunks = D / 8;   // 16-byte chunks per row
  static_assert(kDsPositions * kChunks % kThreads == 0, "whole chunks per thread");
  bf16* out = p.dq + (size_t)bh * p.Sq * D;
#pragma unroll
  for (int it = 0; it < kDsPositions * kChunks / kThreads; ++it) {
    const int q = it * kThreads + (int)threadIdx.x;
    const int row = q / kChunks, c = q % kChunks;
    const u32x4 val = *reinterpret_cast<const u32x4*>(smem + row * L::kOutPitch + c * 16);
    const int qrow = qb * kDsPositions + row;
    if (qrow < p.Sq) *reinterpret_cast<u32x4*>(out + (size_t)qrow * D + c * 8) = val;
  }
}

template <typename K>
hipError_t launch_dyn(K kern, dim3 grid, dim3 block, int lds, hipStream_t stream, const BwdParams& prm) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, block, lds, stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_all(const BwdArgs& a, BwdParams& prm, int phases, hipStream_t stream) {
  // workspace: D [B H Sq] then LSE log2(e) [B H Sq], each rounded to 256 bytes
  const size_t sec = ((size_t)a.B * a.H * a.Sq * sizeof(float) + 255) & ~size_t(255);
  prm.dvec = static_cast<float*>(a.workspace);
  prm.lse2 = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + sec);
  hipError_t e = hipSuccess;
  // PREPARE and DQ in one call: the dQ kernel forms the row terms of its own
  // rows (bit-identical to the prep kernel's) and stores them for DKDV
  const bool fuse = (phases & kBwdPrepare) && (phases & kBwdDq);
  prm.fuse_prep = fuse ? 1 : 0;
  if ((phases & kBwdPrepare) && !fuse) {
    const long long rows = (long long)a.B * a.H * a.Sq;
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(1024), dim3(256), 0, stream, prm, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kBwdDq) {
    const dim3 gq((unsigned)(((a.Sq + dqk::kBM - 1) / dqk::kBM) * prm.BH));
    e = a.causal
            ? launch_dyn(bwd_dq_kernel<D, true>, gq, dim3(dqk::kThreads), dqk::Layout<D>::kLdsBytes, stream, prm)
            : launch_dyn(bwd_dq_kernel<D, false>, gq, dim3(dqk::kThreads), dqk::Layout<D>::kLdsBytes, stream, prm);
    if (e != hipSuccess) return e;
  }
  if (phases & kBwdDkdv) {
    const dim3 gk((unsigned)(((a.Sk + kvk::kBK - 1) / kvk::kBK) * prm.BH));
    e = a.causal
            ? launch_dyn(bwd_dkdv_kernel<D, true>, gk, dim3(kvk::kThreads), kvk::Layout<D>::kLdsBytes, stream, prm)
            : launch_dyn(bwd_dkdv_kernel<D, false>, gk, dim3(kvk::kThreads), kvk::Layout<D>::kLdsBytes, stream, prm);
  }
  return e;
}

size_t ds_bytes(int B, int H, int Sq, int Sk) {
  const size_t nqb = (size_t)((Sq + kDsPositions - 1) / kDsPositions);
  const size_t rows = (size_t)((Sk + kvk::kBK - 1) / kvk::kBK) * kvk::kBK;
  return (size_t)B * H * nqb * rows * kDsPositions * sizeof(bf16);
}

template <int D>
hipError_t launch_ds(const BwdArgs& a, BwdParams& prm, int phases, hipStream_t stream) {
  // workspace: the row terms as in launch_all, then the dS^T slabs
  const size_t sec = ((size_t)a.B * a.H * a.Sq * sizeof(float) + 255) & ~size_t(255);
  prm.dvec = static_cast<float*>(a.workspace);
  prm.lse2 = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + sec);
  prm.ds = reinterpret_cast<bf16*>(static_cast<char*>(a.workspace) + 2 * sec);
  prm.ds_nqb = (a.Sq + kDsPositions - 1) / kDsPositions;
  prm.ds_rows = (a.Sk + kvk::kBK - 1) / kvk::kBK * kvk::kBK;
  prm.fuse_prep = 0;
  hipError_t e = hipSuccess;
  if (phases & kBwdPrepare) {
    const long long rows = (long long)a.B * a.H * a.Sq;
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(1024), dim3(256), 0, stream, prm, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kBwdDkdv) {
    const dim3 gk((unsigned)(((a.Sk + kvk::kBK - 1) / kvk::kBK) * prm.BH));
    e = a.causal ? launch_dyn(bwd_dkdv_kernel<D, true, true>, gk, dim3(kvk::kThreads), kvk::Layout<D>::kLdsBytes,
                              stream, prm)
                 : launch_dyn(bwd_dkdv_kernel<D, false, true>, gk, dim3(kvk::kThreads), kvk::Layout<D>::kLdsBytes,
                              stream, prm);
    if (e != hipSuccess) return e;
  }
  if (phases & kBwdDq) {
    const dim3 gq((unsigned)(prm.ds_nqb * prm.BH));
    e = a.causal ? launch_dyn(bwd_dq_ds_kernel<D, true>, gq, dim3(dsk::kThreads), dsk::Layout<D>::kLdsBytes,
                              stream, prm)
                 : launch_dyn(bwd_dq_ds_kernel<D, false>, gq, dim3(dsk::kThreads), dsk::Layout<D>::kLdsBytes,
                              stream, prm);
  }
  return e;
}

BwdParams make_params(const BwdArgs& a) {
  BwdParams prm{};
  prm.q = static_cast<const bf16*>(a.q);
  prm.k = static_cast<const bf16*>(a.k);
  prm.v = static_cast<const bf16*>(a.v);
  prm.o = static_cast<const bf16*>(a.o);
  prm.lse = a.lse;
  prm.dout = static_cast<const bf16*>(a.dout);
  prm.dq = static_cast<bf16*>(a.dq);
  prm.dk = static_cast<bf16*>(a.dk);
  prm.dv = static_cast<bf16*>(a.dv);
  prm.BH = a.B * a.H;
  prm.Sq = a.Sq;
  prm.Sk = a.Sk;
  prm.scale = a.scale;
  prm.scale_log2 = a.scale * kLog2e;
  return prm;
}

}  // namespace

// ------------------------------------------------- fixed scratch
// Scratch of the allocation-free backward: the row terms (D and LSE log2 e,
// the workspace of launch_bwd) of up to kScratchRows query rows, in a
// file-scope device array.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device, and is kept here.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t bwd_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t bwd_workspace_bytes(int B, int H, int Sq, int /*Sk*/, int /*d*/, bool /*deterministic*/) {
  return 2 * ((((size_t)B * H * Sq * sizeof(float)) + 255) & ~size_t(255));
}

hipError_t launch_bwd(const BwdArgs& a, int phases, hipStream_t stream) {
  BwdParams prm = make_params(a);
  return a.d == 64 ? launch_all<64>(a, prm, phases, stream) : launch_all<128>(a, prm, phases, stream);
}

size_t bwd_ds_workspace_bytes(int B, int H, int Sq, int Sk) {
  return bwd_workspace_bytes(B, H, Sq, Sk, 128, false) + ds_bytes(B, H, Sq, Sk);
}

hipError_t launch_bwd_ds(const BwdArgs& a, int phases, hipStream_t stream) {
  BwdParams prm = make_params(a);
  return a.d == 64 ? launch_ds<64>(a, prm, phases, stream) : launch_ds<128>(a, prm, phases, stream);
}

}  // namespace fa
