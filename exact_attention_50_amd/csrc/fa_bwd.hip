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
// 4 wavefronts x 32 keys = 128 keys per workgroup (one wave per SIMD); query
// tiles of 64 rows.  Per tile a wave runs one fixed sequence of kSteps MFMAs,
//   [S, dP of rows 0-31] [S, dP of rows 32-63] [dV, dK of rows 0-31] [... 32-63]
// whose LDS operands stream through a ring of kRing registers that runs on
// across tiles, and whose P / dS arithmetic is spread element by element over
// the MFMAs of the following block.  Tiles arrive memory-to-LDS in a 3-stage
// ring, issued two tiles ahead; the one barrier per tile sits kRing steps
// before the tile's end, once every operand of the tile has been read.
namespace kvk {
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKW = 32;
constexpr int kBK = kWaves * kKW;
constexpr int kBQ = 64;
constexpr int kStages = 3;
constexpr int kRing = 8;
template <int D>
struct Layout {
  static constexpr int kTileBytes = kBQ * TileGeom<D>::kRowBytes;
  // Q, dO, then four 64-float row blocks: LSE*log2e, D (waves 0, 1) and the
  // same again (waves 2, 3 load a copy so every wave issues the same loads)
  static constexpr int kRowsOff = 2 * kTileBytes;
  static constexpr int kStageBytes = 2 * kTileBytes + 4 * kBQ * 4;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kLoadsPerTile = 2 * TileDMA<D, kBQ, kWaves>::kLoads + 1;   // per wave
};
}  // namespace kvk

// DS: also store the tile's bf16 dS (the five-product form).
template <int D, bool CAUSAL, bool DS = false>
__global__ __launch_bounds__(kvk::kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  using namespace kvk;
  using L = Layout<D>;
  using G = TileGeom<D>;
  constexpr int kKC = D / 16;               // 16-dim steps of S and dP
  constexpr int kDB = D / 32;               // 32-dim blocks of dK^T / dV^T
  constexpr int kNS = 2 * kKC;              // MFMAs of S and dP per 32-row block
  constexpr int kND = 2 * kDB;              // MFMAs of dV and dK per 16-row step
  constexpr int kSteps = 2 * kNS + 4 * kND;
  constexpr int kBar = kSteps - kRing;      // barrier position (before this step)
  // operand j of any tile sits in ring slot j % kRing only if every tile
  // starts on slot 0
  static_assert(kSteps % kRing == 0, "ring must divide the step count");
  constexpr int kPPS = D == 128 ? 1 : 2;    // P/dS elements per step
  constexpr int kPer = L::kLoadsPerTile;
  // the row terms of both blocks are read before the barrier frees the stage,
  // and every bf16 P / dS half is packed before its first dV / dK product
  static_assert(2 * kNS + 2 + 12 / kPPS - 3 < kBar, "row terms read after the barrier");
  static_assert(kNS + 2 + 7 / kPPS < 2 * kNS && kNS + 2 + 15 / kPPS < 2 * kNS + kND, "block 0 P/dS late");
  static_assert(2 * kNS + 2 + 7 / kPPS < 2 * kNS + 2 * kND && 2 * kNS + 2 + 15 / kPPS < 2 * kNS + 3 * kND,
                "block 1 P/dS late");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int kb = blockIdx.x / p.BH;   // small key blocks (most work when causal) first
  const int bh = blockIdx.x % p.BH;
  const int k0 = kb * kBK;
  const int key = k0 + wave * kKW + r32;

  const unsigned head_q = (unsigned)p.Sq * G::kRowBytes;
  const unsigned head_k = (unsigned)p.Sk * G::kRowBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (size_t)bh * p.Sk * D, head_k);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (size_t)bh * p.Sk * D, head_k);
  // row terms: waves 0 and 2 load LSE*log2e, waves 1 and 3 load D
  const __amdgpu_buffer_rsrc_t rrow =
      make_rsrc(((wave & 1) ? p.dvec : p.lse2) + (size_t)bh * p.Sq, (unsigned)p.Sq * 4u);

  const int row_lane = row_lane_offset<D>(lane);
  const int tr_lane = tr_lane_offset<D>(lane);

  // DS: the lane's dS values of a 16-row step (rows 8 (j / 4) + 4 g + j % 4,
  // j < 8) are half g of its key's record in the step's position group of
  // the tile's 128-row query block: one 16-byte buffer store whose per-tile
  // part is a scalar offset
  const size_t ds_slab = (size_t)p.ds_rows * kDsPositions;
  const __amdgpu_buffer_rsrc_t rds =
      make_rsrc(DS ? p.ds + (size_t)bh * p.ds_nqb * ds_slab : nullptr, DS ? (unsigned)(p.ds_nqb * ds_slab * 2) : 0u);
  const int ds_lane = (key % kDsTileKeys) * kDsRecord + 16 * g;
  const int ds_tile = (k0 + wave * kKW) / kDsTileKeys;   // wave-uniform

  // B operands: the lane's K and V rows, dims 16 kc + 8 g .. +8
  bf16x8 kf[kKC], vf[kKC];
#pragma unroll
  for (int kc = 0; kc < kKC; ++kc) {
    const unsigned off = (unsigned)key * G::kRowBytes + (kc * 16 + 8 * g) * 2;
    kf[kc] = __builtin_bit_cast(bf16x8, load16(rk, off));
    vf[kc] = __builtin_bit_cast(bf16x8, load16(rv, off));
    // only ever MFMA operands: keep them in the AGPR file (the s_nop covers
    // the wait states between the moves and a first product right after)
    asm volatile("s_nop 1" : "+a"(kf[kc]), "+a"(vf[kc]));
  }

  f32x16 dk[kDB], dv[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
    // the zeros are VALU writes: fix them here, two wait states ahead of the
    // first product (otherwise they sink next to it)
    asm volatile("s_nop 1" : "+a"(dk[db]), "+a"(dv[db]));
  }

  // Tiles qt_lo .. n_qt-1.  qt_lo < n_qt always holds: causal requires
  // Sq == Sk and k0 < Sk, so k0 / kBQ <= (Sq - 1) / kBQ.
  const int n_qt = (p.Sq + kBQ - 1) / kBQ;
  const int qt_lo = CAUSAL ? k0 / kBQ : 0;
  const int n = n_qt - qt_lo;

  // relative tile t lives in stage t % kStages; the stage is always a
  // compile-time constant below, so every LDS address is a loop-invariant
  // lane offset plus an immediate
  // memory-to-LDS loads of relative tile t into stage S: kPer per wave
  auto issue = [&](int t, auto stage_tag) __attribute__((always_inline)) {
    char* st = smem + decltype(stage_tag)::value * L::kStageBytes;
    const int q0 = (qt_lo + t) * kBQ;
    TileDMA<D, kBQ, kWaves>::load(rq, q0, st, wave, lane);
    TileDMA<D, kBQ, kWaves>::load(rdo, q0, st + L::kTileBytes, wave, lane);
    lds_dma4(rrow, (unsigned)(q0 + lane) * 4, st + L::kRowsOff + wave * kBQ * 4);
  };
  // load i (0 <= i < kPer) of relative tile t into stage S, issued one at a
  // time so that the loads of a tile spread over several MFMA steps
  auto issue_one = [&](int t, auto stage_tag, auto load_tag) __attribute__((always_inline)) {
    constexpr int i = decltype(load_tag)::value;
    constexpr int kL = TileDMA<D, kBQ, kWaves>::kLoads;
    char* st = smem + decltype(stage_tag)::value * L::kStageBytes;
    const int q0 = (qt_lo + t) * kBQ;
    if constexpr (i < kL) {
      TileDMA<D, kBQ, kWaves>::load_one(rq, q0, st, wave, lane, i);
    } else if constexpr (i < 2 * kL) {
      TileDMA<D, kBQ, kWaves>::load_one(rdo, q0, st + L::kTileBytes, wave, lane, i - kL);
    } else {
      lds_dma4(rrow, (unsigned)(q0 + lane) * 4, st + L::kRowsOff + wave * kBQ * 4);
    }
  };

  // operand j of a tile (j < 2 kNS: row reads of Q / dO for S / dP; then
  // transposed reads of dO / Q for dV / dK)
  auto op = [&](const char* st, int j) __attribute__((always_inline)) -> bf16x8 {
    const char* qtile = st;
    const char* otile = st + L::kTileBytes;
    if (j < 2 * kNS) {
      const int b = j / kNS, jj = j % kNS;
      return (jj & 1) ? read_rows<D>(otile, row_lane, b, jj >> 1) : read_rows<D>(qtile, row_lane, b, jj >> 1);
    }
    const int jj = j - 2 * kNS;
    const int ks = jj / kND, db = (jj >> 1) % kDB;
    return (jj & 1) ? read_cols<D>(qtile, tr_lane, ks, db) : read_cols<D>(otile, tr_lane, ks, db);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  static_assert(kStages == 3, "stage constants below assume three stages");

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
  for (int j = 0; j < kRing; ++j) ring[j] = op(smem, j);

  // One tile; MASK: apply the causal mask (only the first kBK / kBQ tiles of
  // a causal key block hold keys after some of their rows).
  // A tile's kPer loads: the first kRing (or all) in the steps after the
  // barrier of the tile three before it, the rest in the first steps of the
  // tile two before it (FIRST: tile 0, whose "tile two ahead" was loaded by
  // the prologue).
  constexpr int kEarly = kPer < kRing ? kPer : kRing;
  auto tile = [&](int t, auto first_tag, auto mask_tag, auto stage_tag) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int kS = decltype(stage_tag)::value;   // == t % kStages
    const char* cur = smem + kS * L::kStageBytes;
    const char* nxt = smem + ((kS + 1) % kStages) * L::kStageBytes;
    const int q0 = (qt_lo + t) * kBQ;
    const float* lrow = reinterpret_cast<const float*>(cur + L::kRowsOff);   // LSE*log2e
    const float* drow = lrow + kBQ;                                           // D
    f32x16 s[2], dp[2];
    bf16x8 bp[4], bs[4];      // bf16 P and dS of the four 16-row steps
    float pe[16], de[16];     // P and dS of the block in progress
    f32x4 l4[4], d4[4];       // LSE*log2e and D of its 16 rows
    // causal: element i of block b is masked iff key - q0 - 32 b - 4 g > 8 (i / 4) + i % 4
    const int delta0 = key - q0 - 4 * g;

    static_for<kSteps>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = J;
      if constexpr (j == kBar) {
        // every operand of tile t has been read; publish tile t + 1 (its
        // loads were all issued before tile t; the kPer loads of tile t + 2
        // may still run)
        if (t + 2 < n) wait_vmcnt<kPer>();
        else wait_vmcnt<0>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (j >= kBar && j - kBar < kEarly) {
        if (t + 3 < n) issue_one(t + 3, stage_tag, std::integral_constant<int, j - kBar>{});
      }
      if constexpr (!FIRST && j < kPer - kEarly) {
        if (t + 2 < n)
          issue_one(t + 2, std::integral_constant<int, (decltype(stage_tag)::value + 2) % kStages>{},
                    std::integral_constant<int, kEarly + j>{});
      }
      // DS: the four bf16 dS steps of this tile, after the barrier (so a
      // whole tile passes before the next vmcnt wait, which counts them too)
      // and before the next tile repacks them.  Non-temporal stores: dS is
      // read once, by the other kernel, and left in the L2 it would evict
      // the Q / dO tiles every key block of the head re-reads (measured:
      // +35 MiB of refetches per launch with ordinary stores)
      if constexpr (DS && j >= kSteps - 4) {
        constexpr int x = j - (kSteps - 4);
        constexpr int kNonTemporal = 2;   // cache-policy bit of the buffer store
        const int pg = (q0 % kDsPositions) / kDsGroup + x;
        const int soff = (q0 / kDsPositions) * p.ds_rows * (kDsPositions * 2) +
                         (ds_tile * (kDsPositions / kDsGroup) + pg) * (kDsTileBytes / (kDsPositions / kDsGroup));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, bs[x]), rds, ds_lane, soff, kNonTemporal);
      }
      const bf16x8 a = ring[j % kRing];
      if constexpr (j + kRing < kSteps) ring[j % kRing] = op(cur, j + kRing);
      else ring[j % kRing] = op(nxt, j + kRing - kSteps);
      // S, dP accumulate in VGPRs (read by the P / dS arithmetic), dK, dV in
      // AGPRs (read once, at the end); K and V are AGPR operands
      if constexpr (j < 2 * kNS) {
        constexpr int b = j / kNS, jj = j % kNS;
        if constexpr (jj < 2) {
          if constexpr (jj & 1) MfmaAsm<'v', 'a'>::init_v(dp[b], a, vf[jj >> 1]);
          else MfmaAsm<'v', 'a'>::init_v(s[b], a, kf[jj >> 1]);
        } else {
          if constexpr (jj & 1) MfmaAsm<'v', 'a'>::acc_v(dp[b], a, vf[jj >> 1]);
          else MfmaAsm<'v', 'a'>::acc_v(s[b], a, kf[jj >> 1]);
        }
      } else {
        constexpr int jj = j - 2 * kNS;
        constexpr int ks = jj / kND, db = (jj >> 1) % kDB;
        if constexpr (jj & 1) MfmaAsm<'v', 'v'>::acc_a(dk[db], a, bs[ks]);
        else MfmaAsm<'v', 'v'>::acc_a(dv[db], a, bp[ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // P / dS of block b, elements from step (b + 1) kNS + 2 on
      static_for<2>([&](auto B) __attribute__((always_inline)) {
        constexpr int b = B;
        constexpr int first = (b + 1) * kNS + 2;
        // row terms of elements 4 i4 .. 4 i4 + 3, three steps before their use
        static_for<4>([&](auto I4) __attribute__((always_inline)) {
          constexpr int i4 = I4;
          if constexpr (j == first + (4 * i4) / kPPS - 3) {
            l4[i4] = *reinterpret_cast<const f32x4*>(lrow + 32 * b + 8 * i4 + 4 * g);
            d4[i4] = *reinterpret_cast<const f32x4*>(drow + 32 * b + 8 * i4 + 4 * g);
          }
        });
        // the last S / dP products of block b were issued two and three steps ago
        if constexpr (j == first) mfma_drain_v2(s[b], dp[b]);
        static_for<kPPS>([&](auto U) __attribute__((always_inline)) {
          constexpr int i = (j - first) * kPPS + U;
          if constexpr (i >= 0 && i < 16) {
            float x = __builtin_fmaf(s[b][i], p.scale_log2, -l4[i >> 2][i & 3]);
            if (MASK && delta0 - 32 * b > 8 * (i >> 2) + (i & 3)) x = kNegInf;
            const float pv = exp2_hw(x);
            pe[i] = pv;
            de[i] = pv * (dp[b][i] - d4[i >> 2][i & 3]);
            if constexpr ((i & 7) == 7) {
              constexpr int h = i - 7;
              bp[2 * b + (i >> 3)] = pack_bf16x8(pe[h], pe[h + 1], pe[h + 2], pe[h + 3], pe[h + 4], pe[h + 5],
                                                 pe[h + 6], pe[h + 7]);
              bs[2 * b + (i >> 3)] = pack_bf16x8(de[h], de[h + 1], de[h + 2], de[h + 3], de[h + 4], de[h + 5],
                                                 de[h + 6], de[h + 7]);
              // keep this work at this step (the IR optimiser would sink it
              // next to the products that use it)
              asm volatile("" ::"v"(bp[2 * b + (i >> 3)]), "v"(bs[2 * b + (i >> 3)]));
            }
          }
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // tiles 0 and 1 (stages 0, 1; masked if causal), then the rest from stage
  // 2 on, three tiles per loop pass
  static_assert(kBK / kBQ == 2, "two masked tiles per causal key block");
  using M = std::integral_constant<bool, CAUSAL>;
  using F = std::false_type;
  using T = std::true_type;
  tile(0, T{}, M{}, S0{});
  if (n > 1) tile(1, F{}, M{}, S1{});
  int t = 2;
  while (t < n) {
    tile(t, F{}, F{}, S2{});
    if (++t >= n) break;
    tile(t, F{}, F{}, S0{});
    if (++t >= n) break;
    tile(t, F{}, F{}, S1{});
    ++t;
  }

  // ---- dK = scale (dK^T)^T, dV = (dV^T)^T -> bf16 (lane = key)
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    mfma_drain_a(dk[db]);
    mfma_drain_a(dv[db]);
  }
  // whole-row stores through LDS, once every wave has read its last tile
  using RS = RowStore<D>;
  static_assert(2 * kWaves * RS::kBytes <= L::kLdsBytes, "output staging exceeds the LDS ring");
  dma_barrier();
  RS::store(smem + wave * RS::kBytes, dk, p.scale, p.dk + (size_t)bh * p.Sk * D, k0 + wave * kKW, p.Sk, lane);
  RS::store(smem + (kWaves + wave) * RS::kBytes, dv, 1.0f, p.dv + (size_t)bh * p.Sk * D, k0 + wave * kKW, p.Sk,
            lane);
}

// ============================================================ dQ from dS
// Five-product form: dQ = scale dS K from the dS^T buffer (layout above) and
// K.  A workgroup owns one slab (128 query rows) and streams 64-key tiles of
// K and of the slab, memory-to-LDS, through a ring of kStages stages issued
// kStages - 1 tiles ahead; per tile and wave (positions 32 w .. +32):
//   dQ^T (D x 32) += K^T (D x 64 keys) . dS^T (64 keys x 32),
// both operands read transposed, so their k slots (keys) follow one order.
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
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
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
};
}  // namespace dsk

template <int D, bool CAUSAL>
__global__ __launch_bounds__(dsk::kThreads, 1) void bwd_dq_ds_kernel(BwdParams p) {
  using namespace dsk;
  using L = Layout<D>;
  constexpr int kDB = D / 32;
  constexpr int kPer = L::kPer;
  constexpr int kSteps = (kBN / 16) * kDB;   // products per tile and wave
  constexpr int kAhead = 4;                  // K^T operands in flight
  static_assert(kWaves * 32 == kDsPositions, "one 32-position block per wave");
  static_assert(kPer <= kSteps, "one load per product at most");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qb = p.ds_nqb - 1 - (int)blockIdx.x / p.BH;   // most key tiles first when causal
  const int bh = (int)blockIdx.x % p.BH;
  const int n_all = (p.Sk + kBN - 1) / kBN;
  const int n = CAUSAL ? min(n_all, (qb + 1) * (kDsPositions / kBN)) : n_all;

  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(p.k + (size_t)bh * p.Sk * D, (unsigned)p.Sk * TileGeom<D>::kRowBytes);
  const size_t slab = (size_t)p.ds_rows * kDsPositions;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.ds + ((size_t)bh * p.ds_nqb + qb) * slab, (unsigned)(slab * 2));
  const int tr_k = tr_lane_offset<D>(lane);
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
  // 32 w + lane % 32): two ds_read_b64_tr_b16 over 4 records x 16 positions of
  // group pg = 2 w + h, h = (lane / 16) % 2; rows 16 ks + 4 g + s / 4 (and + 8)
  const int s16 = lane & 15, hh = (lane >> 4) & 1, gg = lane >> 5;
  const int tr_s = ((2 * wave + hh) * kDsTileKeys + 4 * (gg ^ hh) + (s16 >> 2)) * kDsRecord + 8 * (s16 & 3);
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

  f32x16 acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) acc[db] = f32x16{};

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
      a[J] = read_cols<D>(kt, tr_k, J / kDB, J % kDB);
    });
    static_for<kSteps>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = J;
      constexpr int ks = j / kDB, db = j % kDB;
      const bf16x8 a_j = a[j % kAhead];
      if constexpr (j + kAhead < kSteps) a[j % kAhead] = read_cols<D>(kt, tr_k, (j + kAhead) / kDB, (j + kAhead) % kDB);
      constexpr int every = kSteps / kPer;
      if constexpr (j % every == 0 && j / every < kPer) {
        if (more) load_one(t + kLead, j / every);
      }
      acc[db] = mfma32x32x16(a_j, b[ks], acc[db]);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // dQ = scale (dQ^T)^T -> bf16; lane r + 32 g holds position 32 w + r, i.e.
  // query row 32 w + r with bits 2 and 3 exchanged
  static_assert(kWaves * RowStore<D>::kBytes <= L::kLdsBytes, "output staging exceeds the LDS ring");
  dma_barrier();
  RowStore<D>::store(smem + wave * RowStore<D>::kBytes, acc, p.scale, p.dq + (size_t)bh * p.Sq * D,
                     qb * kDsPositions + 32 * wave, p.Sq, lane, /*swap23=*/true);
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
