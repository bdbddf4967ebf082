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
// MI355X fp32 atomics to one accumulator from many XCDs run at ~1 TB/s, and
// ordering them serialises the key blocks of a head.  Here the backward is
// split by output instead, so every output element is written exactly once:
//   bwd_prep_kernel   D_i;
//   bwd_dq_kernel     a workgroup owns 256 query rows and streams K / V tiles:
//                     S^T = K Q^T, dP^T = V dO^T (one query per lane, so LSE_i
//                     and D_i are per-lane scalars), dS^T, dQ^T += K^T dS^T;
//   bwd_dkdv_kernel   a workgroup owns 128 key rows and streams Q / dO tiles:
//                     S = Q K^T, dP = dO V^T (one key per lane), P, dS,
//                     dV^T += dO^T P, dK^T += Q^T dS.
// That is seven products per tile pair instead of five, no atomics, no
// workspace beyond D, and results that are bit-identical run to run in both
// modes (the deterministic flag costs nothing).  Tiles use the layout of
// fa_tiles.hpp, so Q, dO, K and V are each read both row-wise and transposed
// from one LDS copy.

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
  int BH, Sq, Sk;
  float scale;
  float scale_log2;
};

// ------------------------------------------------------------------- prep
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
    if ((t % kTPR) == 0) p.dvec[row] = s;
  }
}

// ==================================================================== dQ
// 8 wavefronts x 32 query rows; the two groups of four (one wave of each per
// SIMD) alternate between a matrix phase and a vector phase as in the
// forward kernel, one barrier per phase, raised priority in matrix phases.
namespace dqk {
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;
constexpr int kBM = kWaves * kQW;
constexpr int kStages = 4;
constexpr int kAhead = 4;
template <int D>
struct Layout {
  // keys per tile: 32 at d = 128 keeps a wave within 256 registers
  static constexpr int kBN = D == 128 ? 32 : 64;
  static constexpr int kTileBytes = kBN * TileGeom<D>::kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;   // K then V
  static constexpr int kLdsBytes = kStages * kStageBytes;
};
}  // namespace dqk

template <int D, bool CAUSAL>
__global__ __launch_bounds__(dqk::kThreads, 1) void bwd_dq_kernel(BwdParams p) {
  using namespace dqk;
  using L = Layout<D>;
  using G = TileGeom<D>;
  constexpr int kBN = L::kBN;
  constexpr int kKB = kBN / 32;   // 32-key blocks per tile
  constexpr int kKS = kBN / 16;   // 16-key steps of K^T dS^T
  constexpr int kDB = D / 32;     // 32-dim blocks of dQ^T
  constexpr int kKC = D / 16;     // 16-dim steps of S^T and dP^T
  constexpr int kNQ = kKS * kDB;  // dQ products per tile
  constexpr int kNS = kKB * kKC;  // S^T (and as many dP^T) products per tile
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int n_qblocks = (p.Sq + kBM - 1) / kBM;
  const int rank = blockIdx.x / p.BH;
  const int bh = blockIdx.x % p.BH;
  const int qb = CAUSAL ? (n_qblocks - 1 - rank) : rank;

  const unsigned head_q = (unsigned)p.Sq * G::kRowBytes;
  const unsigned head_k = (unsigned)p.Sk * G::kRowBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (size_t)bh * p.Sk * D, head_k);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (size_t)bh * p.Sk * D, head_k);

  const int q_wave_lo = qb * kBM + wave * kQW;
  const int q_lane = q_wave_lo + r32;
  const int row_lane = row_lane_offset<D>(lane);
  const int tr_lane = tr_lane_offset<D>(lane);

  // B operands: Q^T and dO^T of the lane's query, dims 16 kc + 8 g .. +8
  bf16x8 qf[kKC], of[kKC];
#pragma unroll
  for (int kc = 0; kc < kKC; ++kc) {
    const unsigned off = (unsigned)q_lane * G::kRowBytes + (kc * 16 + 8 * g) * 2;
    qf[kc] = __builtin_bit_cast(bf16x8, load16(rq, off));
    of[kc] = __builtin_bit_cast(bf16x8, load16(rdo, off));
  }
  const bool q_ok = q_lane < p.Sq;
  const size_t qi = (size_t)bh * p.Sq + (q_ok ? q_lane : 0);
  const float lse2 = q_ok ? p.lse[qi] * kLog2e : __builtin_huge_valf();   // rows past the end: P = 0
  const float dval = q_ok ? p.dvec[qi] : 0.0f;

  const int kv_end = CAUSAL ? min(p.Sk, (qb + 1) * kBM) : p.Sk;
  const int n = (kv_end + kBN - 1) / kBN;
  const int n_wave = CAUSAL ? min(n, (q_wave_lo + kQW - 1) / kBN + 1) : n;

  f32x16 dq[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) dq[db] = f32x16{};
  f32x16 s[kKB], dp[kKB];
  bf16x8 pk[kKS];   // dS^T in bf16: B operands of K^T dS^T

  // ---- matrix phase: dQ^T += K_{t-1}^T dS_{t-1}^T, then S_t^T = K_t Q^T and
  // dP_t^T = V_t dO^T; one stream of MFMAs whose LDS operands are read
  // kAhead ahead through a register ring.
  auto matrix_body = [&](int t, auto with_dq, auto with_s) __attribute__((always_inline)) {
    constexpr bool DQ = decltype(with_dq)::value;
    constexpr bool SP = decltype(with_s)::value;
    constexpr int j0 = DQ ? 0 : kNQ;
    constexpr int j1 = SP ? kNQ + 2 * kNS : kNQ;
    const char* kprev = smem + ((t + kStages - 1) % kStages) * L::kStageBytes;
    const char* kcur = smem + (t % kStages) * L::kStageBytes;
    const char* vcur = kcur + L::kTileBytes;
    // j < kNQ: (ks, db) = (j / kDB, j % kDB); then pairs (S, dP) for (kc, kb)
    auto operand = [&](int j) __attribute__((always_inline)) -> bf16x8 {
      if (j < kNQ) return read_cols<D>(kprev, tr_lane, j / kDB, j % kDB);
      const int i = (j - kNQ) >> 1;
      const int kb = i % kKB, kc = i / kKB;
      return ((j - kNQ) & 1) ? read_rows<D>(vcur, row_lane, kb, kc) : read_rows<D>(kcur, row_lane, kb, kc);
    };
    if (SP) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
      }
    }
    bf16x8 ring[kAhead];
#pragma unroll
    for (int j = j0; j < j0 + kAhead && j < j1; ++j) ring[(j - j0) % kAhead] = operand(j);
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const bf16x8 a = ring[(j - j0) % kAhead];
      if (j + kAhead < j1) ring[(j - j0) % kAhead] = operand(j + kAhead);
      if (j < kNQ) {
        dq[j % kDB] = mfma32x32x16(a, pk[j / kDB], dq[j % kDB]);
      } else {
        const int i = (j - kNQ) >> 1;
        const int kb = i % kKB, kc = i / kKB;
        if ((j - kNQ) & 1) dp[kb] = mfma32x32x16(a, of[kc], dp[kb]);
        else s[kb] = mfma32x32x16(a, qf[kc], s[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto matrix = [&](int t, auto with_dq, auto with_s) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
    matrix_body(t, with_dq, with_s);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- vector phase: P^T and dS^T of tile t, packed to bf16
  auto vector = [&](int t) __attribute__((always_inline)) {
    if (t >= n_wave) return;
    const int k0 = t * kBN;
    const bool need_mask = (k0 + kBN > p.Sk) || (CAUSAL && k0 + kBN - 1 > q_wave_lo);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = exp2_hw(__builtin_fmaf(s[kb][i], p.scale_log2, -lse2));
        if (need_mask) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= p.Sk || (CAUSAL && key > q_lane)) pv = 0.0f;
        }
        s[kb][i] = pv * (dp[kb][i] - dval);
      }
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const int kb = ks >> 1, h = (ks & 1) * 8;
      pk[ks] = pack_bf16x8(s[kb][h], s[kb][h + 1], s[kb][h + 2], s[kb][h + 3], s[kb][h + 4], s[kb][h + 5],
                           s[kb][h + 6], s[kb][h + 7]);
    }
  };

  TileIO<D, kBN, kWaves> kio, vio;
  auto fetch = [&](int u) __attribute__((always_inline)) {
    if (u < n) {
      kio.fetch(rk, u * kBN, wave, lane);
      vio.fetch(rv, u * kBN, wave, lane);
    }
  };
  auto commit = [&](int u) __attribute__((always_inline)) {
    if (u < n) {
      char* st = smem + (u % kStages) * L::kStageBytes;
      kio.store(st, wave, lane);
      vio.store(st + L::kTileBytes, wave, lane);
    }
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto m_s = [&](int t) __attribute__((always_inline)) { matrix(t, std::false_type{}, std::true_type{}); };
  auto m_full = [&](int t) __attribute__((always_inline)) { matrix(t, std::true_type{}, std::true_type{}); };
  auto m_dq = [&](int t) __attribute__((always_inline)) { matrix(t, std::true_type{}, std::false_type{}); };

  fetch(0);
  commit(0);
  fetch(1);
  commit(1);
  barrier();

  // Same interval schedule as the forward kernel: group 0 runs matrix(t) in
  // interval 2t+1 and vector(t) in 2t+2; group 1 is one interval behind;
  // tile u is fetched in interval 2u-3 and written at the end of 2u-2.
  if (group == 0) {
    fetch(2);
    m_s(0);
    barrier();
    vector(0);
    commit(2);
    barrier();
    for (int t = 1; t < n_wave; ++t) {
      fetch(t + 2);
      m_full(t);
      barrier();
      vector(t);
      commit(t + 2);
      barrier();
    }
    if (n_wave < n) {
      fetch(n_wave + 2);
      m_dq(n_wave);
      barrier();
      commit(n_wave + 2);
      barrier();
      for (int t = n_wave + 1; t < n; ++t) {
        fetch(t + 2);
        barrier();
        commit(t + 2);
        barrier();
      }
      barrier();
      barrier();
    } else {
      m_dq(n);
      barrier();
      barrier();
    }
  } else {
    fetch(2);
    barrier();
    m_s(0);
    commit(2);
    barrier();
    fetch(3);
    vector(0);
    barrier();
    for (int t = 1; t < n_wave; ++t) {
      m_full(t);
      commit(t + 2);
      barrier();
      fetch(t + 3);
      vector(t);
      barrier();
    }
    if (n_wave < n) {
      m_dq(n_wave);
      commit(n_wave + 2);
      barrier();
      fetch(n_wave + 3);
      barrier();
      for (int t = n_wave + 1; t < n; ++t) {
        commit(t + 2);
        barrier();
        fetch(t + 3);
        barrier();
      }
      barrier();
    } else {
      m_dq(n);
      barrier();
    }
  }

  // ---- dQ = scale (dQ^T)^T -> bf16 (lane = query, 4 consecutive dims per group)
  if (q_ok) {
    bf16* row = p.dq + qi * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v4 = {dq[db][4 * i4] * p.scale, dq[db][4 * i4 + 1] * p.scale, dq[db][4 * i4 + 2] * p.scale,
                          dq[db][4 * i4 + 3] * p.scale};
        *reinterpret_cast<bf16x4*>(row + db * 32 + 8 * i4 + 4 * g) = __builtin_convertvector(v4, bf16x4);
      }
  }
}

// =================================================================== dK dV
// 4 wavefronts x 32 keys = 128 keys per workgroup; query tiles of 64 rows in
// a 2-stage LDS ring (register prefetch, one barrier per tile).
namespace kvk {
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKW = 32;
constexpr int kBK = kWaves * kKW;
constexpr int kBQ = 64;
constexpr int kStages = 2;
constexpr int kAhead = 4;
template <int D>
struct Layout {
  static constexpr int kTileBytes = kBQ * TileGeom<D>::kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytes + 2 * kBQ * 4;   // Q, dO, LSE*log2e, D
  static constexpr int kLdsBytes = kStages * kStageBytes;
};
}  // namespace kvk

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kvk::kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  using namespace kvk;
  using L = Layout<D>;
  using G = TileGeom<D>;
  constexpr int kKC = D / 16;   // 16-dim steps of S and dP
  constexpr int kDB = D / 32;   // 32-dim blocks of dK^T / dV^T
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int g = lane >> 5;

  const int kb = blockIdx.x / p.BH;   // small key blocks (most work when causal) first
  const int bh = blockIdx.x % p.BH;
  const int k0 = kb * kBK;
  const int k_wave_lo = k0 + wave * kKW;
  const int key = k_wave_lo + r32;

  const unsigned head_q = (unsigned)p.Sq * G::kRowBytes;
  const unsigned head_k = (unsigned)p.Sk * G::kRowBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + (size_t)bh * p.Sq * D, head_q);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (size_t)bh * p.Sk * D, head_k);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (size_t)bh * p.Sk * D, head_k);

  const int row_lane = row_lane_offset<D>(lane);
  const int tr_lane = tr_lane_offset<D>(lane);

  // B operands: the lane's K and V rows, dims 16 kc + 8 g .. +8
  bf16x8 kf[kKC], vf[kKC];
#pragma unroll
  for (int kc = 0; kc < kKC; ++kc) {
    const unsigned off = (unsigned)key * G::kRowBytes + (kc * 16 + 8 * g) * 2;
    kf[kc] = __builtin_bit_cast(bf16x8, load16(rk, off));
    vf[kc] = __builtin_bit_cast(bf16x8, load16(rv, off));
  }

  f32x16 dk[kDB], dv[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int n_qt = (p.Sq + kBQ - 1) / kBQ;
  const int qt_lo = CAUSAL ? k0 / kBQ : 0;

  TileIO<D, kBQ, kWaves> qio, oio;
  float rowval = 0.0f;   // tid < kBQ: LSE*log2e of a row; kBQ <= tid < 2 kBQ: D of a row
  auto fetch = [&](int qt) __attribute__((always_inline)) {
    qio.fetch(rq, qt * kBQ, wave, lane);
    oio.fetch(rdo, qt * kBQ, wave, lane);
    const int r = qt * kBQ + (tid & (kBQ - 1));
    const bool ok = r < p.Sq;
    const size_t ri = (size_t)bh * p.Sq + (ok ? r : 0);
    if (tid < kBQ) rowval = ok ? p.lse[ri] * kLog2e : __builtin_huge_valf();   // past the end: P = 0
    else if (tid < 2 * kBQ) rowval = ok ? p.dvec[ri] : 0.0f;
  };
  auto commit = [&](int stage) __attribute__((always_inline)) {
    char* st = smem + stage * L::kStageBytes;
    qio.store(st, wave, lane);
    oio.store(st + L::kTileBytes, wave, lane);
    if (tid < 2 * kBQ) reinterpret_cast<float*>(st + 2 * L::kTileBytes)[tid] = rowval;
  };

  if (qt_lo < n_qt) {
    fetch(qt_lo);
    commit(0);
  }
  lds_barrier();

  for (int qt = qt_lo; qt < n_qt; ++qt) {
    const int stage = (qt - qt_lo) & 1;
    const char* qtile = smem + stage * L::kStageBytes;
    const char* otile = qtile + L::kTileBytes;
    const float* rows = reinterpret_cast<const float*>(qtile + 2 * L::kTileBytes);
    const bool has_next = qt + 1 < n_qt;
    if (has_next) fetch(qt + 1);
    const int q0 = qt * kBQ;
    // causal: skip tiles whose rows all precede the wave's keys
    if (!CAUSAL || k_wave_lo <= q0 + kBQ - 1) {
      // Tile body as a short software pipeline over the two 32-row blocks b:
      //   (1) S_0, dP_0            (2) S_1, dP_1  | P_0, dS_0 (VALU)
      //   (3) dV, dK for rows 0-31 | P_1, dS_1    (4) dV, dK for rows 32-63
      // so each block's VALU work overlaps the other block's MFMAs; LDS
      // operands stream through a register ring.
      f32x16 s[2], dp[2];
      bf16x8 bp[kBQ / 16], bs[kBQ / 16];   // bf16 P and dS per 16-row step
      const bool need_mask = (CAUSAL && k_wave_lo + kKW - 1 > q0) || (k0 + kBK > p.Sk);
      // 2 kKC products: (S, dP) pairs over kc, alternating accumulators
      auto sdp = [&](int b) __attribute__((always_inline)) {
        s[b] = f32x16{};
        dp[b] = f32x16{};
        constexpr int kN = 2 * kKC;
        auto op = [&](int j) __attribute__((always_inline)) -> bf16x8 {
          return (j & 1) ? read_rows<D>(otile, row_lane, b, j >> 1) : read_rows<D>(qtile, row_lane, b, j >> 1);
        };
        bf16x8 ring[kAhead];
#pragma unroll
        for (int j = 0; j < kAhead; ++j) ring[j] = op(j);
#pragma unroll
        for (int j = 0; j < kN; ++j) {
          const bf16x8 a = ring[j % kAhead];
          if (j + kAhead < kN) ring[j % kAhead] = op(j + kAhead);
          if (j & 1) dp[b] = mfma32x32x16(a, vf[j >> 1], dp[b]);
          else s[b] = mfma32x32x16(a, kf[j >> 1], s[b]);
        }
      };
      // 2 kDB products per 16-row step, for steps ks0, ks0 + 1
      auto dkdv = [&](int ks0) __attribute__((always_inline)) {
        constexpr int kN = 2 * 2 * kDB;
        auto op = [&](int j) __attribute__((always_inline)) -> bf16x8 {
          const int ks = ks0 + (j / (2 * kDB)), db = (j >> 1) % kDB;
          return (j & 1) ? read_cols<D>(qtile, tr_lane, ks, db) : read_cols<D>(otile, tr_lane, ks, db);
        };
        bf16x8 ring[kAhead];
#pragma unroll
        for (int j = 0; j < kAhead; ++j) ring[j] = op(j);
#pragma unroll
        for (int j = 0; j < kN; ++j) {
          const bf16x8 a = ring[j % kAhead];
          if (j + kAhead < kN) ring[j % kAhead] = op(j + kAhead);
          const int ks = ks0 + (j / (2 * kDB)), db = (j >> 1) % kDB;
          if (j & 1) dk[db] = mfma32x32x16(a, bs[ks], dk[db]);
          else dv[db] = mfma32x32x16(a, bp[ks], dv[db]);
        }
      };
      auto mask = [&](int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = q0 + b * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if ((CAUSAL && key > q) || key >= p.Sk) s[b][i] = kNegInf;
        }
      };
      // P = exp2(s scale log2e - LSE log2e), dS = P (dP - D), packed to bf16
      auto pds = [&](int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r0 = b * 32 + 8 * i4 + 4 * g;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(rows + r0);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(rows + kBQ + r0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 4 * i4 + j;
            const float pv = exp2_hw(__builtin_fmaf(s[b][i], p.scale_log2, -l4[j]));
            s[b][i] = pv;
            dp[b][i] = pv * (dp[b][i] - d4[j]);
          }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int h = hh * 8;
          bp[2 * b + hh] = pack_bf16x8(s[b][h], s[b][h + 1], s[b][h + 2], s[b][h + 3], s[b][h + 4], s[b][h + 5],
                                       s[b][h + 6], s[b][h + 7]);
          bs[2 * b + hh] = pack_bf16x8(dp[b][h], dp[b][h + 1], dp[b][h + 2], dp[b][h + 3], dp[b][h + 4],
                                       dp[b][h + 5], dp[b][h + 6], dp[b][h + 7]);
        }
      };
      sdp(0);
      __builtin_amdgcn_sched_barrier(0);
      if (need_mask) mask(0);
      __builtin_amdgcn_sched_barrier(0);
      sdp(1);
      pds(0);
#pragma unroll
      for (int r = 0; r < 2 * kKC; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // 5 VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      if (need_mask) mask(1);
      __builtin_amdgcn_sched_barrier(0);
      dkdv(0);
      pds(1);
#pragma unroll
      for (int r = 0; r < 4 * kDB; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // 5 VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      dkdv(2);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (has_next) commit(stage ^ 1);
    lds_barrier();
  }

  // ---- dK = scale (dK^T)^T, dV = (dV^T)^T -> bf16 (lane = key)
  if (key < p.Sk) {
    bf16* dkr = p.dk + ((size_t)bh * p.Sk + key) * D;
    bf16* dvr = p.dv + ((size_t)bh * p.Sk + key) * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int c = db * 32 + 8 * i4 + 4 * g;
        const f32x4 a = {dk[db][4 * i4] * p.scale, dk[db][4 * i4 + 1] * p.scale, dk[db][4 * i4 + 2] * p.scale,
                         dk[db][4 * i4 + 3] * p.scale};
        const f32x4 b = {dv[db][4 * i4], dv[db][4 * i4 + 1], dv[db][4 * i4 + 2], dv[db][4 * i4 + 3]};
        *reinterpret_cast<bf16x4*>(dkr + c) = __builtin_convertvector(a, bf16x4);
        *reinterpret_cast<bf16x4*>(dvr + c) = __builtin_convertvector(b, bf16x4);
      }
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
  prm.dvec = static_cast<float*>(a.workspace);
  hipError_t e = hipSuccess;
  if (phases & kBwdPrepare) {
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

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int Sq, int /*Sk*/, int /*d*/, bool /*deterministic*/) {
  return (((size_t)B * H * Sq * sizeof(float)) + 255) & ~size_t(255);
}

hipError_t launch_bwd(const BwdArgs& a, int phases, hipStream_t stream) {
  BwdParams prm;
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
  return a.d == 64 ? launch_all<64>(a, prm, phases, stream) : launch_all<128>(a, prm, phases, stream);
}

}  // namespace fa
