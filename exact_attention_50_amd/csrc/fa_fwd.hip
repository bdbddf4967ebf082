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
//   * workgroup = 4 wavefronts x 32 query rows = 128 rows; grid over
//     (query block, head, batch), heaviest causal blocks first;
//   * S is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     Q^T is the B operand held in registers for the whole loop, K comes from
//     LDS as the A operand; each lane then owns 16 scores of ONE query per
//     32-key block, so the row max / sum need one exchange between the two
//     halves of the wave only (the analogue of the pages' one-thread-one-row
//     softmax);
//   * O^T = V^T P^T: the S^T accumulator, rounded to bf16, is already the B
//     operand (with the keys of each 16-key group in a fixed permuted order);
//     V is transposed into LDS on the way in, in the same permuted order, so
//     the A operand is one 16-byte LDS read per lane;
//   * K and V tiles are double-buffered in LDS; the next tile's global loads
//     are issued before the current tile's math and written to the other
//     buffer after it, one barrier per tile;
//   * LDS rows are padded by 16 bytes so the 16-byte MFMA operand reads of
//     32 consecutive rows hit distinct banks.

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;               // query rows per wavefront
constexpr int kBM = kWaves * kQW;     // query rows per workgroup
constexpr int kBN = 64;               // keys per tile

struct FwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int BH;            // B * H
  int Sq, Sk;
  int n_qblocks;
  float scale_log2;  // scale * log2(e)
  float tau;
};

template <int D>
struct FwdLayout {
  static constexpr int kKStride = D + 8;        // bf16 per K row in LDS
  static constexpr int kVStride = kBN + 8;      // bf16 per V^T row in LDS
  static constexpr int kKElems = kBN * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kStageElems = kKElems + kVElems;
  static constexpr int kKChunks = kBN * D / 8;  // 16-byte chunks of a K tile
  static constexpr int kKPerThread = kKChunks / kThreads;
  static constexpr int kVUnits = (kBN / 4) * (D / 8);   // 4 keys x 8 dims each
  static constexpr int kVPerThread = (kVUnits + kThreads - 1) / kThreads;
  static_assert(kKChunks % kThreads == 0, "K tile must split evenly");
};

template <int D>
struct TileRegs {
  u32x4 k[FwdLayout<D>::kKPerThread];
  u32x4 v[FwdLayout<D>::kVPerThread][4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const bf16* kh, const bf16* vh, int k0, int Sk,
                                          int tid) {
  using L = FwdLayout<D>;
#pragma unroll
  for (int i = 0; i < L::kKPerThread; ++i) {
    const int c = tid + i * kThreads;
    const int row = c / (D / 8);
    const int col = (c % (D / 8)) * 8;
    const int key = k0 + row;
    r.k[i] = key < Sk ? *reinterpret_cast<const u32x4*>(kh + (size_t)key * D + col) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < L::kVPerThread; ++i) {
    const int u = tid + i * kThreads;
    const int kq = u % (kBN / 4);
    const int dq = u / (kBN / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * kq + j;
      const bool ok = (u < L::kVUnits) && key < Sk;
      r.v[i][j] = ok ? *reinterpret_cast<const u32x4*>(vh + (size_t)key * D + 8 * dq) : u32x4{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, bf16* ks, bf16* vt, int tid) {
  using L = FwdLayout<D>;
#pragma unroll
  for (int i = 0; i < L::kKPerThread; ++i) {
    const int c = tid + i * kThreads;
    const int row = c / (D / 8);
    const int col = (c % (D / 8)) * 8;
    *reinterpret_cast<u32x4*>(ks + row * L::kKStride + col) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < L::kVPerThread; ++i) {
    const int u = tid + i * kThreads;
    if (u < L::kVUnits) {
      const int kq = u % (kBN / 4);
      const int dq = u / (kBN / 4);
      const int col = 16 * (kq / 4) + 4 * quad_slot(kq % 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // word w of each key row holds dims 8dq+2w (low half) and 8dq+2w+1 (high half)
        const uint32_t a = r.v[i][0][w], b = r.v[i][1][w], c2 = r.v[i][2][w], d2 = r.v[i][3][w];
        u32x2 even = {lo_pair(a, b), lo_pair(c2, d2)};
        u32x2 odd = {hi_pair(a, b), hi_pair(c2, d2)};
        *reinterpret_cast<u32x2*>(vt + (8 * dq + 2 * w) * L::kVStride + col) = even;
        *reinterpret_cast<u32x2*>(vt + (8 * dq + 2 * w + 1) * L::kVStride + col) = odd;
      }
    }
  }
}

template <int D, bool CAUSAL, int EMU>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdParams p) {
  using L = FwdLayout<D>;
  constexpr int kKB = kBN / 32;   // 32-key blocks per tile
  constexpr int kDB = D / 32;     // 32-dim blocks of the output
  constexpr int kKC = D / 16;     // 16-dim steps of Q K^T
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * L::kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  // heaviest causal query blocks are launched first; heads interleave so the
  // blocks of one head share an XCD's L2 (workgroups go round-robin to XCDs)
  const int rank = blockIdx.x / p.BH;
  const int bh = blockIdx.x % p.BH;
  const int qb = CAUSAL ? (p.n_qblocks - 1 - rank) : rank;

  const bf16* qh = p.q + (size_t)bh * p.Sq * D;
  const bf16* kh = p.k + (size_t)bh * p.Sk * D;
  const bf16* vh = p.v + (size_t)bh * p.Sk * D;

  const int q_wave_lo = qb * kBM + wave * kQW;
  const int q_lane = q_wave_lo + r32;

  // Q^T operand: lane holds Q[q_lane][16 kc + 8 g .. +8]
  bf16x8 qf[kKC];
#pragma unroll
  for (int kc = 0; kc < kKC; ++kc) {
    if (q_lane < p.Sq) {
      qf[kc] = *reinterpret_cast<const bf16x8*>(qh + (size_t)q_lane * D + kc * 16 + 8 * g);
    } else {
      qf[kc] = bf16x8{};
    }
  }

  const int kv_end = CAUSAL ? min(p.Sk, (qb + 1) * kBM) : p.Sk;
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  f32x16 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x16{};
  float m_ref = kNegInf;
  float l_part = 0.0f;

  TileRegs<D> regs;
  load_tile<D>(regs, kh, vh, 0, p.Sk, tid);
  store_tile<D>(regs, smem, smem + L::kKElems, tid);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    bf16* ks = smem + (t & 1) * L::kStageElems;
    bf16* vt = ks + L::kKElems;
    const bool has_next = t + 1 < n_tiles;
    if (has_next) load_tile<D>(regs, kh, vh, (t + 1) * kBN, p.Sk, tid);

    const int k0 = t * kBN;
    const bool active = !CAUSAL || k0 <= q_wave_lo + kQW - 1;
    if (active) {
      // ---- S^T = K Q^T for this tile: lane holds 16 keys per 32-key block
      f32x16 s[kKB];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        s[kb] = f32x16{};
        const bf16* krow = ks + (kb * 32 + r32) * L::kKStride + 8 * g;
#pragma unroll
        for (int kc = 0; kc < kKC; ++kc) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + kc * 16);
          s[kb] = mfma32x32x16(a, qf[kc], s[kb]);
        }
      }
      // ---- mask keys past the end and (causal) keys after the query
      const bool need_mask = (k0 + kBN > p.Sk) || (CAUSAL && k0 + kBN - 1 > q_wave_lo);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key >= p.Sk || (CAUSAL && key > q_lane)) s[kb][i] = kNegInf;
          }
      }
      // ---- row max: within the lane, then across the two wave halves
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, s[kb][i]);
      mx = __builtin_fmaxf(mx, swap_halves(mx));
      const float m_tile = mx * p.scale_log2;
      const float m_new = __builtin_fmaxf(m_ref, m_tile);
      // ---- conditional rescale: the branch is taken per wavefront (no
      // divergence); inside it only the rows whose max rose by more than tau
      // move their reference, the others multiply by exactly 1
      const bool need = (m_new - m_ref) > p.tau;   // first tile: +inf > tau
      if (__any(need)) {
        const float alpha = need ? exp2_hw(m_ref - m_new) : 1.0f;   // exp2(-inf) = 0
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; ++db) o[db] *= alpha;
        m_ref = need ? m_new : m_ref;
      }
      // ---- P = 2^(s * scale_log2 - m_ref); a fixed share in software
      const float neg_m = (m_ref == kNegInf) ? 0.0f : -m_ref;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = __builtin_fmaf(s[kb][i], p.scale_log2, neg_m);
          const float e = (kb * 16 + i < EMU) ? exp2_sw(x) : exp2_hw(x);
          s[kb][i] = e;
          l_part += e;
        }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int ks16 = 0; ks16 < kBN / 16; ++ks16) {
        const int kb = ks16 >> 1, h = (ks16 & 1) * 8;
        const bf16x8 b = pack_bf16x8(s[kb][h + 0], s[kb][h + 1], s[kb][h + 2], s[kb][h + 3], s[kb][h + 4],
                                     s[kb][h + 5], s[kb][h + 6], s[kb][h + 7]);
        const bf16* vrow = vt + r32 * L::kVStride + ks16 * 16 + 8 * g;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + db * 32 * L::kVStride);
          o[db] = mfma32x32x16(a, b, o[db]);
        }
      }
    }

    if (has_next) {
      bf16* ks_n = smem + ((t + 1) & 1) * L::kStageElems;
      store_tile<D>(regs, ks_n, ks_n + L::kKElems, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: O = O / l (bf16), LSE = (m_ref + log2 l) ln 2
  const float l = l_part + swap_halves(l_part);
  const float inv_l = 1.0f / l;
  if (q_lane < p.Sq) {
    bf16* orow = p.o + ((size_t)bh * p.Sq + q_lane) * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v4 = {o[db][4 * i4 + 0] * inv_l, o[db][4 * i4 + 1] * inv_l, o[db][4 * i4 + 2] * inv_l,
                          o[db][4 * i4 + 3] * inv_l};
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * i4 + 4 * g) = __builtin_convertvector(v4, bf16x4);
      }
    if (g == 0) p.lse[(size_t)bh * p.Sq + q_lane] = (m_ref + __builtin_log2f(l)) * kLn2;
  }
}

// Software-exponential counts per lane per tile that are instantiated.
constexpr int kEmuCounts[] = {0, 3, 8, 16, 32};

template <int D, bool CAUSAL>
hipError_t launch_d_causal(const FwdParams& prm, int emu, dim3 grid, hipStream_t stream) {
  switch (emu) {
    case 0: hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, 0>), grid, dim3(kThreads), 0, stream, prm); break;
    case 3: hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, 3>), grid, dim3(kThreads), 0, stream, prm); break;
    case 8: hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, 8>), grid, dim3(kThreads), 0, stream, prm); break;
    case 16: hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, 16>), grid, dim3(kThreads), 0, stream, prm); break;
    case 32: hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, 32>), grid, dim3(kThreads), 0, stream, prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int fwd_exps_per_lane_tile(int /*d*/) { return kBN / 32 * 16; }

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
  prm.lse = a.lse;
  prm.BH = a.B * a.H;
  prm.Sq = a.Sq;
  prm.Sk = a.Sk;
  prm.n_qblocks = (a.Sq + kBM - 1) / kBM;
  prm.scale_log2 = a.scale * kLog2e;
  prm.tau = a.tau;
  const dim3 grid((unsigned)(prm.n_qblocks * prm.BH));
  if (a.d == 64) {
    return a.causal ? launch_d_causal<64, true>(prm, a.emu_count, grid, stream)
                    : launch_d_causal<64, false>(prm, a.emu_count, grid, stream);
  }
  return a.causal ? launch_d_causal<128, true>(prm, a.emu_count, grid, stream)
                  : launch_d_causal<128, false>(prm, a.emu_count, grid, stream);
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
