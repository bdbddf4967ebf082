// Fused exact-attention backward for gfx950.
//
// Method.  The gradients of O = softmax(scale Q K^T) V, with P recomputed
// from the forward's log-sum-exp, by five matrix products per tile (FA4 paper
// §3.2.1, Eq. 7-8, as summarised on "FlashAttention-4: Algorithm and Kernel
// Pipelining Co-Design for Asymmetric Hardware Scaling"):
//   S = Q K^T,  P = exp(scale S - LSE),  dP = dO V^T,  dS = P (dP - D),
//   dV += P^T dO,  dK += scale dS^T Q,  dQ += scale dS K,
// with D_i = sum_c dO_ic O_ic.  dQ is summed over key blocks in a float32
// accumulator; the deterministic mode fixes the order of those additions with
// a per-query-block turn counter (paper §1; the Korean summary of the paper,
// §2.2, describes a lock that orders the dQ atomic adds).
//
// Kernels (one launch sequence per call, all on the caller's stream):
//   bwd_prep     D_i, zeroed dQ accumulator, turn counters and work ticket;
//   bwd_main     persistent workgroups take (key block, head) items from an
//                atomic ticket; 4 wavefronts x 32 keys = 128 keys per item;
//                query blocks of 64 rows are visited in DESCENDING order so
//                that in the deterministic mode the items of one head meet
//                each query block one after another (j = 0, 1, 2, ...) and
//                waits stay short;
//   bwd_dq_out   dQ = bf16(scale * accumulator).
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, lane layout in fa_device.hpp):
//   S  = Q K^T    A = Q rows from LDS, B = the wave's K rows held in registers
//   dP = dO V^T   A = dO rows from LDS, B = the wave's V rows in registers
//     -> both accumulators hold one KEY per lane (16 query rows each);
//   dV^T += dO^T P   B = P straight from the accumulator; A = dO^T staged
//                    transposed in LDS in the accumulator's row order;
//   dK^T += Q^T dS   likewise with Q^T;
//   dQ  = dS K       dS goes through LDS (row-major, bf16); B = K^T staged
//                    once per item in LDS; each wave owns 32 rows x d/2.
//
// Deadlock freedom of the deterministic mode: an item only waits for the
// item of the same head with the next smaller key block, whose ticket is
// smaller, so it was claimed earlier by a workgroup that is running or done;
// by induction every wait ends.  Waits are also bounded: after a very long
// spin the workgroup records an error flag and proceeds (the result is then
// not reproducible, but the kernel terminates).

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBK = 128;   // keys per item (32 per wavefront)
constexpr int kBQ = 64;    // query rows per step
constexpr long long kSpinLimit = 1LL << 24;

struct WorkspaceLayout {
  size_t dqacc_off, dvec_off, turns_off, ctrl_off, total;
};

WorkspaceLayout workspace_layout(int B, int H, int Sq, int d) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  WorkspaceLayout w;
  const size_t rows = (size_t)B * H * Sq;
  const size_t n_qb = (size_t)B * H * ((Sq + kBQ - 1) / kBQ);
  w.dqacc_off = 0;
  w.dvec_off = up(rows * d * sizeof(float));
  w.turns_off = w.dvec_off + up(rows * sizeof(float));
  w.ctrl_off = w.turns_off + up(n_qb * sizeof(int));
  w.total = w.ctrl_off + 256;   // [0] work ticket, [1] error flag
  return w;
}

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
  float* dqacc;
  float* dvec;
  int* turns;
  int* ctrl;
  int BH, Sq, Sk;
  int n_qb, n_kb, n_items;
  float scale;
  float scale_log2;
};

template <int D>
struct BwdLayout {
  static constexpr int kRowStride = D + 8;     // Q, dO row-major [q][d]
  static constexpr int kTStride = kBQ + 8;     // Q^T, dO^T [d][q slot]
  static constexpr int kSStride = kBK + 8;     // dS [q][key]
  static constexpr int kKTStride = kBK + 8;    // K^T [d][key]
  static constexpr int kQ = 0;
  static constexpr int kDO = kQ + kBQ * kRowStride;
  static constexpr int kQT = kDO + kBQ * kRowStride;
  static constexpr int kDOT = kQT + D * kTStride;
  static constexpr int kDS = kDOT + D * kTStride;
  static constexpr int kKT = kDS + kBQ * kSStride;
  static constexpr int kEnd = kKT + D * kKTStride;          // bf16 elements
  static constexpr int kBytes = kEnd * 2 + 2 * kBQ * 4;     // + LSE*log2e, D
  // staging units of a Q / dO block: 4 rows x 8 dims
  static constexpr int kUnits = (kBQ / 4) * (D / 8);
  static constexpr int kUnitsPerThread = (kUnits + kThreads - 1) / kThreads;
  // staging units of the K^T block
  static constexpr int kKUnits = (kBK / 4) * (D / 8);
  static constexpr int kKUnitsPerThread = kKUnits / kThreads;
  static_assert(kKUnits % kThreads == 0, "K^T staging must split evenly");
};

// ------------------------------------------------------------------ prep
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p, long long rows, long long acc_vec4,
                                                      int n_turns) {
  // D_i = sum_c dO_ic O_ic: D/8 threads per row, 16 bytes each
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
  f32x4* acc = reinterpret_cast<f32x4*>(p.dqacc);
  for (long long t = gtid; t < acc_vec4; t += nthreads) acc[t] = f32x4{0, 0, 0, 0};
  for (long long t = gtid; t < n_turns; t += nthreads) p.turns[t] = 0;
  if (gtid < 64) p.ctrl[gtid] = 0;
}

// ------------------------------------------------------------- dQ out
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_out_kernel(BwdParams p, long long n_vec4) {
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nthreads = (long long)gridDim.x * blockDim.x;
  const f32x4* acc = reinterpret_cast<const f32x4*>(p.dqacc);
  for (long long t = gtid; t < n_vec4; t += nthreads) {
    const f32x4 a = acc[t] * p.scale;
    *reinterpret_cast<bf16x4*>(p.dq + t * 4) = __builtin_convertvector(a, bf16x4);
  }
}

// ------------------------------------------------------------- main
template <int D>
struct QBlockRegs {
  u32x4 q[BwdLayout<D>::kUnitsPerThread][4];
  u32x4 o[BwdLayout<D>::kUnitsPerThread][4];   // dO
  float lse2;    // LSE * log2(e) of row tid (tid < kBQ)
  float dval;    // D of row tid - kBQ (kBQ <= tid < 2 kBQ)
};

template <int D>
__device__ __forceinline__ void load_qblock(QBlockRegs<D>& r, const BwdParams& p, int bh, int q0, int tid) {
  using L = BwdLayout<D>;
  const bf16* qh = p.q + (size_t)bh * p.Sq * D;
  const bf16* oh = p.dout + (size_t)bh * p.Sq * D;
#pragma unroll
  for (int i = 0; i < L::kUnitsPerThread; ++i) {
    const int u = tid + i * kThreads;
    const int rq = u % (kBQ / 4);
    const int dq = u / (kBQ / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = q0 + 4 * rq + j;
      const bool ok = (u < L::kUnits) && row < p.Sq;
      r.q[i][j] = ok ? *reinterpret_cast<const u32x4*>(qh + (size_t)row * D + 8 * dq) : u32x4{0, 0, 0, 0};
      r.o[i][j] = ok ? *reinterpret_cast<const u32x4*>(oh + (size_t)row * D + 8 * dq) : u32x4{0, 0, 0, 0};
    }
  }
  if (tid < kBQ) {
    const int row = q0 + tid;
    // rows past the end get LSE = +inf, so their probabilities are exactly 0
    r.lse2 = row < p.Sq ? p.lse[(size_t)bh * p.Sq + row] * kLog2e : __builtin_huge_valf();
  } else if (tid < 2 * kBQ) {
    const int row = q0 + tid - kBQ;
    r.dval = row < p.Sq ? p.dvec[(size_t)bh * p.Sq + row] : 0.0f;
  }
}

template <int D>
__device__ __forceinline__ void store_qblock(const QBlockRegs<D>& r, bf16* smem, float* sf, int tid) {
  using L = BwdLayout<D>;
#pragma unroll
  for (int i = 0; i < L::kUnitsPerThread; ++i) {
    const int u = tid + i * kThreads;
    if (u < L::kUnits) {
      const int rq = u % (kBQ / 4);
      const int dq = u / (kBQ / 4);
      // row-major copies
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<u32x4*>(smem + L::kQ + (4 * rq + j) * L::kRowStride + 8 * dq) = r.q[i][j];
        *reinterpret_cast<u32x4*>(smem + L::kDO + (4 * rq + j) * L::kRowStride + 8 * dq) = r.o[i][j];
      }
      // transposed copies, rows of each 16-row group in accumulator order
      const int col = 16 * (rq / 4) + 4 * quad_slot(rq % 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        {
          const uint32_t a = r.q[i][0][w], b = r.q[i][1][w], c = r.q[i][2][w], d = r.q[i][3][w];
          *reinterpret_cast<u32x2*>(smem + L::kQT + (8 * dq + 2 * w) * L::kTStride + col) =
              u32x2{lo_pair(a, b), lo_pair(c, d)};
          *reinterpret_cast<u32x2*>(smem + L::kQT + (8 * dq + 2 * w + 1) * L::kTStride + col) =
              u32x2{hi_pair(a, b), hi_pair(c, d)};
        }
        {
          const uint32_t a = r.o[i][0][w], b = r.o[i][1][w], c = r.o[i][2][w], d = r.o[i][3][w];
          *reinterpret_cast<u32x2*>(smem + L::kDOT + (8 * dq + 2 * w) * L::kTStride + col) =
              u32x2{lo_pair(a, b), lo_pair(c, d)};
          *reinterpret_cast<u32x2*>(smem + L::kDOT + (8 * dq + 2 * w + 1) * L::kTStride + col) =
              u32x2{hi_pair(a, b), hi_pair(c, d)};
        }
      }
    }
  }
  if (tid < kBQ) sf[tid] = r.lse2;
  else if (tid < 2 * kBQ) sf[tid] = r.dval;
}

// K^T of the item's 128 keys into LDS, natural key order: kt[d][key].
template <int D>
__device__ __forceinline__ void stage_kt(const BwdParams& p, int bh, int k0, bf16* kt, int tid) {
  using L = BwdLayout<D>;
  const bf16* kh = p.k + (size_t)bh * p.Sk * D;
#pragma unroll
  for (int i = 0; i < L::kKUnitsPerThread; ++i) {
    const int u = tid + i * kThreads;
    const int kq = u % (kBK / 4);
    const int dq = u / (kBK / 4);
    u32x4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * kq + j;
      r[j] = key < p.Sk ? *reinterpret_cast<const u32x4*>(kh + (size_t)key * D + 8 * dq) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      *reinterpret_cast<u32x2*>(kt + (8 * dq + 2 * w) * L::kKTStride + 4 * kq) =
          u32x2{lo_pair(r[0][w], r[1][w]), lo_pair(r[2][w], r[3][w])};
      *reinterpret_cast<u32x2*>(kt + (8 * dq + 2 * w + 1) * L::kKTStride + 4 * kq) =
          u32x2{hi_pair(r[0][w], r[1][w]), hi_pair(r[2][w], r[3][w])};
    }
  }
}

template <int D, bool CAUSAL, bool DET>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdParams p) {
  using L = BwdLayout<D>;
  constexpr int kKC = D / 16;       // 16-dim steps of S and dP
  constexpr int kDB = D / 32;       // 32-dim blocks of dK^T / dV^T
  constexpr int kQDB = D / 64;      // 32-dim blocks of one wave's dQ slice
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  float* sf = reinterpret_cast<float*>(smem + L::kEnd);   // [0,64) LSE*log2e, [64,128) D
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int g = lane >> 5;

  for (;;) {
    if (tid == 0) s_item = atomicAdd(&p.ctrl[0], 1);
    __syncthreads();
    const int item = s_item;
    if (item >= p.n_items) break;
    const int kb = item / p.BH;            // small key blocks (most work when causal) first
    const int bh = item % p.BH;
    const int k0 = kb * kBK;
    const int key = k0 + wave * 32 + r32;  // this lane's key (B operand / accumulator column)

    // the wave's K and V rows as B operands: lane holds row `key`, dims 16kc + 8g .. +8
    bf16x8 kf[kKC], vf[kKC];
    {
      const bf16* kr = p.k + ((size_t)bh * p.Sk + key) * D + 8 * g;
      const bf16* vr = p.v + ((size_t)bh * p.Sk + key) * D + 8 * g;
#pragma unroll
      for (int kc = 0; kc < kKC; ++kc) {
        kf[kc] = key < p.Sk ? *reinterpret_cast<const bf16x8*>(kr + kc * 16) : bf16x8{};
        vf[kc] = key < p.Sk ? *reinterpret_cast<const bf16x8*>(vr + kc * 16) : bf16x8{};
      }
    }
    stage_kt<D>(p, bh, k0, smem + L::kKT, tid);

    f32x16 dk[kDB], dv[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      dk[db] = f32x16{};
      dv[db] = f32x16{};
    }

    // query blocks that see at least one of these keys, visited top down
    const int qb_lo = CAUSAL ? k0 / kBQ : 0;
    const int qb_hi = p.n_qb - 1;
    QBlockRegs<D> regs;
    if (qb_lo <= qb_hi) load_qblock<D>(regs, p, bh, qb_hi * kBQ, tid);
    __syncthreads();   // previous item done with LDS
    if (qb_lo <= qb_hi) store_qblock<D>(regs, smem, sf, tid);
    __syncthreads();

    for (int qb = qb_hi; qb >= qb_lo; --qb) {
      const int q0 = qb * kBQ;
      const bool has_next = qb - 1 >= qb_lo;
      if (has_next) load_qblock<D>(regs, p, bh, q0 - kBQ, tid);

      // ---- S = Q K^T and dP = dO V^T: 2 blocks of 32 query rows
      f32x16 s[2], dp[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b] = f32x16{};
        dp[b] = f32x16{};
        const bf16* qrow = smem + L::kQ + (b * 32 + r32) * L::kRowStride + 8 * g;
        const bf16* orow = smem + L::kDO + (b * 32 + r32) * L::kRowStride + 8 * g;
#pragma unroll
        for (int kc = 0; kc < kKC; ++kc) {
          s[b] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(qrow + kc * 16), kf[kc], s[b]);
          dp[b] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(orow + kc * 16), vf[kc], dp[b]);
        }
      }
      // ---- P and dS (lane = key, 16 query rows per block)
      const bool need_mask = (CAUSAL && q0 < k0 + kBK - 1) || key >= p.Sk;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r0 = b * 32 + 8 * i4 + 4 * g;   // first of 4 consecutive rows
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(sf + r0);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(sf + kBQ + r0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 4 * i4 + j;
            float pv = exp2_hw(__builtin_fmaf(s[b][i], p.scale_log2, -l4[j]));
            if (need_mask && ((CAUSAL && key > q0 + r0 + j) || key >= p.Sk)) pv = 0.0f;
            s[b][i] = pv;
            dp[b][i] = pv * (dp[b][i] - d4[j]);
          }
        }
      // ---- dS -> LDS (bf16, row-major [q][key]) for the dQ product
      {
        bf16* dsb = smem + L::kDS + wave * 32 + r32;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            dsb[(b * 32 + 8 * (i >> 2) + 4 * g + (i & 3)) * L::kSStride] = (bf16)dp[b][i];
      }
      // ---- dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
      for (int ks = 0; ks < kBQ / 16; ++ks) {
        const int b = ks >> 1, h = (ks & 1) * 8;
        const bf16x8 bp = pack_bf16x8(s[b][h], s[b][h + 1], s[b][h + 2], s[b][h + 3], s[b][h + 4], s[b][h + 5],
                                      s[b][h + 6], s[b][h + 7]);
        const bf16x8 bs = pack_bf16x8(dp[b][h], dp[b][h + 1], dp[b][h + 2], dp[b][h + 3], dp[b][h + 4],
                                      dp[b][h + 5], dp[b][h + 6], dp[b][h + 7]);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int off = (db * 32 + r32) * L::kTStride + ks * 16 + 8 * g;
          dv[db] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(smem + L::kDOT + off), bp, dv[db]);
          dk[db] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(smem + L::kQT + off), bs, dk[db]);
        }
      }
      __syncthreads();   // dS complete

      // ---- dQ slice of this wave: rows 32 (wave / 2) .. +32, dims (wave % 2) D/2 .. +D/2
      f32x16 dqp[kQDB];
      {
        const int qr = (wave >> 1) * 32;
        const int dc = (wave & 1) * (D / 2);
        const bf16* arow = smem + L::kDS + (qr + r32) * L::kSStride + 8 * g;
#pragma unroll
        for (int db = 0; db < kQDB; ++db) {
          dqp[db] = f32x16{};
          const bf16* brow = smem + L::kKT + (dc + db * 32 + r32) * L::kKTStride + 8 * g;
#pragma unroll
          for (int ks = 0; ks < kBK / 16; ++ks)
            dqp[db] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(arow + ks * 16),
                                   *reinterpret_cast<const bf16x8*>(brow + ks * 16), dqp[db]);
        }
      }
      int* turn = p.turns + (size_t)bh * p.n_qb + qb;
      if (DET) {
        if (tid == 0) {
          long long spins = 0;
          while (__hip_atomic_load(turn, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != kb) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > kSpinLimit) {
              __hip_atomic_store(&p.ctrl[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          }
        }
        __syncthreads();
      }
      {
        const int qr = (wave >> 1) * 32;
        const int dc = (wave & 1) * (D / 2);
        float* accb = p.dqacc + ((size_t)bh * p.Sq + q0 + qr) * D + dc + r32;
#pragma unroll
        for (int db = 0; db < kQDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = 8 * (i >> 2) + 4 * g + (i & 3);
            if (q0 + qr + row < p.Sq) unsafeAtomicAdd(accb + (size_t)row * D + db * 32, dqp[db][i]);
          }
      }
      if (DET) {
        __threadfence();
        __syncthreads();
        if (tid == 0) __hip_atomic_store(turn, kb + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();   // all LDS reads of this block done
      if (has_next) store_qblock<D>(regs, smem, sf, tid);
      __syncthreads();
    }

    // ---- dK = scale dK^T^T, dV = dV^T^T (lane = key; 4 consecutive dims per group)
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
}

template <int D, bool CAUSAL, bool DET>
hipError_t launch_main(const BwdParams& prm, hipStream_t stream, int n_cu) {
  using L = BwdLayout<D>;
  const int per_cu = (160 * 1024) / L::kBytes >= 2 ? 2 : 1;
  int grid = n_cu * per_cu;
  if (grid > prm.n_items) grid = prm.n_items;
  auto kern = bwd_main_kernel<D, CAUSAL, DET>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, L::kBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), L::kBytes, stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_all(const BwdArgs& a, BwdParams& prm, hipStream_t stream) {
  const WorkspaceLayout w = workspace_layout(a.B, a.H, a.Sq, D);
  char* ws = static_cast<char*>(a.workspace);
  prm.dqacc = reinterpret_cast<float*>(ws + w.dqacc_off);
  prm.dvec = reinterpret_cast<float*>(ws + w.dvec_off);
  prm.turns = reinterpret_cast<int*>(ws + w.turns_off);
  prm.ctrl = reinterpret_cast<int*>(ws + w.ctrl_off);
  const long long rows = (long long)a.B * a.H * a.Sq;
  const long long acc_vec4 = rows * D / 4;
  const int n_turns = prm.BH * prm.n_qb;

  int dev = 0, n_cu = 256;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;

  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(2048), dim3(256), 0, stream, prm, rows, acc_vec4, n_turns);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.causal) {
    e = a.deterministic ? launch_main<D, true, true>(prm, stream, n_cu) : launch_main<D, true, false>(prm, stream, n_cu);
  } else {
    e = a.deterministic ? launch_main<D, false, true>(prm, stream, n_cu)
                        : launch_main<D, false, false>(prm, stream, n_cu);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_out_kernel<D>, dim3(2048), dim3(256), 0, stream, prm, acc_vec4);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int Sq, int /*Sk*/, int d, bool /*deterministic*/) {
  return workspace_layout(B, H, Sq, d).total;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
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
  prm.n_qb = (a.Sq + kBQ - 1) / kBQ;
  prm.n_kb = (a.Sk + kBK - 1) / kBK;
  prm.n_items = prm.n_kb * prm.BH;
  prm.scale = a.scale;
  prm.scale_log2 = a.scale * kLog2e;
  return a.d == 64 ? launch_all<64>(a, prm, stream) : launch_all<128>(a, prm, stream);
}

}  // namespace fa
