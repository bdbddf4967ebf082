// Device-side building blocks shared by the forward and backward kernels
// (gfx950 / CDNA4, wave64).
//
// MFMA lane layout used throughout (v_mfma_f32_32x32x16_bf16, checked on the
// hardware): with lane l, g = l / 32 and r = l % 32,
//   A (32 x 16, rows x k):  lane holds A[r][8g .. 8g+7]
//   B (16 x 32, k x cols):  lane holds B[8g .. 8g+7][r]
//   C (32 x 32):            lane holds C[8(i/4) + 4g + (i%4)][r], i = 0..15
// so an accumulator column belongs to one lane pair (l, l^32).
#pragma once

#include <type_traits>
#include <utility>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exp2_poly.h"

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product written out as one instruction with the register file of
// every operand fixed ("v": VGPR, "a": AGPR), for loops where the register
// allocator would otherwise move accumulators between the two files.  The
// compiler does not know these are MFMAs, so two latencies it would cover
// are the caller's:
//   * a VALU write of an input needs two wait states before the MFMA reads
//     it: callers produce inputs well ahead (ring loads, packed P / dS), and
//     tests/test_kernel_asm.py checks the built code for such pairs;
//   * mfma_drain_*() (>= 20 wait states, tied to the accumulator so that no
//     read is scheduled above it) must separate the last product into an
//     accumulator from any VALU read of it.
// A product into the same accumulator as the previous one needs nothing
// (srcC is exactly the previous vdst).
template <char CA, char CB>
struct MfmaAsm;
#define FA_MFMA_ASM(CA, CB, SA, SB)                                                                      \
  template <>                                                                                            \
  struct MfmaAsm<CA, CB> {                                                                               \
    __device__ __forceinline__ static void init_v(f32x16& d, bf16x8 a, bf16x8 b) {                       \
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : SA(a), SB(b));        \
    }                                                                                                    \
    __device__ __forceinline__ static void acc_v(f32x16& d, bf16x8 a, bf16x8 b) {                        \
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : SA(a), SB(b));       \
    }                                                                                                    \
    __device__ __forceinline__ static void acc_a(f32x16& d, bf16x8 a, bf16x8 b) {                        \
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : SA(a), SB(b));       \
    }                                                                                                    \
  };
FA_MFMA_ASM('v', 'v', "v", "v")
FA_MFMA_ASM('v', 'a', "v", "a")
#undef FA_MFMA_ASM

__device__ __forceinline__ void mfma_drain_v(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc));
}
__device__ __forceinline__ void mfma_drain_v2(f32x16& a0, f32x16& a1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(a0), "+v"(a1));
}
__device__ __forceinline__ void mfma_drain_a(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(acc));
}

// Hardware 2^x (v_exp_f32).  -inf and inputs below the normal range give 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Software 2^x on the FMA pipes: Cody-Waite range reduction x = n + f with
// n = floor(x), f in [0, 1); 2^f by a degree-3 minimax polynomial with
// p(0) = 1 in Horner form (three FMAs); 2^n applied with ldexp.  Inputs below
// -126 (and -inf) give exactly 0, as the hardware exponential does.
// (FA4 paper §3.1.3, Table 2, as summarised on "FlashAttention-4: Algorithm
// and Kernel Pipelining Co-Design for Asymmetric Hardware Scaling".)
__device__ __forceinline__ float exp2_sw(float x) {
  const float xc = __builtin_fmaxf(x, -127.0f);
  const float f = __builtin_amdgcn_fractf(xc);
  const int n = (int)__builtin_floorf(xc);
  float p = __builtin_fmaf(FA_EXP2_D3_C3, f, FA_EXP2_D3_C2);
  p = __builtin_fmaf(p, f, FA_EXP2_D3_C1);
  p = __builtin_fmaf(p, f, 1.0f);
  const float r = __builtin_amdgcn_ldexpf(p, n);
  return x < -126.0f ? 0.0f : r;
}

// ---------------------------------------------------------------------------
// The online softmax of one key tile, shared by the bf16 and e4m3 forwards
// (FlashAttention-4 paper §3.1.4, Eq. 6, as summarised on "FlashAttention-4:
// Algorithm and Kernel Pipelining Co-Design for Asymmetric Hardware
// Scaling").  A wavefront holds S^T of KB 32-key blocks in the MFMA C layout:
// lane (r, g) holds 16 scores of query r per block, element i of block kb
// being key 32 kb + 8 (i / 4) + 4 g + i % 4 of the tile.  The kernels call
// these steps in order: mask (edge tiles only), row max, conditional
// rescale, exponentials with row sums; then each packs P for its products.

// x if C <= lim, else -inf: one compare into VCC and one select, so that a
// run of these keeps no lane masks alive in scalar registers.
template <int C>
__device__ __forceinline__ float keep_if_le(float x, int lim) {
  float r;
  asm("v_cmp_le_i32 vcc, %2, %3\n\tv_cndmask_b32 %0, %4, %1, vcc"
      : "=v"(r)
      : "v"(x), "i"(C), "v"(lim), "v"(kNegInf)
      : "vcc");
  return r;
}

// Causal / ragged-end mask: the keys a row sees form a prefix of the tile,
// so score (kb, i) is kept iff 32 kb + 8 (i / 4) + i % 4 <= lim, where lim is
// (the row's last visible key) - (tile's first key) - 4 g; masked scores
// become -inf (so their P is exactly 0).
template <int KB>
__device__ __forceinline__ void softmax_mask_prefix(f32x16 (&s)[KB], int lim);

// The row max of the raw scores over the lane pair (l, l ^ 32): 8 independent
// chains of v_max3_f32 (two scores per instruction), then a short tree.
template <int KB>
__device__ __forceinline__ float softmax_row_max(const f32x16 (&s)[KB]);

// The conditional rescale: m_new = max(m_ref, m_tile) (log2 units); if any
// row of the wavefront rose by more than tau over its reference (a
// wave-uniform branch, "gated at warp granularity"), rescale(alpha) applies
// alpha = 2^(m_ref - m_new) to this lane's running output and sums, where
// only the rows that rose by more than tau move their reference (the others
// get alpha = 1 exactly).  The first tile (m_ref = -inf) always takes it.
// Returns whether the branch was taken.
template <typename Rescale>
__device__ __forceinline__ bool softmax_conditional_rescale(float& m_ref, float m_tile, float tau,
                                                            Rescale&& rescale) {
  const float m_new = __builtin_fmaxf(m_ref, m_tile);
  const bool need = (m_new - m_ref) > tau;   // first tile: +inf > tau
  if (__any(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;   // 2^-inf = 0
    rescale(alpha);
    m_ref = need ? m_new : m_ref;
    return true;
  }
  return false;
}

// P = 2^(s c - m_ref) for every score (c: the score scale in log2 units) and
// the four partial row sums of this lane; the first EMU of every 32 scores of
// a lane (per 64 keys) use the software 2^x, the others v_exp_f32.
template <int KB, int EMU>
__device__ __forceinline__ void softmax_exp_rowsum(f32x16 (&s)[KB], float c, float m_ref, float (&l_part)[4]);

// Exchange a value with the other half of the wave (lane l <-> l ^ 32).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// max / sum of a value over the lane pair (l, l ^ 32), without LDS: after
// v_permlane32_swap the two results hold x[l % 32] and x[l % 32 + 32].
// max of three floats as one v_max3_f32 (no canonicalisation of the inputs;
// the operands here are never signalling NaNs)
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Buffer resource over `bytes` bytes at `base`: raw buffer loads beyond it
// return zeros, which replaces per-lane bounds branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each group of 16 lanes, source lane s supplies
// the address of 4 consecutive 16-bit values of row s/4, columns 4(s%4)..+3
// of a 4 x 16 block; lane i receives column i of the block, rows 0..3.
__device__ __forceinline__ bf16x4_t lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4_t*)(lds_addr));
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>) in order,
// every index a compile-time constant (unrolling that does not depend on the
// optimiser's size limits).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier that waits for this wave's LDS operations only (global
// prefetches stay in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Memory-to-LDS loads (buffer_load ... lds) written out as instructions.
// Lane i's bytes land at the LDS address in M0 plus 4 i (dword) or 16 i
// (dwordx4); M0 must be wave-uniform.  The compiler's own form of these loads
// makes it wait for every outstanding vector-memory load before any later
// LDS read that it cannot prove disjoint from the load's target, which in a
// ring of stages is every read, and so throws away the lead the loads were
// issued with.  Callers order the loads themselves: s_waitcnt vmcnt, then a
// barrier, before any wave reads what they wrote.  The s_nop is the wait
// state required between the write of M0 and its use by the load.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned voffset, const void* lds_dst) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(r), "{m0}"(lds_addr(lds_dst)) : "memory");
}
// The same with the non-temporal hint: data read once, so its lines are the
// first the L2 gives up (other data stays resident).
__device__ __forceinline__ void lds_dma16_stream(__amdgpu_buffer_rsrc_t r, unsigned voffset, const void* lds_dst) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :: "v"(voffset), "s"(r), "{m0}"(lds_addr(lds_dst)) : "memory");
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, unsigned voffset, const void* lds_dst) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(r), "{m0}"(lds_addr(lds_dst)) : "memory");
}

// Workgroup barrier that also waits for this wave's memory-to-LDS loads (and
// every other vector-memory load of the wave).
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A operand of v_mfma_f32_16x16x32_bf16 that turns it into per-query row
// sums of a 32x32x16 B operand (lane l = 32 g + r holding 8 values of query r).
// In the 16x16x32 product lane l supplies A row l % 16 at k-group l / 16 and
// B column l % 16 at k-group l / 16; the B k-groups 0 and 2 (lanes 0-15,
// 32-47) hold queries c = l % 16, groups 1 and 3 hold queries c + 16.  Row 0
// of the selector is one on groups 0 and 2, row 1 on groups 1 and 3, all
// other rows zero, so C[0][c] and C[1][c] (lane c < 16, elements 0 and 1)
// collect the sums of queries c and c + 16 and every other element stays 0.
__device__ __forceinline__ bf16x8 row_sum_selector(int lane) {
  const int row = lane & 15, kg = lane >> 4;
  const bool one = (row == 0 && (kg & 1) == 0) || (row == 1 && (kg & 1) == 1);
  const __bf16 v = one ? (__bf16)1.0f : (__bf16)0.0f;
  return bf16x8{v, v, v, v, v, v, v, v};
}

// Round eight floats to bf16 (nearest-even) and pack them as an MFMA operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                              float a6, float a7) {
  f32x8 v = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(v, bf16x8);
}

// Byte permutes that interleave the 16-bit halves of two words:
// lo_pair(a, b) = {a.lo, b.lo}, hi_pair(a, b) = {a.hi, b.hi}.
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// MFMA k-slot order.  In the C layout a lane holds, for i = 8h + j, the row
// 16h + 8(j/4) + 4g + (j%4); used as a B operand (k-slot 8g + j) the rows of
// each 16-row group therefore arrive with bits 2 and 3 of the offset
// swapped.  Tensors staged in LDS as the matching A operand store each
// group's 4-row quads at this position.
__device__ __forceinline__ int quad_slot(int quad_in_group) {
  return ((quad_in_group & 1) << 1) | ((quad_in_group >> 1) & 1);
}

template <int KB>
__device__ __forceinline__ void softmax_mask_prefix(f32x16 (&s)[KB], int lim) {
  static_for<KB * 16>([&](auto e) __attribute__((always_inline)) {
    constexpr int kb = decltype(e)::value / 16, i = decltype(e)::value % 16;
    s[kb][i] = keep_if_le<kb * 32 + 8 * (i >> 2) + (i & 3)>(s[kb][i], lim);
  });
}

template <int KB>
__device__ __forceinline__ float softmax_row_max(const f32x16 (&s)[KB]) {
  constexpr int kPerChain = KB * 16 / 8;
  auto score = [&](int e) __attribute__((always_inline)) -> float { return s[e / 16][e % 16]; };
  float m8[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    m8[c] = score(c);
#pragma unroll
    for (int k = 1; k + 1 < kPerChain; k += 2) m8[c] = max3(m8[c], score(c + 8 * k), score(c + 8 * (k + 1)));
    // (max3 with a repeated operand, so no fmaxf has to canonicalise an asm result)
    if constexpr (kPerChain % 2 == 0) {
      const float x = score(c + 8 * (kPerChain - 1));
      m8[c] = max3(m8[c], x, x);
    }
  }
  const float mx = max3(max3(m8[0], m8[1], m8[2]), max3(m8[3], m8[4], m8[5]), max3(m8[6], m8[7], m8[7]));
  return pair_max(mx);
}

template <int KB, int EMU>
__device__ __forceinline__ void softmax_exp_rowsum(f32x16 (&s)[KB], float c, float m_ref, float (&l_part)[4]) {
  const float neg_m = (m_ref == kNegInf) ? 0.0f : -m_ref;   // no key yet: every P is 2^-inf = 0
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = __builtin_fmaf(s[kb][i], c, neg_m);
      const float e = ((kb & 1) * 16 + i < EMU) ? exp2_sw(x) : exp2_hw(x);
      s[kb][i] = e;
      l_part[i & 3] += e;
    }
}

}  // namespace fa

