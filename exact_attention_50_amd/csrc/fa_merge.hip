// Merge of partial attention results over disjoint key ranges (the combine
// step of split-KV and ring / context-parallel attention).
//
// Each part s holds, per query row, the attention output normalised over its
// own keys, O_s, and the log-sum-exp of its scores, LSE_s (natural log).
// Over the union of the ranges the softmax weights of part s are
// exp(LSE_s - LSE) with LSE = log sum_s exp(LSE_s), so
//     O = sum_s exp(LSE_s - LSE) O_s.
// This is the same rescale-and-add the forward's online softmax performs
// between key tiles (FlashAttention-4 page, Method: the running output is
// kept unnormalised relative to a reference max and rescaled when it moves),
// applied once to whole ranges.  A part whose rows saw no key carries
// LSE_s = -inf and weight 0; a row no part saw gets O = 0, LSE = -inf.
//
// HBM-bound: per row, n x (4 d + 4) bytes read and 2 d + 4 written.  One
// lane per four output dims (d / 4 lanes per row, 16-byte float32 loads,
// consecutive rows in consecutive lanes), so a wave reads whole 512- or
// 256-byte row segments of each part.

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_parts,
                                                    const float* __restrict__ lse_parts, int n_parts, int rows,
                                                    bf16* __restrict__ o, float* __restrict__ lse) {
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int c = (threadIdx.x % kLanesPerRow) * 4;
  if (row >= rows) return;
  float m = kNegInf;
  for (int s = 0; s < n_parts; ++s) m = __builtin_fmaxf(m, lse_parts[(size_t)s * rows + row]);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;
  if (m != kNegInf) {
    for (int s = 0; s < n_parts; ++s) {
      const float ls = lse_parts[(size_t)s * rows + row];
      const float w = exp2_hw((ls - m) * kLog2e);   // exp2(-inf) = 0 for an empty part
      const f32x4 x = *reinterpret_cast<const f32x4*>(o_parts + ((size_t)s * rows + row) * D + c);
      acc += w * x;
      wsum += w;
    }
  }
  const bool empty = !(wsum > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / wsum;
  *reinterpret_cast<bf16x4*>(o + (size_t)row * D + c) = __builtin_convertvector(acc * inv, bf16x4);
  if (c == 0) lse[row] = empty ? kNegInf : m + __builtin_log2f(wsum) * kLn2;
}

template <int D>
hipError_t launch_merge_d(const float* o_parts, const float* lse_parts, int n_parts, int rows, void* o, float* lse,
                          hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / (D / 4);
  const unsigned blocks = (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(merge_kernel<D>, dim3(blocks), dim3(256), 0, stream, o_parts, lse_parts, n_parts, rows,
                     static_cast<bf16*>(o), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int n_parts, int rows, int d, void* o,
                        float* lse, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  return d == 64 ? launch_merge_d<64>(o_parts, lse_parts, n_parts, rows, o, lse, stream)
                 : launch_merge_d<128>(o_parts, lse_parts, n_parts, rows, o, lse, stream);
}

}  // namespace fa
