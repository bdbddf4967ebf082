// Host-side interface between the C ABI (fa_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;               // bf16 output, used when o32 is null
  float* o32 = nullptr;  // float32 output
  float* lse;
  int B, H, Sq, Sk, d;
  int q_off = 0;         // global index of query row 0
  int k_begin = 0;       // keys k_begin .. k_end - 1 are attended to
  int k_end = 0;
  bool causal;
  float scale;
  float tau;
  int emu_count;  // exponentials per lane per tile computed in software
  unsigned* events = nullptr;   // non-null: the instrumented instantiation, which
                                // adds its correction counts per (b, h) here
};

// Exponentials of one lane per 64 keys (64 keys x 32 queries / 64 lanes): the
// unit over which the software share is placed.
int fwd_exps_per_lane_tile(int d);
// Software-exponential counts the forward kernel is instantiated for.
int fwd_nearest_emu_count(int d, float emu_frac);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// e4m3 forward (d = 128): Q, K, V are e4m3 bytes dequantised by one factor
// each; O bf16, LSE float32
struct FwdFp8Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Sq, Sk;
  int d = 128;   // 128, or 64 for the e4m3 forwards
  bool causal;
  float scale, q_descale, k_descale, v_descale, tau;
  const float* head_descales;   // null or [3][B*H] on the device
  const void* q_scales = nullptr;   // MXFP4: E8M0 scales [B*H][Sq][4], [B*H][Sk][4]
  const void* k_scales = nullptr;
  // per-block factors (one per kFp8ScaleBlock rows of a (batch, head) slice):
  // float32 [B*H][ceil(Sq / 128)], [B*H][ceil(Sk / 128)] twice; null for the
  // per-tensor form (then q_descale, k_descale, v_descale, head_descales apply)
  const float* q_blocks = nullptr;
  const float* k_blocks = nullptr;
  const float* v_blocks = nullptr;
};
constexpr int kFp8ScaleBlock = 128;
hipError_t launch_fwd_fp8(const FwdFp8Args& a, hipStream_t stream);
// MXFP4 Q, K (E2M1 elements, d/2 bytes per row; E8M0 scales per 32 dims),
// e4m3 V: q_descale and k_descale unused, head_descales null
hipError_t launch_fwd_mxfp4(const FwdFp8Args& a, hipStream_t stream);

// rows = B * H * Sq; parts are n_parts consecutive [rows, d] / [rows] arrays
hipError_t launch_merge(const float* o_parts, const float* lse_parts, int n_parts, int rows, int d, void* o,
                        float* lse, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  int B, H, Sq, Sk, d;
  bool causal;
  float scale;
  bool deterministic;
  void* workspace;
};

size_t bwd_workspace_bytes(int B, int H, int Sq, int Sk, int d, bool deterministic);
// Fixed device scratch for the allocation-free backward: 16 MiB holds the
// workspace of B * H * Sq <= 2^21 query rows (two 8 MiB sections).
constexpr size_t kScratchBytes = size_t(16) << 20;
// This device's scratch address (resolved once per device; no allocation).
hipError_t bwd_scratch(void** out);
// phases: bit mask of the kernels to enqueue, in this order
constexpr int kBwdPrepare = 1, kBwdDq = 2, kBwdDkdv = 4;
hipError_t launch_bwd(const BwdArgs& a, int phases, hipStream_t stream);
// Five-product backward: prep, dK/dV (also writing dS^T), dQ from dS, in
// that order (phases: the kBwd* bits).  Its workspace: the row terms, then
// ceil(Sq/128) slabs of [Sk rounded up to 128, 128] bf16 per (b, h).
size_t bwd_ds_workspace_bytes(int B, int H, int Sq, int Sk);
hipError_t launch_bwd_ds(const BwdArgs& a, int phases, hipStream_t stream);

hipError_t launch_exp2_probe(const float* x, float* y_hw, float* y_emu, long long n, hipStream_t stream);

}  // namespace fa
