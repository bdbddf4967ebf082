// C ABI of the attention library: argument validation, then one launch
// sequence on the caller's stream.  Declarations and contracts: include/fa.h.

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool sizes_ok(int B, int H, int Sq, int Sk) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return false;
  // index arithmetic uses size_t offsets per (b, h) slice and int row indices
  const long long rows = (long long)B * H * (Sq > Sk ? Sq : Sk);
  return rows < (1LL << 31);
}

bool d_supported(int d) { return d == FA_D_SMALL || d == FA_D_LARGE; }

// The kernels address one head of a tensor with 31-bit byte offsets and may
// read up to a few tiles past its last row (those reads return zeros).
bool head_addressable(int Sq, int Sk, int d) {
  const long long rows = (Sq > Sk ? Sq : Sk) + 1024LL;
  return rows * d * 2 < (1LL << 31);
}

}  // namespace

extern "C" {

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_SCRATCH: return "request exceeds the library's fixed scratch (B * H * Sq > FA_NOALLOC_MAX_ROWS)";
  }
  return "unknown status";
}

float fa_fwd_realised_emu_frac(int d, float emu_frac) {
  if (!d_supported(d) || !(emu_frac >= 0.0f && emu_frac <= 1.0f)) return -1.0f;
  return (float)fa::fwd_nearest_emu_count(d, emu_frac) / (float)fa::fwd_exps_per_lane_tile(d);
}

fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int Sq, int Sk,
                 int d, int causal, float scale, float tau, float emu_frac, void* stream) {
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_INVALID;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  if (!(isfinite(tau) && tau >= 0.0f && tau <= 64.0f)) return FA_ERR_INVALID;
  if (!(emu_frac >= 0.0f && emu_frac <= 1.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d)) return FA_ERR_UNSUPPORTED;

  fa::FwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.q_off = 0; a.k_begin = 0; a.k_end = Sk;
  a.causal = causal != 0;
  a.scale = scale;
  a.tau = tau;
  a.emu_count = fa::fwd_nearest_emu_count(d, emu_frac);
  const hipError_t e = fa::launch_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_rescale_count(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                int Sq, int Sk, int d, int causal, float scale, float tau, unsigned int* events,
                                void* stream) {
  if (!events || (reinterpret_cast<uintptr_t>(events) & 3u) != 0) return FA_ERR_INVALID;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_INVALID;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  if (!(isfinite(tau) && tau >= 0.0f && tau <= 64.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d)) return FA_ERR_UNSUPPORTED;

  fa::FwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.q_off = 0; a.k_begin = 0; a.k_end = Sk;
  a.causal = causal != 0;
  a.scale = scale;
  a.tau = tau;
  a.emu_count = 0;
  a.events = events;
  const hipError_t e = fa::launch_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_fp8(const void* Q8, const void* K8, const void* V8, float q_descale, float k_descale,
                     float v_descale, const float* head_descales, void* O, float* LSE, int B, int H, int Sq, int Sk,
                     int d, int causal, float scale, float tau, void* stream) {
  if (!Q8 || !K8 || !V8 || !O || !LSE) return FA_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(head_descales) % alignof(float) != 0) return FA_ERR_INVALID;
  if (!aligned16(Q8) || !aligned16(K8) || !aligned16(V8) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  for (float f : {q_descale, k_descale, v_descale})
    if (!(isfinite(f) && f > 0.0f)) return FA_ERR_INVALID;
  // the kernel folds the score factors into one float: it must stay a
  // finite normal number (each factor alone can pass while the product
  // overflows or underflows)
  const float score_factor = scale * q_descale * k_descale * 1.4426950408889634f;
  if (!(isfinite(score_factor) && score_factor >= FLT_MIN)) return FA_ERR_INVALID;
  if (!(isfinite(tau) && tau >= 0.0f && tau <= 8.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d)) return FA_ERR_UNSUPPORTED;

  fa::FwdFp8Args a;
  a.q = Q8; a.k = K8; a.v = V8; a.o = O; a.lse = LSE;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.q_descale = q_descale; a.k_descale = k_descale; a.v_descale = v_descale;
  a.head_descales = head_descales;
  a.tau = tau;
  const hipError_t e = fa::launch_fwd_fp8(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_fp8_blocks(const void* Q8, const void* K8, const void* V8, const float* q_factors,
                            const float* k_factors, const float* v_factors, void* O, float* LSE, int B, int H,
                            int Sq, int Sk, int d, int causal, float scale, float tau, void* stream) {
  if (!Q8 || !K8 || !V8 || !q_factors || !k_factors || !v_factors || !O || !LSE) return FA_ERR_INVALID;
  if (!aligned16(Q8) || !aligned16(K8) || !aligned16(V8) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_INVALID;
  for (const float* f : {q_factors, k_factors, v_factors})
    if (reinterpret_cast<uintptr_t>(f) % alignof(float) != 0) return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  if (!(isfinite(scale * 1.4426950408889634f) && scale * 1.4426950408889634f >= FLT_MIN)) return FA_ERR_INVALID;
  if (!(isfinite(tau) && tau >= 0.0f && tau <= 8.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d)) return FA_ERR_UNSUPPORTED;

  fa::FwdFp8Args a;
  a.q = Q8; a.k = K8; a.v = V8; a.o = O; a.lse = LSE;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.q_descale = a.k_descale = a.v_descale = 1.0f;
  a.head_descales = nullptr;
  a.q_blocks = q_factors; a.k_blocks = k_factors; a.v_blocks = v_factors;
  a.tau = tau;
  const hipError_t e = fa::launch_fwd_fp8(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_mxfp4(const void* Q4, const void* Q_scales, const void* K4, const void* K_scales, const void* V8,
                        float v_descale, void* O, float* LSE, int B, int H, int Sq, int Sk, int d, int causal,
                        float scale, float tau, void* stream) {
  if (!Q4 || !Q_scales || !K4 || !K_scales || !V8 || !O || !LSE) return FA_ERR_INVALID;
  if (!aligned16(Q4) || !aligned16(K4) || !aligned16(V8) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(Q_scales) & 3u) != 0 || (reinterpret_cast<uintptr_t>(K_scales) & 3u) != 0)
    return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  if (!(isfinite(v_descale) && v_descale > 0.0f)) return FA_ERR_INVALID;
  if (!(isfinite(scale * 1.4426950408889634f) && scale * 1.4426950408889634f >= FLT_MIN)) return FA_ERR_INVALID;
  if (!(isfinite(tau) && tau >= 0.0f && tau <= 8.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (d != FA_D_LARGE) return FA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d)) return FA_ERR_UNSUPPORTED;

  fa::FwdFp8Args a;
  a.q = Q4; a.k = K4; a.v = V8; a.o = O; a.lse = LSE;
  a.q_scales = Q_scales; a.k_scales = K_scales;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk;
  a.causal = causal != 0;
  a.scale = scale;
  a.q_descale = 1.0f; a.k_descale = 1.0f; a.v_descale = v_descale;
  a.head_descales = nullptr;
  a.tau = tau;
  const hipError_t e = fa::launch_fwd_mxfp4(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_partial(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part, int B, int H,
                         int Sq, int Sk, int d, int q_offset, int k_begin, int k_end, int causal, float scale,
                         float tau, float emu_frac, void* stream) {
  if (!Q || !K || !V || !O_part || !LSE_part) return FA_ERR_INVALID;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O_part) || !aligned16(LSE_part))
    return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (q_offset < 0 || k_begin < 0 || k_end <= k_begin || k_end > Sk) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  if (!(isfinite(tau) && tau >= 0.0f && tau <= 64.0f)) return FA_ERR_INVALID;
  if (!(emu_frac >= 0.0f && emu_frac <= 1.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d)) return FA_ERR_UNSUPPORTED;
  // the kernel forms causal bounds as q_offset + (row block end) + (one
  // tile) in 32-bit ints, up to q_offset + Sq + 414
  if ((long long)q_offset + Sq + 512 >= (1LL << 31)) return FA_ERR_UNSUPPORTED;

  fa::FwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = nullptr; a.o32 = O_part; a.lse = LSE_part;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.q_off = q_offset; a.k_begin = k_begin; a.k_end = k_end;
  a.causal = causal != 0;
  a.scale = scale;
  a.tau = tau;
  a.emu_count = fa::fwd_nearest_emu_count(d, emu_frac);
  const hipError_t e = fa::launch_fwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_merge(const float* O_parts, const float* LSE_parts, int n_parts, int B, int H, int Sq, int d, void* O,
                   float* LSE, void* stream) {
  if (!O_parts || !LSE_parts || !O || !LSE) return FA_ERR_INVALID;
  if (!aligned16(O_parts) || !aligned16(LSE_parts) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_INVALID;
  if (n_parts < 1 || !sizes_ok(B, H, Sq, Sq)) return FA_ERR_INVALID;
  if ((long long)n_parts * B * H * Sq >= (1LL << 31)) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  const hipError_t e = fa::launch_merge(O_parts, LSE_parts, n_parts, B * H * Sq, d, O, LSE,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int H, int Sq, int Sk, int d, int causal, int deterministic) {
  (void)causal;
  if (!sizes_ok(B, H, Sq, Sk) || !d_supported(d)) return 0;
  return fa::bwd_workspace_bytes(B, H, Sq, Sk, d, deterministic != 0);
}

fa_status fa_bwd_phase(int phases, const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                       const void* dO, void* dQ, void* dK, void* dV, int B, int H, int Sq, int Sk, int d, int causal,
                       float scale, int deterministic, void* workspace, size_t workspace_bytes, void* stream) {
  if (phases < 1 || phases > FA_BWD_ALL) return FA_ERR_INVALID;
  if (!Q || !K || !V || !O || !LSE || !dO || !dQ || !dK || !dV || !workspace) return FA_ERR_INVALID;
  const void* ptrs[] = {Q, K, V, O, LSE, dO, dQ, dK, dV, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (deterministic != 0 && deterministic != 1) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d)) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa::bwd_workspace_bytes(B, H, Sq, Sk, d, deterministic != 0)) return FA_ERR_INVALID;

  fa::BwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE; a.dout = dO;
  a.dq = dQ; a.dk = dK; a.dv = dV;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.deterministic = deterministic != 0;
  a.workspace = workspace;
  const hipError_t e = fa::launch_bwd(a, phases, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE, const void* dO,
                 void* dQ, void* dK, void* dV, int B, int H, int Sq, int Sk, int d, int causal, float scale,
                 int deterministic, void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_phase(FA_BWD_ALL, Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, Sq, Sk, d, causal, scale, deterministic,
                      workspace, workspace_bytes, stream);
}

namespace {
// dS^T of one (b, h) slice within a 2^31-byte buffer range (32-bit offsets)
bool ds_addressable(int Sq, int Sk) {
  const long long nqb = (Sq + 127) / 128, rows = (Sk + 127) / 128 * 128LL;
  return nqb * rows * 128 * 2 < (1LL << 31);
}
}  // namespace

size_t fa_bwd_ds_workspace_bytes(int B, int H, int Sq, int Sk, int d, int causal, int deterministic) {
  (void)causal;
  (void)deterministic;
  if (!sizes_ok(B, H, Sq, Sk) || !d_supported(d) || !ds_addressable(Sq, Sk)) return 0;
  return fa::bwd_ds_workspace_bytes(B, H, Sq, Sk);
}

fa_status fa_bwd_ds_phase(int phases, const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                          const void* dO, void* dQ, void* dK, void* dV, int B, int H, int Sq, int Sk, int d,
                          int causal, float scale, int deterministic, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (phases < 1 || phases > FA_BWD_ALL) return FA_ERR_INVALID;
  if (!Q || !K || !V || !O || !LSE || !dO || !dQ || !dK || !dV || !workspace) return FA_ERR_INVALID;
  const void* ptrs[] = {Q, K, V, O, LSE, dO, dQ, dK, dV, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (deterministic != 0 && deterministic != 1) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d) || !ds_addressable(Sq, Sk)) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa::bwd_ds_workspace_bytes(B, H, Sq, Sk)) return FA_ERR_INVALID;

  fa::BwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE; a.dout = dO;
  a.dq = dQ; a.dk = dK; a.dv = dV;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.deterministic = deterministic != 0;
  a.workspace = workspace;
  const hipError_t e = fa::launch_bwd_ds(a, phases, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd_ds(const void* Q, const void* K, const void* V, const void* O, const float* LSE, const void* dO,
                    void* dQ, void* dK, void* dV, int B, int H, int Sq, int Sk, int d, int causal, float scale,
                    int deterministic, void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_ds_phase(FA_BWD_ALL, Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, Sq, Sk, d, causal, scale,
                         deterministic, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                         const void* dO, void* dQ, void* dK, void* dV, int B, int H, int Sq, int Sk, int d,
                         int causal, float scale, int deterministic, void* stream) {
  if (!Q || !K || !V || !O || !LSE || !dO || !dQ || !dK || !dV) return FA_ERR_INVALID;
  const void* ptrs[] = {Q, K, V, O, LSE, dO, dQ, dK, dV};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID;
  if (!sizes_ok(B, H, Sq, Sk)) return FA_ERR_INVALID;
  if (!(isfinite(scale) && scale > 0.0f)) return FA_ERR_INVALID;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID;
  if (deterministic != 0 && deterministic != 1) return FA_ERR_INVALID;
  if (!d_supported(d)) return FA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return FA_ERR_UNSUPPORTED;
  if (!head_addressable(Sq, Sk, d)) return FA_ERR_UNSUPPORTED;
  if (fa::bwd_workspace_bytes(B, H, Sq, Sk, d, deterministic != 0) > fa::kScratchBytes) return FA_ERR_SCRATCH;

  void* ws = nullptr;
  if (fa::bwd_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  fa::BwdArgs a;
  a.q = Q; a.k = K; a.v = V; a.o = O; a.lse = LSE; a.dout = dO;
  a.dq = dQ; a.dk = dK; a.dv = dV;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.deterministic = deterministic != 0;
  a.workspace = ws;
  const hipError_t e = fa::launch_bwd(a, fa::kBwdPrepare | fa::kBwdDq | fa::kBwdDkdv, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_exp2_probe(const float* x, float* y_hw, float* y_emu, long long n, void* stream) {
  if (n < 0) return FA_ERR_INVALID;
  if (n > 0 && (!x || !y_hw || !y_emu)) return FA_ERR_INVALID;
  const hipError_t e = fa::launch_exp2_probe(x, y_hw, y_emu, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
