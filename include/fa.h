/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact-attention library.
 *
 * What it computes.  Exact softmax attention, O = softmax(scale * Q K^T
 * [+ causal mask]) V, and the per-row log-sum-exp, tile by tile with an
 * online softmax so that neither the score matrix S nor the probabilities P
 * ever reach device memory; and the gradients dQ, dK, dV of that function.
 * The forward follows the FlashAttention-4 paper as summarised on the page
 * "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for Asymmetric
 * Hardware Scaling" (Key claims and Method): conditional rescaling of the
 * running output with threshold tau (paper §3.1.4, Eq. 6) and a software
 * 2^x (Cody-Waite range reduction + polynomial, paper §3.1.3, Table 2) for a
 * share of the exponentials.  The backward recomputes P from the LSE and
 * forms the gradients from the products of paper §3.2.1 (Eq. 7-8); every
 * output is written once in a fixed order, so it is deterministic (the
 * paper's deterministic mode, §1).
 *
 * Conventions shared by every entry point.
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc / torch CUDA
 *     memory) on the current device.  bf16 tensors are passed as void* to
 *     16-bit IEEE bfloat16 patterns.
 *   - Layout: Q, O, dO, dQ are [B, H, Sq, d]; K, V, dK, dV are [B, H, Sk, d];
 *     LSE is [B, H, Sq] float32 (natural log); all dense row-major
 *     (contiguous, d fastest).  Pointers must be 16-byte aligned.
 *   - Causal: key j is visible to query i iff j <= i (top-left aligned);
 *     causal requires Sq == Sk.
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     state between calls and is thread-safe.  Work is enqueued on `stream`
 *     (0 = the null stream) and calls return without synchronising;
 *     asynchronous faults surface at the caller's next synchronisation.
 *   - Errors: arguments are validated before any HIP call; on error nothing
 *     is enqueued and no output is touched.  No C++ exception crosses the
 *     ABI.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = 1,      /* null pointer, bad size, bad scalar, misaligned pointer, small workspace */
  FA_ERR_UNSUPPORTED = 2,  /* valid request outside what the kernels implement (d, causal Sq != Sk,
                              a head longer than the limit below) */
  FA_ERR_HIP = 3,          /* the HIP runtime reported an error while launching */
  FA_ERR_SCRATCH = 4       /* a no-allocation entry point was asked for more than its fixed scratch holds */
} fa_status;

/* Head dimensions the kernels are built for.  One head of any tensor must
 * be addressable with 31-bit byte offsets: (max(Sq, Sk) + 1024) * d * 2 <
 * 2^31, i.e. up to about 8.4 M rows at d = 128; longer heads return
 * FA_ERR_UNSUPPORTED. */
#define FA_D_SMALL 64
#define FA_D_LARGE 128

/* Forward.  Q, K, V bf16 in; O bf16 out; LSE float32 out.
 *   scale     > 0 and finite; multiplies Q K^T (usually 1/sqrt(d)).
 *   tau       threshold of the conditional rescale in log2 units, 0 <= tau
 *             <= 64 (8 = log2 256 is the paper's default, §3.1.4).  The
 *             correction of the running output is skipped while a row's max
 *             (in log2 units) rises by at most tau over the max currently
 *             applied; tau = 0 is the eager online softmax.  Exact after the
 *             final normalisation for every tau.
 *   emu_frac  share of the exponentials computed by the software 2^x
 *             instead of the hardware one, 0 <= emu_frac <= 1 (the paper's
 *             10-25 %, §3.1.3).  Realised as a fixed count of each lane's
 *             per-tile exponentials, the supported count nearest emu_frac;
 *             fa_fwd_realised_emu_frac() reports the share actually used.
 *   B, H, Sq, Sk >= 1; d in {64, 128}.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED or FA_ERR_HIP. */
fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int B, int H, int Sq, int Sk, int d, int causal, float scale,
                 float tau, float emu_frac, void* stream);

/* The forward of fa_fwd (hardware exponentials only), instrumented to make
 * the conditional rescale observable (the FlashAttention-4 summary, Key
 * claims §3.1.4, Eq. 6: the correction is gated per warp; here per
 * wavefront of 32 query rows).  Writes O and LSE exactly as fa_fwd with
 * emu_frac = 0 does, and adds to events[(b * H + h) * ceil(Sq / 32) + i],
 * for the wavefront of rows 32 i .. 32 i + 31 of head (b, h), the number of
 * its key tiles after its first one in which the correction branch ran (some
 * row of the wavefront saw its max rise by more than tau over the reference
 * max); in the few-blocks causal form two wavefronts share those rows and
 * both add to the slot.  Tiles are those of the launch form
 * fa_fwd picks for the same shape: 128 keys per tile visited in order when
 * ceil(Sq / 256) * B * H >= 512 or non-causal; otherwise (few causal
 * blocks) each wavefront visits every other 64-key tile and its first tile
 * is the first it visits.
 *   events   device uint32 [B, H, ceil(Sq / 32)], 4-byte aligned,
 *            caller-owned; the call adds to it (zero it first), with atomics,
 *            so counts are exact.
 *   Other arguments and errors as for fa_fwd.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED or FA_ERR_HIP. */
fa_status fa_fwd_rescale_count(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                int Sq, int Sk, int d, int causal, float scale, float tau, unsigned int* events,
                                void* stream);

/* Forward with e4m3 (FP8, OCP e4m3fn) operands, the next operand format of the
 * FlashAttention-4 summary's precision discussion.  Q8, K8, V8 are e4m3
 * bytes, [B,H,Sq,d], [B,H,Sk,d], [B,H,Sk,d]; the attention is computed on
 * Q = q_descale * Q8, K = k_descale * K8, V = v_descale * V8 (descales > 0,
 * finite), each descale optionally times a factor of its (batch, head)
 * slice: head_descales is null (per-tensor factors only) or a float32
 * device array [3][B][H] holding the slices' Q, K and V factors, read by the
 * kernel (caller-owned; finite and > 0, which the library cannot check before
 * the launch: other values give non-finite outputs).  Scores accumulate in float32; the unnormalised probabilities
 * P = 2^(s - m_ref) <= 2^tau are rounded to e4m3 (nearest even) before P V;
 * the row sum and LSE use the float32 P.  O is bf16 [B,H,Sq,d], LSE float32
 * [B,H,Sq] (natural log, exact up to float32 rounding of the scores).
 *   0 <= tau <= 8 (P must stay below e4m3's largest value, 448);
 *   d = 64 or 128 (else FA_ERR_UNSUPPORTED); causal requires Sq = Sk; other
 *   arguments and errors as for fa_fwd.  16-byte aligned device pointers.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED or FA_ERR_HIP. */
fa_status fa_fwd_fp8(const void* Q8, const void* K8, const void* V8, float q_descale, float k_descale,
                     float v_descale, const float* head_descales, void* O, float* LSE, int B, int H, int Sq,
                     int Sk, int d, int causal, float scale, float tau, void* stream);

/* Forward with e4m3 (OCP e4m3fn) operands and one dequantisation factor per
 * block of FA_FP8_SCALE_BLOCK = 128 consecutive rows of each (batch, head)
 * slice: the finer of the two scale forms the FlashAttention-4 summary's
 * precision discussion leaves open for FP8 operands.  Q8, K8, V8 are e4m3
 * bytes as for fa_fwd_fp8; q_factors is a float32 device array
 * [B][H][ceil(Sq / 128)], k_factors and v_factors [B][H][ceil(Sk / 128)]
 * (caller-owned, read by the kernel: finite and > 0, which the library
 * cannot check before the launch; other values give non-finite outputs).
 * The attention is computed on Q[b,h,i] = q_factors[b,h,i / 128] * Q8[b,h,i]
 * (K, V likewise).  Scores accumulate in float32 and take the Q and K block
 * factors as one score factor per 32-row wavefront and 128-key tile; the
 * unnormalised probabilities are rounded to e4m3 as r P, r = the key block's
 * V factor / the head's largest V factor (<= 1), before P V, and O is
 * multiplied by that largest factor; the row sum and LSE use the float32 P.
 * O is bf16 [B,H,Sq,d], LSE float32 [B,H,Sq].
 *   0 <= tau <= 8; d = 64 or 128 (else FA_ERR_UNSUPPORTED); causal requires
 *   Sq = Sk; 16-byte aligned Q8, K8, V8, O, LSE; 4-byte aligned factors;
 *   other arguments and errors as for fa_fwd.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED or FA_ERR_HIP. */
#define FA_FP8_SCALE_BLOCK 128
fa_status fa_fwd_fp8_blocks(const void* Q8, const void* K8, const void* V8, const float* q_factors,
                            const float* k_factors, const float* v_factors, void* O, float* LSE, int B, int H,
                            int Sq, int Sk, int d, int causal, float scale, float tau, void* stream);

/* Forward with MXFP4 queries and keys and e4m3 values: the FP4 operand
 * experiment of the lecture notes "How FlashAttention 4 Works" (FP4 among
 * Blackwell's new formats, experimental in their map of which attention
 * operands tolerate which precision, FP4 channels among the open questions).
 * Q4 and K4 hold MXFP4 rows: d/2 bytes per row, two E2M1 elements per byte
 * (the even-indexed element in the low nibble; E2M1 = sign, 2-bit exponent
 * with bias 1, 1-bit mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), layout
 * [B,H,Sq,d/2] and [B,H,Sk,d/2]; Q_scales and K_scales hold one E8M0 byte
 * (2^(s - 127)) per 32 consecutive elements of a row, [B,H,Sq,d/32] and
 * [B,H,Sk,d/32] (4-byte aligned); V8 is e4m3 [B,H,Sk,d] with one descale.
 * The attention is computed on the decoded tensors: S = scale * Q K^T from
 * scaled fp4 x fp4 products with float32 accumulation, P = 2^(s - m_ref)
 * rounded to e4m3 before P V (as in fa_fwd_fp8), row sum and LSE from the
 * float32 P.  O bf16 [B,H,Sq,d], LSE float32 [B,H,Sq].
 *   d = 128 only (else FA_ERR_UNSUPPORTED); 0 <= tau <= 8; v_descale finite
 *   and > 0; causal requires Sq = Sk; other arguments and errors as for
 *   fa_fwd.  Scale bytes of 255 (NaN) give non-finite outputs.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED or FA_ERR_HIP. */
fa_status fa_fwd_mxfp4(const void* Q4, const void* Q_scales, const void* K4, const void* K_scales, const void* V8,
                       float v_descale, void* O, float* LSE, int B, int H, int Sq, int Sk, int d, int causal,
                       float scale, float tau, void* stream);

/* Forward over a range of keys, for split-KV and ring (context-parallel)
 * attention: queries i = 0 .. Sq-1 of Q (global index q_offset + i) attend to
 * the keys j = k_begin .. k_end-1 of K, V only (causal: key j is visible iff
 * j <= q_offset + i).  Writes, per row, the output normalised over those keys
 * alone, O_part = softmax(scale q K_r^T) V_r (float32 [B,H,Sq,d]), and the
 * log-sum-exp of its scores, LSE_part (float32 [B,H,Sq], natural log).  A row
 * that sees no key of the range gets O_part = 0 and LSE_part = -inf.  The
 * method is fa_fwd's (online softmax with conditional rescale, software 2^x
 * share); fa_merge combines parts over disjoint ranges into the result over
 * their union.  This is the single-GPU piece of the fused ring attention
 * that the lecture notes "How FlashAttention 4 Works" list among the open
 * directions for multi-GPU FA4 (their closing list of what comes next).
 *   Q is [B,H,Sq,d], K and V are [B,H,Sk,d] (all heads' full key arrays; the
 *   range selects rows inside each head).
 *   0 <= k_begin < k_end <= Sk; q_offset >= 0; causal 0 or 1 (Sq != Sk is
 *   allowed); other arguments as for fa_fwd.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED or FA_ERR_HIP. */
fa_status fa_fwd_partial(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part,
                         int B, int H, int Sq, int Sk, int d, int q_offset, int k_begin, int k_end,
                         int causal, float scale, float tau, float emu_frac, void* stream);

/* Merge of n_parts partial results (as written by fa_fwd_partial over
 * disjoint key ranges of the same queries) into the attention over the union
 * of the ranges: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s,
 * rounded to bf16; rows that no part saw get O = 0, LSE = -inf.
 *   O_parts: n_parts consecutive float32 [B,H,Sq,d] arrays; LSE_parts:
 *   n_parts consecutive float32 [B,H,Sq] arrays (device memory, caller-owned,
 *   read only).  O: bf16 [B,H,Sq,d] out; LSE: float32 [B,H,Sq] out.
 *   n_parts >= 1; d in {64, 128}.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED or FA_ERR_HIP. */
fa_status fa_merge(const float* O_parts, const float* LSE_parts, int n_parts, int B, int H, int Sq, int d,
                   void* O, float* LSE, void* stream);

/* The share of exponentials fa_fwd computes in software for a requested
 * emu_frac (a pure function of its arguments; no HIP call). Negative when
 * the arguments are invalid. */
float fa_fwd_realised_emu_frac(int d, float emu_frac);

/* Bytes of device workspace fa_bwd needs: two float32 [B,H,Sq] arrays of
 * row terms, D_i = sum_c dO_ic O_ic and LSE_i log2(e), each rounded up to
 * 256 bytes.  0 on invalid sizes. */
size_t fa_bwd_workspace_bytes(int B, int H, int Sq, int Sk, int d, int causal, int deterministic);

/* Backward.  Q, K, V, O, dO bf16 and LSE float32 in (O and LSE as written
 * by fa_fwd on the same inputs); dQ, dK, dV bf16 out.  P is recomputed from
 * LSE as exp(scale q.k - LSE); fp32 accumulation; outputs rounded to bf16
 * (nearest-even) once.  dQ is produced by workgroups that own query rows and
 * dK, dV by workgroups that own key rows, so every output element is written
 * by exactly one workgroup in a fixed summation order (no atomics).
 *   deterministic  0 or 1.  Results are bit-identical run to run in both
 *                  modes; the paper's deterministic mode (ordered dQ
 *                  accumulation, §1) is therefore met at no cost, and the
 *                  flag selects the same kernels.
 *   workspace      device memory of at least fa_bwd_workspace_bytes(...);
 *                  its contents on entry do not matter; it must not be used
 *                  concurrently by another call.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED or FA_ERR_HIP. */
fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                 const void* dO, void* dQ, void* dK, void* dV,
                 int B, int H, int Sq, int Sk, int d, int causal, float scale, int deterministic,
                 void* workspace, size_t workspace_bytes, void* stream);

/* The three parts of fa_bwd, enqueued separately (a bit mask, executed in
 * this order within one call):
 *   FA_BWD_PREPARE  D_i = sum_c dO_ic O_ic and LSE_i log2(e) into the
 *                   workspace;
 *   FA_BWD_DQ       dQ (reads the row terms; writes dQ only);
 *   FA_BWD_DKDV     dK and dV (reads the row terms; writes dK, dV only).
 * PREPARE and DQ in the same call run as one launch: the dQ kernel forms the
 * row terms of its rows itself (bit-identical to PREPARE's) and stores them
 * in the workspace before DKDV reads them.  After a PREPARE call has
 * completed, DQ and DKDV are independent and may run on different streams
 * (the caller orders them with events).  Arguments and validation are those
 * of fa_bwd; fa_bwd is fa_bwd_phase(FA_BWD_ALL, ...). */
#define FA_BWD_PREPARE 1
#define FA_BWD_DQ 2
#define FA_BWD_DKDV 4
#define FA_BWD_ALL 7
fa_status fa_bwd_phase(int phases, const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                       const void* dO, void* dQ, void* dK, void* dV,
                       int B, int H, int Sq, int Sk, int d, int causal, float scale, int deterministic,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace fa_bwd_ds needs: the row terms of
 * fa_bwd_workspace_bytes, then the dS buffer: per (b, h), ceil(Sq/128)
 * slabs of (Sk rounded up to 128) x 128 bf16 (Sq x Sk x 2 bytes, rounded
 * up; 512 MiB for B 1, H 16, Sq = Sk = 4096).  0 on invalid sizes or when
 * one (b, h) slice of the buffer would reach 2^31 bytes (Sq = Sk up to
 * 32640). */
size_t fa_bwd_ds_workspace_bytes(int B, int H, int Sq, int Sk, int d, int causal, int deterministic);

/* Backward in the paper's five products per tile pair (S, dP, dV, dK, dQ;
 * FA4 paper §3.2.1, Eq. 7-8, as summarised on "FlashAttention-4: Algorithm
 * and Kernel Pipelining Co-Design for Asymmetric Hardware Scaling"), without
 * its dQ atomics: the kernel that owns a block of keys forms S, dP, P, dS,
 * dV and dK and also writes dS (rounded to bf16, the operand its dK product
 * uses) to the workspace; a second kernel forms dQ = scale dS K per block of
 * 128 query rows.  Inputs, outputs, rounding and arguments as for fa_bwd;
 * results agree with fa_bwd's to rounding (not bitwise: the summation
 * orders differ) and are bit-identical run to run in both modes.
 *   workspace  device memory of at least fa_bwd_ds_workspace_bytes(...);
 *              contents on entry do not matter; not to be used concurrently
 *              by another call.
 * Returns FA_OK, FA_ERR_INVALID (also for a workspace that is too small),
 * FA_ERR_UNSUPPORTED (also when fa_bwd_ds_workspace_bytes would be 0 for
 * valid sizes) or FA_ERR_HIP. */
fa_status fa_bwd_ds(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                    const void* dO, void* dQ, void* dK, void* dV,
                    int B, int H, int Sq, int Sk, int d, int causal, float scale, int deterministic,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The three launches of fa_bwd_ds, enqueued separately (the FA_BWD_* bit
 * mask of fa_bwd_phase, executed in this order within one call):
 *   FA_BWD_PREPARE  D_i and LSE_i log2(e) into the workspace;
 *   FA_BWD_DKDV     dK and dV, and dS into the workspace (reads the row
 *                   terms);
 *   FA_BWD_DQ       dQ from the workspace's dS and K (writes dQ only).
 * Each phase reads what the earlier ones wrote into the same workspace, so
 * separate calls must run in this order (one stream, or events).  Arguments
 * and validation as for fa_bwd_ds; fa_bwd_ds is
 * fa_bwd_ds_phase(FA_BWD_ALL, ...). */
fa_status fa_bwd_ds_phase(int phases, const void* Q, const void* K, const void* V, const void* O,
                          const float* LSE, const void* dO, void* dQ, void* dK, void* dV,
                          int B, int H, int Sq, int Sk, int d, int causal, float scale, int deterministic,
                          void* workspace, size_t workspace_bytes, void* stream);

/* fa_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results as fa_bwd (bit for bit), with the workspace taken
 * from a fixed scratch array inside the library instead of a caller buffer.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); on its first call on a device it looks up that device's copy of
 * the array (16 MiB per GPU, held until the process ends).
 *   Limit: B * H * Sq <= FA_NOALLOC_MAX_ROWS (2^21); larger requests return
 *   FA_ERR_SCRATCH before anything is enqueued.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap on
 *   one GPU (different streams, or host threads without ordering) race and
 *   give wrong gradients.  Calls on one stream are ordered and safe.  The
 *   scratch keeps the last call's contents; nothing in it needs clearing
 *   (every row term is written before it is read).
 *   Other arguments, validation and errors as for fa_bwd.
 * Returns FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_SCRATCH or
 * FA_ERR_HIP. */
#define FA_NOALLOC_MAX_ROWS (1 << 21)
fa_status fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                         const void* dO, void* dQ, void* dK, void* dV,
                         int B, int H, int Sq, int Sk, int d, int causal, float scale, int deterministic,
                         void* stream);

/* Element-wise probe of the two exponentials the forward uses, so their
 * agreement can be measured (paper §3.1.3, Table 2): y_hw[i] = hardware
 * 2^x[i] (v_exp_f32), y_emu[i] = the software 2^x[i] of the forward kernel.
 * x, y_hw, y_emu are device float32 arrays of n >= 0 elements. */
fa_status fa_exp2_probe(const float* x, float* y_hw, float* y_emu, long long n, void* stream);

/* Static description of a status code; never NULL. */
const char* fa_status_str(fa_status s);

#ifdef __cplusplus
}
#endif
#endif /* FA_H_ */
