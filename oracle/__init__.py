"""CPU oracle for fused exact attention -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct float64 description of what
the GPU library computes.  It exists to check the GPU path, never to serve it:
only the test-suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code,
constants or generators with the HIP kernels and imports nothing from the
product package.

Sources.  Three web pages on FlashAttention-4 (FA4):
  * "How FlashAttention 4 Works" -- GPU MODE lecture 80 notes (Korean);
  * "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for
    Asymmetric Hardware Scaling" -- English summary of the paper, which
    carries the paper's section / equation / table pointers;
  * the Korean summary of the same paper (arXiv 2603.05451) on gist.science.

Modules
  attention        exact softmax attention forward (O, LSE) and its analytic
                   gradients -- the textbook definition the FA4 kernel reaches
                   exactly ("recovers the exact result at the final
                   normalisation", paper §3.1.4).
  online_softmax   the FA4 forward algorithm step by step: tile loop, online
                   max, conditional rescaling with threshold tau (paper
                   §3.1.4, Eq. 6), final 1/l normalisation.
  exp2_emulation   Cody-Waite range-reduced polynomial 2^x (paper §3.1.3,
                   Table 2) with the oracle's own minimax fit, bf16 rounding
                   and ULP distance.
  partial          attention over one key range (output normalised over the
                   range + its log-sum-exp) and the merge of such parts over
                   disjoint ranges -- the single-GPU pieces of ring attention.
  fp8              e4m3 decoding, exact attention of dequantised e4m3 inputs,
                   and the per-element error bound of rounding P to e4m3.
  mxfp4            MXFP4 (E2M1 elements, E8M0 scales per 32) decoding and
                   exact attention of MXFP4 Q, K with e4m3 V, with the bounds
                   of ``fp8`` on the decoded tensors.
  roofline         per-tile cycle model (paper §3.1.1 Table 1; §3.2.1 Eq. 7-8)
                   with B200 constants and with CDNA4 constants.

Parity status: every function here is pinned by tests under tests/ that do
not re-type its formula (brute force, closed forms, invariants, finite
differences, an independent LP minimax, the pages' printed cycle counts).
The pages' own polynomial coefficients and the text of Eq. 6 are not on the
pages: those are "parity unpinned"; the oracle's own choices are pinned
instead.
"""
from .attention import attention_forward, attention_backward, attention_probs
from .online_softmax import conditional_rescale_forward
from .exp2_emulation import (fit_exp2_minimax, exp2_emulated_f32, bf16_round,
                             bf16_ulp_distance, relative_error_curve)
from .partial import attention_partial, merge_partials
from .fp8 import (e4m3_decode, dequantise, attention_fp8_reference, fp8_output_bound, fp8_score_error_bound,
                  fp8_float32_bound, summation_gamma)
from .mxfp4 import e2m1_decode, e8m0_decode, mx_decode, attention_mxfp4_reference, mxfp4_bounds
from .fp8_blocks import dequantise_blocks, v_ratios, attention_fp8_blockscaled_reference, fp8_blockscaled_bounds
from . import roofline

__all__ = [
    "attention_forward", "attention_backward", "attention_probs",
    "conditional_rescale_forward",
    "fit_exp2_minimax", "exp2_emulated_f32", "bf16_round", "bf16_ulp_distance",
    "relative_error_curve", "attention_partial", "merge_partials", "roofline",
    "e4m3_decode", "dequantise", "attention_fp8_reference", "fp8_output_bound", "fp8_score_error_bound",
    "fp8_float32_bound", "summation_gamma",
    "e2m1_decode", "e8m0_decode", "mx_decode", "attention_mxfp4_reference", "mxfp4_bounds",
    "dequantise_blocks", "v_ratios", "attention_fp8_blockscaled_reference", "fp8_blockscaled_bounds",
]
