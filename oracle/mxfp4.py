"""Attention with MXFP4 queries and keys, in float64 -- test infrastructure only.

What it computes.  "How FlashAttention 4 Works" lists FP4 among the formats
Blackwell adds, places it as experimental (it needs calibration) in its map
of which attention operands tolerate which precision, and leaves FP4
channels open among its questions.  The experiment built here keeps V and P
in e4m3 (as the FP8 forward does) and takes Q and K in MXFP4, the OCP
microscaling format of 4-bit elements:

  * an element is E2M1: sign bit 3, exponent bits 2-1 with bias 1, mantissa
    bit 0; exponent 0 is subnormal (0 or 0.5), so the magnitudes of codes
    0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (no infinity or NaN);
  * every 32 consecutive elements of a row (along the head dimension) share
    one E8M0 scale: the byte s stands for 2^(s - 127), 255 for NaN;
  * two elements per byte, the even-indexed one in the low nibble.

The attention the inputs stand for is the exact attention of the decoded
tensors:

  Q = decode(Q4, Q scales),  K = decode(K4, K scales),  V = v_descale * e4m3(V8),
  O, LSE = attention_forward(Q, K, V)   (the definition in ``attention``).

The kernel rounds the unnormalised probabilities to e4m3 before P V as the
FP8 forward does, so the per-element bounds of ``fp8`` (the rounding of P,
and the float32 arithmetic) apply to the decoded tensors unchanged; the
products of E2M1 values with power-of-two scales are exact in float32.

Pins (tests/test_oracle_mxfp4.py): the element decoder against the format's
named values and structure (sign symmetry, monotone magnitudes, every value
exact in e4m3); the scale decoder against torch's float8_e8m0fnu on all 256
codes; block decoding against a scalar loop; the reference against
attention_forward of the decoded tensors; the bounds hold for a brute-force
pipeline that rounds P with torch's e4m3 conversion.
"""
import numpy as np

from .attention import attention_forward
from .fp8 import e4m3_decode, float32_bound_of, output_bound_of, score_error_bound_of

E2M1_BLOCK = 32


def _np(x):
    return np.asarray(x.cpu().numpy() if hasattr(x, "cpu") else x)


def e2m1_decode(codes):
    """float64 values of E2M1 codes 0..15 (array or tensor of integers)."""
    c = _np(codes).astype(np.int64) & 0xF
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * mag


def e8m0_decode(scales):
    """float64 values 2^(s - 127) of E8M0 bytes (255: NaN)."""
    s = _np(scales).astype(np.int64) & 0xFF
    return np.where(s == 255, np.nan, np.exp2(s - 127.0))


def mx_decode(packed, scales, block=E2M1_BLOCK):
    """Decode MXFP4 rows: packed uint8 [..., d/2] (element 2j in the low
    nibble of byte j, 2j + 1 in the high nibble) and E8M0 scales
    [..., d/block] -> float64 [..., d]."""
    p = _np(packed).astype(np.int64)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    elems = np.stack([e2m1_decode(lo), e2m1_decode(hi)], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
    sc = e8m0_decode(scales)
    return elems * np.repeat(sc, block, axis=-1)


def attention_mxfp4_reference(q4, q_scales, k4, k_scales, v8, v_descale, scale, causal=False):
    """(O, LSE) of exact attention on the decoded MXFP4 Q, K and e4m3 V."""
    q, k = mx_decode(q4, q_scales), mx_decode(k4, k_scales)
    v = e4m3_decode(v8) * float(v_descale)
    return attention_forward(q, k, v, scale, causal)


def mxfp4_bounds(q4, q_scales, k4, k_scales, v8, v_descale, scale, causal=False):
    """Per-element bound [B,H,Sq,d] on |O_kernel - O_exact| (the rounding of
    P to e4m3 plus the float32 arithmetic, on the decoded tensors) and the
    per-row float32 score-error bound [B,H,Sq] (natural log units)."""
    q, k = mx_decode(q4, q_scales), mx_decode(k4, k_scales)
    v = e4m3_decode(v8) * float(v_descale)
    return (output_bound_of(q, k, v, scale, causal) + float32_bound_of(q, k, v, scale, causal),
            score_error_bound_of(q, k, scale, causal))
