"""Attention on e4m3 inputs with per-block dequantisation factors, in float64
-- test infrastructure only.

What it computes.  The FA4 paper summary ("FlashAttention-4: Algorithm and
Kernel Pipelining Co-Design for Asymmetric Hardware Scaling", precision
discussion) and the lecture notes "How FlashAttention 4 Works" (their map of
which attention operands tolerate FP8) name FP8 operands without a scaling
recipe.  Beside one factor per tensor or per (batch, head), the finer form
read here gives every 128 consecutive rows of a (batch, head) slice of Q, K
and V a float factor of its own:

  Q[b,h,i] = q_f[b,h,i // 128] * e4m3(Q8[b,h,i])   (K, V likewise over keys),
  O, LSE = attention_forward(Q, K, V)   (the definition in ``attention``).

Rounding P.  A kernel whose P V product works on the e4m3 codes of V needs
one V factor per product; the one read here rounds r_j P_j to e4m3, with
r_j = v_f(block of key j) / (the head's largest V factor) <= 1, and
multiplies O by that largest factor at the end, normalising by the sum of
the unrounded P_j.  Per output element the rounding then moves O by at most

  sum_j (2^-4 r_j P_j + 2^-10 [r_j P_j < 2^-6]) |v_j| / (r_j l)
      <= 2^-4 sum_j p_j |v_j| + 2^-10 sum_j |v_j| / (r_j l_max)

(half an e4m3 step, as for one factor per tensor; v = the dequantised V, p the
exact weights, l_max = sum_j exp(s_j - max s) <= l).  With all factors equal,
r_j = 1 and the bound is that of ``fp8_output_bound``.  The float32 arithmetic
adds ``float32_bound_of`` on the dequantised tensors, with the exponent shift
log2 r_j (r_j and its log2 each rounded once) and two more roundings per
row-sum term (the tile's partial sum is multiplied by 2^-log2 r) counted in.

Pins (tests/test_oracle_fp8_blocks.py): block dequantisation against a scalar
loop (ragged last block included) and, with equal factors, against the
per-tensor form; the ratios r against their definition; the bound holds for a
brute-force pipeline that rounds r_j P_j with torch's e4m3 conversion and is
not vacuous; with equal factors the bound equals the per-tensor one.
"""
import numpy as np

from .attention import attention_forward, attention_probs
from .fp8 import e4m3_decode, float32_bound_of, score_error_bound_of

FP8_BLOCK = 128


def _np(x):
    return np.asarray(x.cpu().numpy() if hasattr(x, "cpu") else x, dtype=np.float64)


def dequantise_blocks(codes, factors, block=FP8_BLOCK):
    """e4m3 codes [B,H,S,d] times the factor of each row's block
    (factors [B,H,ceil(S / block)])."""
    v = e4m3_decode(codes)
    f = _np(factors)
    S = v.shape[2]
    per_row = np.repeat(f, block, axis=2)[:, :, :S]
    return v * per_row[..., None]


def v_ratios(v_factors, Sk, block=FP8_BLOCK):
    """r_j = v_f(block of key j) / max over the head's V factors, [B,H,Sk]."""
    f = _np(v_factors)
    r = f / f.max(axis=2, keepdims=True)
    return np.repeat(r, block, axis=2)[:, :, :Sk]


def attention_fp8_blockscaled_reference(q8, k8, v8, q_f, k_f, v_f, scale, causal=False, block=FP8_BLOCK):
    """(O, LSE) of exact attention on the block-dequantised e4m3 inputs."""
    return attention_forward(dequantise_blocks(q8, q_f, block), dequantise_blocks(k8, k_f, block),
                             dequantise_blocks(v8, v_f, block), scale, causal)


def fp8_blockscaled_bounds(q8, k8, v8, q_f, k_f, v_f, scale, causal=False, block=FP8_BLOCK):
    """Per-element bound [B,H,Sq,d] on |O_kernel - O_exact| (the rounding of
    r P to e4m3 plus the float32 arithmetic) and the per-row float32
    score-error bound [B,H,Sq] (natural log units)."""
    q, k, v = (dequantise_blocks(t, f, block) for t, f in ((q8, q_f), (k8, k_f), (v8, v_f)))
    Sk = k.shape[2]
    r = v_ratios(v_f, Sk, block)                                   # [B,H,Sk]
    p = attention_probs(q, k, scale, causal)
    av = np.abs(v)
    rel = np.einsum("bhij,bhjc->bhic", p, av)
    lmax = 1.0 / np.max(p, axis=-1, keepdims=True)
    Sq = p.shape[-2]
    vis = np.tril(np.ones((Sq, Sk))) if causal else np.ones((Sq, Sk))
    absum = np.einsum("ij,bhjc->bhic", vis, av / r[..., None])     # sum_j |v_j| / r_j over visible keys
    rounding = 2.0 ** -4 * rel + 2.0 ** -10 * absum / lmax
    shift = np.abs(np.log2(r)).max(axis=2)                         # [B,H]
    f32 = float32_bound_of(q, k, v, scale, causal, shift_max=shift, extra_roundings=2)
    return rounding + f32, score_error_bound_of(q, k, scale, causal)
