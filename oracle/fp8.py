"""Attention on e4m3 (FP8) inputs, in float64 -- test infrastructure only.

What it computes.  The FA4 paper summary ("FlashAttention-4: Algorithm and
Kernel Pipelining Co-Design for Asymmetric Hardware Scaling", precision
discussion) names FP8 as the next operand format.  Inputs are e4m3 codes
with one dequantisation factor per tensor, so the attention they stand for is
the ordinary exact attention of the dequantised tensors:

  Q = q_descale * e4m3(Q8),  K = k_descale * e4m3(K8),  V = v_descale * e4m3(V8),
  O, LSE = attention_forward(Q, K, V)   (the definition in ``attention``),

with each descale one number for the tensor or one per (batch, head) slice.

e4m3 here is the OCP 8-bit format with 4 exponent bits (bias 7), 3 mantissa
bits, subnormals, no infinities and one NaN pattern per sign (S.1111.111);
the largest finite value is 448.  ``e4m3_decode`` writes that definition out.

Rounding the probabilities.  A kernel that rounds its unnormalised
probabilities P_j = 2^(s_j - m) (m at most the row's max, so the largest
P_j >= 1) to e4m3 before P V, while normalising by the sum l of the unrounded
P_j, is off from the exact O by at most

  sum_j (2^-4 P_j + 2^-10 [P_j < 2^-6]) |v_j| / l
      <= 2^-4 sum_j p_j |v_j| + 2^-10 sum_j |v_j| / l_max

per output element (round-to-nearest: half an e4m3 step is 2^-4 of the value
for normal values and 2^-10 below 2^-6; p = exact softmax weights; l_max =
sum_j exp(s_j - max_j s_j) <= l).  ``fp8_output_bound`` returns that bound
per element; the LSE is unaffected (the row sum uses the unrounded P).

Accumulating the scores.  The d products of a score are summed in float32;
the classic summation bound (Higham, Accuracy and Stability of Numerical
Algorithms, ch. 4) puts the error of a sum of n terms in precision u below
gamma_n sum |terms|, gamma_n = n u / (1 - n u).  LSE = log sum_j exp(s_j)
moves by at most the largest score error, so
``fp8_score_error_bound`` returns gamma_d * scale * max_j sum_c |q_c k_jc|
per row (visible keys j).  With e4m3 inputs of large magnitude this exceeds
the float32 LSE tolerance of small-|LSE| rows and is added to it.

Float32 arithmetic on O.  Beside rounding P, the kernel's O moves by the
float32 arithmetic of its steps; ``fp8_float32_bound`` bounds that per
element by

  [ expm1(2 eps) + 2 g_n + 16 u ] * sum_j p_j |v_j|

with u = 2^-24, n = the row's visible keys and
  * eps = the score error of the row (``fp8_score_error_bound``) plus
    8 u max_j |s_j|: the folded score factor (three roundings), the
    scale-and-subtract FMA; a score error delta_j changes the weight p_j by
    at most a factor exp(+-2 max|delta|) after normalisation;
  * g_n for each of the two sums over the keys, the numerator sum_j P_j v_j
    and the row sum l (each term passes through at most n - 1 roundings,
    in any summation order or blocking): the smaller of the worst case
    gamma_n = n u / (1 - n u) and the probabilistic bound of Higham and Mary
    ("A New Approach to Probabilistic Rounding Error Analysis", SIAM J. Sci.
    Comput. 41(5), 2019, Theorem 2.4 and its summation corollary):
    exp(lambda sqrt(n) u + n u^2 / (1 - u)) - 1, which holds with
    probability at least 1 - 2 n exp(-lambda^2 (1 - u)^2 / 2) when the
    rounding errors are independent and of mean zero; lambda = 10 puts the
    failure probability below n * 4e-22.  For the 8.4 M-key rows the worst
    case is vacuous (n u = 0.5) and the probabilistic bound 1.7e-3;
  * 16 u for the fixed number of roundings per element: the exponential
    (within one ulp), the rescale and final 1/l multiplies.
The bf16 rounding of the output is a separate term of the tests (2^-8 |O|).

Pins (tests/test_oracle_fp8.py): the score bound holds for float32
sequential and library sums; the decoder against the format's named
values (0, min subnormal 2^-9, min normal 2^-6, 1, 448, NaN) and against
torch's float8_e4m3fn on all 256 codes; per-slice descales equal the
per-tensor form applied slice by slice; the bound holds for a brute-force
attention that rounds P with torch's e4m3 conversion; the summation bound
holds for float32 sums (sequential, pairwise and library) of up to 4 M
terms and is within 50x of their actual error (not vacuous).
"""
import numpy as np

from .attention import _f64, attention_forward, attention_probs


def e4m3_decode(codes):
    """float64 values of e4m3 codes (uint8 array or tensor)."""
    c = np.asarray(codes.cpu().numpy() if hasattr(codes, "cpu") else codes).astype(np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def dequantise(codes, descale):
    """Values of e4m3 codes [B,H,S,d] times their dequantisation factor: one
    per tensor (a scalar) or one per (batch, head) slice (an array [B,H])."""
    f = np.asarray(descale.cpu().numpy() if hasattr(descale, "cpu") else descale, dtype=np.float64)
    if f.ndim == 2:
        f = f[:, :, None, None]
    elif f.ndim != 0:
        raise ValueError(f"descale must be a scalar or [B,H], got shape {f.shape}")
    return e4m3_decode(codes) * f


def attention_fp8_reference(q8, k8, v8, q_descale, k_descale, v_descale, scale, causal=False):
    """(O, LSE) of exact attention on the dequantised e4m3 inputs."""
    return attention_forward(dequantise(q8, q_descale), dequantise(k8, k_descale), dequantise(v8, v_descale),
                             scale, causal)


def output_bound_of(q, k, v, scale, causal=False):
    """fp8_output_bound on dequantised float arrays q, k, v (any operand
    format whose P is rounded to e4m3 before P V)."""
    p = attention_probs(q, k, scale, causal)                 # exact softmax weights
    av = np.abs(_f64(v))
    rel = np.einsum("bhij,bhjc->bhic", p, av)                # sum_j p_j |v_j|
    # l_max = 1 / max_j p_j (the row sum relative to the row's max score)
    lmax = 1.0 / np.max(p, axis=-1, keepdims=True)
    Sq, Sk = p.shape[-2], p.shape[-1]
    vis = np.tril(np.ones((Sq, Sk))) if causal else np.ones((Sq, Sk))   # visible keys
    absum = np.einsum("ij,bhjc->bhic", vis, av)                          # sum_j |v_j| over them
    return 2.0 ** -4 * rel + 2.0 ** -10 * absum / lmax


def fp8_output_bound(q8, k8, v8, q_descale, k_descale, v_descale, scale, causal=False):
    """Per-element bound [B,H,Sq,d] on |O_kernel - O_exact| from rounding the
    unnormalised probabilities to e4m3 (see the module text)."""
    return output_bound_of(dequantise(q8, q_descale), dequantise(k8, k_descale), dequantise(v8, v_descale),
                           scale, causal)


def score_error_bound_of(q, k, scale, causal=False):
    """fp8_score_error_bound on dequantised float arrays q, k."""
    q, k = np.abs(_f64(q)), np.abs(_f64(k))
    d = q.shape[-1]
    u = 2.0 ** -24
    gamma = d * u / (1.0 - d * u)
    ab = np.einsum("bhic,bhjc->bhij", q, k)
    if causal:
        Sq, Sk = ab.shape[-2:]
        ab = np.where(np.tril(np.ones((Sq, Sk), dtype=bool)), ab, 0.0)
    return gamma * scale * ab.max(axis=-1)


def fp8_score_error_bound(q8, k8, q_descale, k_descale, scale, causal=False):
    """Per-row bound [B,H,Sq] on the float32 accumulation error of the row's
    scores (and so of its LSE): gamma_d * scale * max over visible keys of
    sum_c |q_c k_c| on the dequantised inputs (see the module text)."""
    return score_error_bound_of(dequantise(q8, q_descale), dequantise(k8, k_descale), scale, causal)


U32 = 2.0 ** -24


def summation_gamma(n, lam=10.0):
    """Relative error bound of a float32 sum of n terms, relative to
    sum |terms| (see the module text): min(worst case, probabilistic)."""
    n = np.asarray(n, dtype=np.float64)
    nu = n * U32
    worst = np.where(nu < 1.0, nu / np.maximum(1.0 - nu, 1e-300), np.inf)
    prob = np.expm1(lam * np.sqrt(n) * U32 + n * U32 * U32 / (1.0 - U32))
    return np.minimum(worst, prob)


def float32_bound_of(q, k, v, scale, causal=False, shift_max=None, extra_roundings=0):
    """fp8_float32_bound on dequantised float arrays q, k, v.  shift_max
    ([B,H] or scalar, default none): the largest |log2 r| of a per-key factor
    r the kernel folds into the exponent: r (one rounding, u relative) and its
    log2 (within an ulp, 2 u |log2 r|) add 2 u (|log2 r| + 1) to a score's
    error; extra_roundings: further roundings per term of the row sum or per
    output element beyond the 16 counted here."""
    p = attention_probs(q, k, scale, causal)
    rel = np.einsum("bhij,bhjc->bhic", p, np.abs(_f64(v)))        # sum_j p_j |v_j|
    Sq, Sk = p.shape[-2], p.shape[-1]
    vis = np.tril(np.ones((Sq, Sk), dtype=bool)) if causal else np.ones((Sq, Sk), dtype=bool)
    s_abs = np.abs(scale * np.einsum("bhic,bhjc->bhij", _f64(q), _f64(k)))
    smax = np.where(vis, s_abs, 0.0).max(axis=-1)
    eps = score_error_bound_of(q, k, scale, causal) + 8.0 * U32 * smax
    if shift_max is not None:
        shift = np.asarray(shift_max, dtype=np.float64)
        if shift.ndim == 2:
            shift = shift[:, :, None]
        eps = eps + 2.0 * U32 * (shift + 1.0)
    n = vis.sum(axis=-1).astype(np.float64)                          # [Sq]
    factor = np.expm1(2.0 * eps) + 2.0 * summation_gamma(n) + (16.0 + extra_roundings) * U32
    return factor[..., None] * rel


def fp8_float32_bound(q8, k8, v8, q_descale, k_descale, v_descale, scale, causal=False):
    """Per-element bound [B,H,Sq,d] on what float32 arithmetic adds to the
    kernel's O error beside the rounding of P (see the module text)."""
    return float32_bound_of(dequantise(q8, q_descale), dequantise(k8, k_descale), dequantise(v8, v_descale),
                            scale, causal)
