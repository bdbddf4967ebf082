"""Exact softmax attention in float64 -- test infrastructure only.

Definition followed.  The FA4 paper summary ("FlashAttention-4: Algorithm and
Kernel Pipelining Co-Design for Asymmetric Hardware Scaling", TL;DR and
Method) describes a kernel that computes ordinary exact attention,
O = softmax(scale * Q K^T) V, tile by tile; its conditional rescaling keeps the
result exact once the final 1/l normalisation is applied (§3.1.4).  The
oracle is therefore that definition written out, one (batch, head) slice at a
time, with the full score matrix materialised.

Readings of points the pages leave open (each also listed in the design doc):
  * causal mask: key j is visible to query i iff j <= i (top-left aligned);
  * LSE: natural log of sum_j exp(scale * q_i . k_j) over visible keys;
  * masked scores are exactly -inf, so masked probabilities are exactly 0.

Backward.  The pages give only its shape (five matrix products plus two
element-wise steps, paper §3.2.1); the formulas below are the textbook
derivatives of the forward definition:
  dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P * (dP - D),
  dQ = scale * dS K,  dK = scale * dS^T Q.

Layout: q [B,H,Sq,d], k and v [B,H,Sk,d]; any real dtype, widened exactly to
float64 (bf16 and fp32 values are exactly representable).
"""
import numpy as np


def _f64(x):
    """Widen a numpy array or a CPU torch tensor to a float64 numpy array."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch  # local: the oracle works on numpy; torch only converts
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _scores(q2, k2, scale, causal):
    """S = scale * q2 @ k2^T with masked entries set to -inf (one head)."""
    s = scale * (q2 @ k2.T)
    if causal:
        sq, sk = s.shape
        # visible iff key index <= query index
        hidden = np.arange(sk)[None, :] > np.arange(sq)[:, None]
        s[hidden] = -np.inf
    return s


def attention_probs(q, k, scale, causal=False):
    """P = softmax(scale * Q K^T [+ mask]) as float64 [B,H,Sq,Sk]."""
    q, k = _f64(q), _f64(k)
    B, H, Sq, _ = q.shape
    Sk = k.shape[2]
    P = np.empty((B, H, Sq, Sk))
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], scale, causal)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            P[b, h] = e / e.sum(axis=1, keepdims=True)
    return P


def attention_forward(q, k, v, scale, causal=False):
    """Exact attention: returns (O [B,H,Sq,d], LSE [B,H,Sq]) in float64.

    Per (b, h): S = scale * Q K^T (masked -> -inf); m_i = max_j S_ij;
    l_i = sum_j exp(S_ij - m_i); O = (exp(S - m) / l) V; LSE_i = m_i + ln l_i.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, d = q.shape
    O = np.empty((B, H, Sq, v.shape[3]))
    LSE = np.empty((B, H, Sq))
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], scale, causal)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            O[b, h] = (e / l) @ v[b, h]
            LSE[b, h] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_backward(q, k, v, dout, scale, causal=False):
    """Analytic gradients of exact attention: returns (dQ, dK, dV) in float64.

    The probabilities are recomputed in float64 from q and k; the oracle uses
    its own O for D_i = sum_c dO_ic O_ic.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, Sq, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], scale, causal)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            p = e / e.sum(axis=1, keepdims=True)
            o = p @ v[b, h]
            do = dout[b, h]
            dv[b, h] = p.T @ do
            dp = do @ v[b, h].T
            D = (do * o).sum(axis=1, keepdims=True)
            ds = p * (dp - D)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv
