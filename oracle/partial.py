"""Attention over a range of keys and the merge of such partial results, in
float64 -- test infrastructure only.

What it computes.  The lecture notes "How FlashAttention 4 Works" list a
fused ring attention for multi-GPU FA4 among the open directions (closing
list).  Its single-GPU pieces are (a) exact attention of a block of queries
over one contiguous range of keys, returning the output normalised over that
range and its log-sum-exp, and (b) the combination of such partial results
over disjoint ranges into attention over their union.  Both are written out
from the definition of softmax attention (the one in ``attention``):

  partial over keys R:  s_ij = scale q_i . k_j for j in R, -inf if masked;
                        LSE_i = log sum_{j in R} exp(s_ij);
                        O_i = sum_{j in R} exp(s_ij - LSE_i) v_j;
                        a row with no visible key: O_i = 0, LSE_i = -inf;
  merge of parts s:     LSE = log sum_s exp(LSE_s);
                        O = sum_s exp(LSE_s - LSE) O_s  (0 and -inf if every
                        part is empty).

Reading taken (also in the design doc): with a key range, the causal mask compares
global indices -- query row i of the block is global query q_offset + i, key
j of the range is global key k_begin + j, visible iff k_begin + j <=
q_offset + i (the top-left-aligned mask of the full problem).

Pins (tests/test_oracle_partial.py): merging partials over any partition of
the keys reproduces ``attention_forward`` over all keys; the full range with
zero offsets is ``attention_forward`` itself; a one-part merge is the
identity; empty parts change nothing; brute force on a tiny case.
"""
import numpy as np

from .attention import _f64


def attention_partial(q, k, v, scale, q_offset, k_begin, k_end, causal=False):
    """(O_part [B,H,Sq,d], LSE_part [B,H,Sq]) over keys k_begin..k_end-1."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, _ = q.shape
    d_v = v.shape[3]
    O = np.zeros((B, H, Sq, d_v))
    LSE = np.full((B, H, Sq), -np.inf)
    kk = k[:, :, k_begin:k_end]
    vv = v[:, :, k_begin:k_end]
    hidden = None
    if causal:
        gq = q_offset + np.arange(Sq)[:, None]
        gk = k_begin + np.arange(k_end - k_begin)[None, :]
        hidden = gk > gq
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ kk[b, h].T)
            if hidden is not None:
                s[hidden] = -np.inf
            m = s.max(axis=1)
            seen = np.isfinite(m)
            if not seen.any():
                continue
            e = np.exp(s[seen] - m[seen][:, None])
            l = e.sum(axis=1)
            O[b, h, seen] = (e / l[:, None]) @ vv[b, h]
            LSE[b, h, seen] = m[seen] + np.log(l)
    return O, LSE


def merge_partials(O_parts, LSE_parts):
    """Combine parts over disjoint key ranges: O_parts [n,...,d], LSE_parts [n,...]."""
    O_parts, LSE_parts = _f64(O_parts), _f64(LSE_parts)
    m = LSE_parts.max(axis=0)
    seen = np.isfinite(m)
    w = np.zeros_like(LSE_parts)
    w[:, seen] = np.exp(LSE_parts[:, seen] - m[seen])
    wsum = w.sum(axis=0)
    O = np.zeros(O_parts.shape[1:])
    LSE = np.full(m.shape, -np.inf)
    O[seen] = (w[:, seen][..., None] * O_parts[:, seen]).sum(axis=0) / wsum[seen][..., None]
    LSE[seen] = m[seen] + np.log(wsum[seen])
    return O, LSE
