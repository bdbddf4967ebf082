"""The FA4 forward algorithm, step by step, in float64 -- test infrastructure.

This is a model of the method's steps, not of its hardware mapping.  It
follows the FA4 paper summary ("FlashAttention-4: Algorithm and Kernel
Pipelining Co-Design for Asymmetric Hardware Scaling", Key claims and Method,
paper §3.1.4, Eq. 6) and the lazy-rescale item of "How FlashAttention 4
Works":

  keys are visited one block of ``block_n`` at a time; each row keeps a
  reference maximum m_ref that is applied to its running output and row sum;
  when a block raises a row's maximum by more than tau, the running output
  and sum are multiplied by 2^(m_ref - m_new) and m_ref moves up; otherwise
  the correction is skipped and the block's exponentials are taken against
  the stale m_ref (each then at most 2^tau); the output is exact after the
  final division by the row sum.

Readings (listed in the design doc):
  * m and tau are in log2 units: s = scale * log2(e) * q.k, so tau = log2(256)
    = 8 bounds every unnormalised probability by 256;
  * "m_{j-1}" is the reference max currently applied (not the previous
    block's running max), strict test m_new - m_ref > tau, and the first
    block always sets m_ref;
  * gating "at warp granularity": rows are taken in consecutive groups of
    ``group_rows`` (one warp / wavefront); the correction step runs for a
    group when any of its rows needs it, and inside it only the rows whose
    max rose by more than tau move their reference (the others are multiplied
    by exactly 1).  The arithmetic of each row therefore depends on that row
    alone; the group size only changes how often the step runs
    (``group_events``);
  * LSE = (m_ref + log2 l) * ln 2.
"""
import numpy as np

from .attention import _f64

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def conditional_rescale_forward(q, k, v, scale, causal=False, tau=8.0,
                                block_n=64, group_rows=1):
    """Tile-by-tile forward with conditional rescaling.

    Returns (O, LSE, stats).  stats holds, over all (b, h):
      row_rescales   int array [B,H,Sq]: corrections applied to a row (its max
                     rose by more than tau), after its first block
      group_events   number of (group, block) corrections after the first block
      group_counts   int array [B,H,ceil(Sq/group_rows)]: the same per group
      rising_steps   number of (row, block) steps where the row max rose,
                     after the first block
      max_p          largest unnormalised probability seen (<= 2^tau)
      min_l          smallest final row sum (>= 1)
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    c = scale * LOG2E
    O = np.empty((B, H, Sq, v.shape[3]))
    LSE = np.empty((B, H, Sq))
    row_rescales = np.zeros((B, H, Sq), dtype=np.int64)
    group_counts = np.zeros((B, H, (Sq + group_rows - 1) // group_rows), dtype=np.int64)
    group_events = 0
    rising_steps = 0
    max_p = 0.0
    min_l = np.inf
    qi = np.arange(Sq)
    for b in range(B):
        for h in range(H):
            m_ref = np.full(Sq, -np.inf)
            l = np.zeros(Sq)
            acc = np.zeros((Sq, v.shape[3]))
            for blk, k0 in enumerate(range(0, Sk, block_n)):
                k1 = min(k0 + block_n, Sk)
                s = c * (q[b, h] @ k[b, h, k0:k1].T)
                if causal:
                    s[np.arange(k0, k1)[None, :] > qi[:, None]] = -np.inf
                m_blk = s.max(axis=1)
                m_new = np.maximum(m_ref, m_blk)
                if blk > 0:
                    rising_steps += int(np.count_nonzero(m_new > m_ref))
                with np.errstate(invalid="ignore"):
                    need = (m_new - m_ref) > tau        # -inf ref -> inf > tau
                for g0 in range(0, Sq, group_rows):
                    g = slice(g0, min(g0 + group_rows, Sq))
                    if not need[g].any():
                        continue
                    ng = need[g]
                    if blk > 0:
                        group_events += 1
                        group_counts[b, h, g0 // group_rows] += 1
                        row_rescales[b, h, g] += ng
                    with np.errstate(invalid="ignore"):
                        alpha = np.where(np.isfinite(m_ref[g]),
                                         np.exp2(m_ref[g] - m_new[g]), 0.0)
                    alpha = np.where(ng, alpha, 1.0)
                    acc[g] *= alpha[:, None]
                    l[g] *= alpha
                    m_ref[g] = np.where(ng, m_new[g], m_ref[g])
                with np.errstate(invalid="ignore"):
                    p = np.exp2(s - m_ref[:, None])
                p[np.isnan(p)] = 0.0                    # -inf - -inf: no key yet
                max_p = max(max_p, float(p.max()))
                l += p.sum(axis=1)
                acc += p @ v[b, h, k0:k1]
            O[b, h] = acc / l[:, None]
            LSE[b, h] = (m_ref + np.log2(l)) * LN2
            min_l = min(min_l, float(l.min()))
    stats = dict(row_rescales=row_rescales, group_events=group_events, group_counts=group_counts,
                 rising_steps=rising_steps, max_p=max_p, min_l=min_l)
    return O, LSE, stats
