"""Helpers shared by the GPU parity tests: oracle values on sampled outputs
and the error statistics checked against the stated tolerances.

Tolerances (fixed by the task's acceptance criteria, written here once):
  O        max |err| <= 1e-2 and mean |err| <= 1e-3 (bf16 output)
  LSE      |err| <= 1e-4 * max(1, |LSE|)   (relative, with an absolute floor
           of 1e-4 where the LSE itself is near 0, e.g. causal row 0)
  dQ/dK/dV max |err| <= 2e-2
"""
import numpy as np
import torch

from oracle import attention_forward, attention_backward
from oracle.exp2_emulation import bf16_round

O_MAX, O_MEAN, LSE_REL, GRAD_MAX = 1e-2, 1e-3, 1e-4, 2e-2


def oracle_rows(q, k, v, scale, causal, bh_list, rows):
    """Oracle O and LSE for selected (b, h) slices and query rows.

    A causal row i equals the non-causal result over keys 0..i, so it is
    computed on that prefix."""
    d = q.shape[-1]
    O = np.zeros((len(bh_list), len(rows), d))
    L = np.zeros((len(bh_list), len(rows)))
    for n, (b, h) in enumerate(bh_list):
        qs = q[b, h].double().numpy()
        ks = k[b, h].double().numpy()
        vs = v[b, h].double().numpy()
        if not causal:
            o, l = attention_forward(qs[None, None, rows], ks[None, None], vs[None, None], scale)
            O[n], L[n] = o[0, 0], l[0, 0]
        else:
            for m, i in enumerate(rows):
                o, l = attention_forward(qs[None, None, i:i + 1], ks[None, None, :i + 1], vs[None, None, :i + 1],
                                         scale)
                O[n, m], L[n, m] = o[0, 0, 0], l[0, 0, 0]
    return O, L


def check_forward(o_gpu, lse_gpu, O_ref, L_ref, what=""):
    """Compare GPU (bf16 O, fp32 LSE) with the oracle; returns stats."""
    o = o_gpu.double().numpy() if isinstance(o_gpu, torch.Tensor) else o_gpu
    lse = lse_gpu.double().numpy() if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    err = np.abs(o - O_ref)
    # floor: what rounding the exact result to bf16 alone costs
    floor = np.abs(bf16_round(O_ref.astype(np.float32)).astype(np.float64) - O_ref)
    lse_err = np.abs(lse - L_ref) / np.maximum(1.0, np.abs(L_ref))
    stats = dict(o_max=float(err.max()), o_mean=float(err.mean()), o_floor=float(floor.max()),
                 lse_rel=float(lse_err.max()))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    assert stats["o_max"] <= O_MAX, (what, stats)
    assert stats["o_mean"] <= O_MEAN, (what, stats)
    assert stats["lse_rel"] <= LSE_REL, (what, stats)
    return stats


def check_grads(got, ref, what=""):
    out = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        gg = g.double().numpy() if isinstance(g, torch.Tensor) else g
        e = float(np.abs(gg - r).max())
        floor = float(np.abs(bf16_round(r.astype(np.float32)).astype(np.float64) - r).max())
        out[name] = (e, floor)
        assert np.all(np.isfinite(gg)), (what, name)
        assert e <= GRAD_MAX, (what, name, e, floor)
    return out


def oracle_backward_heads(q, k, v, do, scale, causal, bh_list):
    res = []
    for b, h in bh_list:
        args = [t[b:b + 1, h:h + 1].double().numpy() for t in (q, k, v, do)]
        res.append(attention_backward(*args, scale, causal))
    return res
