"""The conditional rescale, observed (FA4 paper §3.1.4, Eq. 6, as summarised
on "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for
Asymmetric Hardware Scaling"; the lazy-rescale item of "How FlashAttention 4
Works"): the instrumented forward counts, per (b, h), the wavefront-level
corrections it takes after each wavefront's first key tile; the oracle's
step-by-step model (oracle.conditional_rescale_forward with 128-key blocks and
groups of 32 rows, the kernel's tile and wavefront) counts the same events.

Decisions near the threshold may differ between the kernel's float32 scores
and the oracle's float64 ones.  A flipped decision also moves later ones (an
early correction raises the reference max, so later rises exceed tau less
often), so the count is not monotone in tau; each head's count is checked
against the range of the model's counts at tau - delta, tau and tau + delta
(delta = 1e-3 in log2 units, far above the float32 score error at these
magnitudes), widened by 2."""
import sys

import numpy as np
import pytest
import torch

import exact_attention_50_amd as fa
from oracle import conditional_rescale_forward
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DELTA = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def counted(q, k, v, causal, tau):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, H, Sq, d = q.shape
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    ev = torch.zeros((B, H), dtype=torch.int32, device=DEV)
    fa.fa_fwd_rescale_count(qd, kd, vd, o, lse, ev, causal=causal, tau=tau)
    o2, lse2 = fa.forward(qd, kd, vd, causal=causal, tau=tau)
    torch.cuda.synchronize()
    # the instrumented kernel computes exactly what fa_fwd computes
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    return ev.cpu().numpy()


def model_events(q, k, v, scale, causal, tau):
    _, _, st = conditional_rescale_forward(q, k, v, scale, causal, tau=tau, block_n=128, group_rows=32)
    return st["group_events"]


@pytest.mark.parametrize("tau", [8.0, 2.0])
def test_rescale_stress_counts_match_model(tau):
    """The rescale-stress workload (B4 H32 S4096 d64 causal, 256-row
    workgroups with 128-key tiles): four heads' counts against the model."""
    w = WORKLOADS[4]
    say(f"rescale events {w.name} tau={tau}")
    q, k, v = workload_inputs(w)
    ev = counted(q, k, v, True, tau)
    for b, h in [(0, 0), (1, 7), (2, 20), (3, 31)]:
        sl = [t[b:b + 1, h:h + 1] for t in (q, k, v)]
        m = [model_events(*sl, w.scale, True, t) for t in (tau - DELTA, tau, tau + DELTA)]
        say(f"  head ({b},{h}): kernel {ev[b, h]}, model at tau -/0/+ delta {m}")
        assert min(m) - 2 <= ev[b, h] <= max(m) + 2, (b, h, ev[b, h], m)
        assert ev[b, h] > 0
    say(f"  all heads: {int(ev.sum())} corrections after the first tile")


def test_counts_fall_with_tau_and_noncausal_counts():
    """tau = 0 (the eager online softmax) corrects at every rise of a
    wavefront's max, tau = 8 far less often and tau = 64 never after the first
    tile; non-causal 256-row workgroups counted against the model too."""
    q, k, v = make_inputs(2, 64, 1024, 1024, 64, seed=71, key_ramp=6.0)
    c0, c8, c64 = (int(counted(q, k, v, False, t).sum()) for t in (0.0, 8.0, 64.0))
    say(f"non-causal B2 H64 S1024 d64 ramp: tau 0 / 8 / 64 -> {c0} / {c8} / {c64}")
    assert c0 > c8 > 0 and c64 == 0
    ev = counted(q, k, v, False, 8.0)
    for b, h in [(0, 3), (1, 60)]:
        sl = [t[b:b + 1, h:h + 1] for t in (q, k, v)]
        m = [model_events(*sl, 1 / 8, False, t) for t in (8.0 - DELTA, 8.0, 8.0 + DELTA)]
        say(f"  head ({b},{h}): kernel {ev[b, h]}, model at tau -/0/+ delta {m}")
        assert min(m) - 2 <= ev[b, h] <= max(m) + 2, (b, h, ev[b, h], m)


def test_split_form_counts_and_outputs():
    """Few causal blocks: the split form (each wavefront visits every other
    64-key tile).  Outputs are bitwise those of fa_fwd (checked in counted())
    and the counts are non-negative and fall with tau."""
    q, k, v = make_inputs(1, 2, 2048, 2048, 128, seed=73, key_ramp=6.0)
    c0, c8 = (counted(q, k, v, True, t) for t in (0.0, 8.0))
    say(f"split form causal B1 H2 S2048 d128 ramp: tau 0 {c0.tolist()}, tau 8 {c8.tolist()}")
    assert np.all(c0 >= c8) and int(c0.sum()) > 0
