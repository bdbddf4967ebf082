"""The conditional rescale, observed (FA4 paper §3.1.4, Eq. 6, as summarised
on "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for
Asymmetric Hardware Scaling"; the lazy-rescale item of "How FlashAttention 4
Works"): the instrumented forward counts, per 32-row wavefront, the
corrections it takes after its first key tile; the oracle's step-by-step model
(oracle.conditional_rescale_forward with 128-key blocks and groups of 32 rows,
the kernel's tile and wavefront) counts the same events per group.

Decisions near the threshold may differ between the kernel's float32 scores
and the oracle's float64 ones.  A flipped decision also moves later ones (an
early correction raises the reference max, so later rises exceed tau less
often), so counts are not monotone in tau; each wavefront's count is checked
against the range of the model's counts at tau - delta, tau and tau + delta
(delta = 1e-3 in log2 units, far above the float32 score error at these
magnitudes) widened by 1, at least 95 % of the wavefronts must equal the model
at tau, and each head's total must lie in the totals' range widened by 2."""
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
    ev = torch.zeros((B, H, -(-Sq // 32)), dtype=torch.int32, device=DEV)
    fa.fa_fwd_rescale_count(qd, kd, vd, o, lse, ev, causal=causal, tau=tau)
    o2, lse2 = fa.forward(qd, kd, vd, causal=causal, tau=tau)
    torch.cuda.synchronize()
    # the instrumented kernel computes exactly what fa_fwd computes
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    return ev.cpu().numpy()


def model_slots(q, k, v, scale, causal, tau):
    """The model's corrections per 32-row group (the kernel's wavefront)."""
    _, _, st = conditional_rescale_forward(q, k, v, scale, causal, tau=tau, block_n=128, group_rows=32)
    return st["group_counts"][0, 0]


def check_head(ev_head, sl, scale, causal, tau, what):
    """One head: the kernel's per-wavefront counts against the model's per-group
    counts at tau - delta, tau, tau + delta (a flipped near-threshold decision
    moves a wavefront's count by one and its later decisions with it): every
    wavefront within the range widened by 1, at least 95 % equal to the model
    at tau, and the head's total within the totals' range widened by 2."""
    m = [model_slots(*sl, scale, causal, t) for t in (tau - DELTA, tau, tau + DELTA)]
    lo, hi = np.minimum.reduce(m), np.maximum.reduce(m)
    eq = float(np.mean(ev_head == m[1]))
    tot = [int(x.sum()) for x in m]
    say(f"  {what}: kernel total {int(ev_head.sum())}, model totals at tau -/0/+ delta {tot}; "
        f"wavefronts equal to the model {100 * eq:.1f} %; histogram {np.bincount(ev_head, minlength=4)[:6].tolist()}")
    assert np.all((lo - 1 <= ev_head) & (ev_head <= hi + 1)), what
    assert eq >= 0.95, (what, eq)
    assert min(tot) - 2 <= int(ev_head.sum()) <= max(tot) + 2, (what, int(ev_head.sum()), tot)
    return int(ev_head.sum())


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
        assert check_head(ev[b, h], sl, w.scale, True, tau, f"head ({b},{h})") > 0
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
        check_head(ev[b, h], sl, 1 / 8, False, 8.0, f"head ({b},{h})")


def test_split_form_counts_and_outputs():
    """Few causal blocks: the split form (each wavefront visits every other
    64-key tile).  Outputs are bitwise those of fa_fwd (checked in counted())
    and the counts are non-negative and fall with tau."""
    q, k, v = make_inputs(1, 2, 2048, 2048, 128, seed=73, key_ramp=6.0)
    c0, c8 = (counted(q, k, v, True, t).sum(axis=-1) for t in (0.0, 8.0))
    say(f"split form causal B1 H2 S2048 d128 ramp: tau 0 {c0.tolist()}, tau 8 {c8.tolist()}")
    assert np.all(c0 >= c8) and int(c0.sum()) > 0
