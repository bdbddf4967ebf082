"""GPU parity of the MXFP4 forward (fa_fwd_mxfp4: MXFP4 Q and K, e4m3 V)
against the oracle: exact attention of the decoded tensors, within the
per-element bound of rounding P to e4m3 and the float32 arithmetic
(oracle.mxfp4_bounds) plus the bf16 output rounding; LSE within the
forward's LSE tolerance plus the float32 score-accumulation bound."""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_50_amd as fa
from oracle import attention_mxfp4_reference, mxfp4_bounds
from parity import LSE_REL
from workloads import make_inputs, quantise_e4m3, quantise_mxfp4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def quantised(B, H, Sq, Sk, seed, key_ramp=0.0, row_mag=False):
    q, k, v = make_inputs(B, H, Sq, Sk, D, seed=seed, key_ramp=key_ramp)
    q, k = q.float(), k.float()
    if row_mag:
        # rows of very different magnitudes, so the blocks' E8M0 scales vary widely
        g = torch.Generator().manual_seed(seed + 1)
        q = q * torch.exp2(torch.randint(-4, 5, (B, H, Sq, 1), generator=g).float())
        k = k * torch.exp2(torch.randint(-4, 5, (B, H, Sk, 1), generator=g).float())
    q4, qs = quantise_mxfp4(q)
    k4, ks = quantise_mxfp4(k)
    v8, vs = quantise_e4m3(v.float())
    return q4, qs, k4, ks, v8, vs


def run(q4, qs, k4, ks, v8, vs, causal, tau=8.0):
    o, lse = fa.forward_mxfp4(q4.to(DEV), qs.to(DEV), k4.to(DEV), ks.to(DEV), v8.to(DEV), vs, causal=causal,
                              tau=tau)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def check(o, lse, O, L, bound, score_bound, what):
    err = np.abs(o - O)
    allowed = bound + 2.0 ** -8 * np.abs(O)
    lse_err = np.maximum(np.abs(lse - L) - score_bound, 0.0) / np.maximum(1.0, np.abs(L))
    stats = dict(o_max=float(err.max()), o_mean=float(err.mean()), worst_ratio=float(np.where(allowed > 0, err / np.where(allowed > 0, allowed, 1.0), 0.0).max()),
                 lse_rel=float(lse_err.max()))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    assert np.all(err <= allowed), (what, stats)
    assert stats["lse_rel"] <= LSE_REL, (what, stats)
    return stats


def full_check(inputs, causal, tau, what):
    q4, qs, k4, ks, v8, vs = inputs
    o, lse = run(q4, qs, k4, ks, v8, vs, causal, tau)
    scale = 1 / math.sqrt(D)
    O, L = attention_mxfp4_reference(q4, qs, k4, ks, v8, vs, scale, causal)
    bound, sb = mxfp4_bounds(q4, qs, k4, ks, v8, vs, scale, causal)
    return check(o, lse, O, L, bound, sb, what)


@pytest.mark.parametrize("Sq,Sk,causal", [(1, 1, False), (17, 17, True), (128, 128, False), (257, 257, True),
                                          (200, 333, False), (384, 384, True)])
def test_mxfp4_small_shapes_every_element(Sq, Sk, causal):
    say(f"mxfp4 fwd B2 H3 Sq={Sq} Sk={Sk} causal={causal}")
    say(full_check(quantised(2, 3, Sq, Sk, seed=Sq * 5 + Sk), causal, 8.0, f"{Sq}x{Sk} c{causal}"))


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_mxfp4_many_heads_every_element(tau):
    say(f"mxfp4 fwd B1 H64 S1000 causal tau={tau}")
    say(full_check(quantised(1, 64, 1000, 1000, seed=91), True, tau, f"H64 S1000 tau={tau}"))


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_mxfp4_key_ramp_and_row_magnitudes_every_element(tau):
    """Keys biased along the queries' mean direction (six standard deviations
    of q.k by the last key: the row max keeps rising, so the conditional
    rescale fires) and rows scaled by 2^-4 .. 2^4 (block scales spread over
    eight binades)."""
    say(f"mxfp4 fwd B1 H4 S1536 causal key ramp, row magnitudes, tau={tau}")
    say(full_check(quantised(1, 4, 1536, 1536, seed=93, key_ramp=6.0, row_mag=True), True, tau, f"ramp tau={tau}"))


def test_mxfp4_zero_query_rows_are_the_mean_of_visible_v():
    """Query rows of all-zero elements score 0 against every key: their
    output is the plain mean of the visible (decoded) V rows."""
    say("mxfp4 fwd zero query rows")
    q4, qs, k4, ks, v8, vs = quantised(2, 2, 300, 300, seed=95)
    q4[:, :, ::7] = 0
    from oracle import e4m3_decode
    v = e4m3_decode(v8) * vs
    for causal in (False, True):
        say(full_check((q4, qs, k4, ks, v8, vs), causal, 8.0, f"zero rows causal={causal}"))
        O, L = attention_mxfp4_reference(q4, qs, k4, ks, v8, vs, 1 / math.sqrt(D), causal)
        for i in range(0, 300, 7):
            n_vis = i + 1 if causal else 300
            assert np.abs(O[:, :, i] - v[:, :, :n_vis].mean(axis=2)).max() < 1e-12
            assert np.abs(L[:, :, i] - math.log(n_vis)).max() < 1e-12


def test_mxfp4_long_causal_sampled():
    """The causal B1 H16 S8192 d128 shape, sampled heads and rows, each on
    its key prefix."""
    say("mxfp4 fwd B1 H16 S8192 causal, sampled")
    S = 8192
    q4, qs, k4, ks, v8, vs = quantised(1, 16, S, S, seed=3)
    o, lse = run(q4, qs, k4, ks, v8, vs, True)
    scale = 1 / math.sqrt(D)
    rng = np.random.default_rng(3)
    rows = sorted(set(rng.choice(S, size=16, replace=False).tolist()) | {0, 1, 255, 256, S - 1})
    for h in (0, 9):
        for i in rows:
            sl = lambda t, n: t[:, h:h + 1, :n]                                  # noqa: E731
            qi = lambda t: t[:, h:h + 1, i:i + 1]                                 # noqa: E731
            O, L = attention_mxfp4_reference(qi(q4), qi(qs), sl(k4, i + 1), sl(ks, i + 1), sl(v8, i + 1), vs,
                                             scale, False)
            bound, sb = mxfp4_bounds(qi(q4), qi(qs), sl(k4, i + 1), sl(ks, i + 1), sl(v8, i + 1), vs, scale, False)
            check(o[:, h:h + 1, i:i + 1], lse[:, h:h + 1, i:i + 1], O, L, bound, sb, f"head {h} row {i}")
    say(f"sampled rows {len(rows)} x 2 heads ok")


def test_mxfp4_causal_prefix_independence_and_run_to_run_bitwise():
    say("mxfp4 fwd causal prefix independence, run to run")
    S, i = 320, 150
    q4, qs, k4, ks, v8, vs = quantised(1, 2, S, S, seed=97)
    o1, l1 = run(q4, qs, k4, ks, v8, vs, True)
    o1b, l1b = run(q4, qs, k4, ks, v8, vs, True)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    k2, ks2, v2 = k4.clone(), ks.clone(), v8.clone()
    k2[:, :, i + 1:] = 0x77                                  # every element 6 ...
    ks2[:, :, i + 1:] = 135                                  # ... times 2^8
    v2[:, :, i + 1:] = 0xFE                                  # -448
    o2, l2 = run(q4, qs, k2, ks2, v2, vs, True)
    assert np.array_equal(o1[:, :, :i + 1], o2[:, :, :i + 1])
    assert np.array_equal(l1[:, :, :i + 1], l2[:, :, :i + 1])
    assert not np.array_equal(o1[:, :, i + 1:], o2[:, :, i + 1:])
