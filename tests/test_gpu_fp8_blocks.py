"""GPU parity of the e4m3 forward with per-block factors (fa_fwd_fp8_blocks:
one float factor per 128 rows of each (batch, head) slice of Q, K, V)
against the oracle: exact attention of the block-dequantised tensors, within
the bound of rounding r P to e4m3 and the float32 arithmetic
(oracle.fp8_blockscaled_bounds) plus the bf16 output rounding; LSE within
the forward's LSE tolerance plus the float32 score-accumulation bound."""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_50_amd as fa
from oracle import attention_fp8_blockscaled_reference, fp8_blockscaled_bounds
from parity import LSE_REL
from workloads import make_inputs, quantise_e4m3_blocks

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def quantised(B, H, Sq, Sk, seed, key_ramp=0.0, spread=0, d=D):
    """Seeded bf16 inputs in float32; spread > 0 scales each 128-row block by
    2^u, u uniform in -spread .. spread (V's blocks then span a wide range of
    ratios to the largest), before block quantisation."""
    q, k, v = (t.float() for t in make_inputs(B, H, Sq, Sk, d, seed=seed, key_ramp=key_ramp))
    if spread:
        g = torch.Generator().manual_seed(seed + 1)
        for t in (q, k, v):
            S = t.shape[2]
            nb = -(-S // 128)
            e = torch.randint(-spread, spread + 1, (B, H, nb), generator=g).float()
            t.mul_(torch.exp2(e).repeat_interleave(128, dim=2)[:, :, :S, None])
    return quantise_e4m3_blocks(q) + quantise_e4m3_blocks(k) + quantise_e4m3_blocks(v)


def run(q8, qf, k8, kf, v8, vf, causal, tau=8.0):
    o, lse = fa.forward_fp8_blocks(q8.to(DEV), k8.to(DEV), v8.to(DEV), qf.to(DEV), kf.to(DEV), vf.to(DEV),
                                   causal=causal, tau=tau)
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
    q8, qf, k8, kf, v8, vf = inputs
    o, lse = run(q8, qf, k8, kf, v8, vf, causal, tau)
    scale = 1 / math.sqrt(q8.shape[-1])
    O, L = attention_fp8_blockscaled_reference(q8, k8, v8, qf, kf, vf, scale, causal)
    bound, sb = fp8_blockscaled_bounds(q8, k8, v8, qf, kf, vf, scale, causal)
    return check(o, lse, O, L, bound, sb, what)


@pytest.mark.parametrize("Sq,Sk,causal", [(1, 1, False), (17, 17, True), (128, 128, False), (257, 257, True),
                                          (200, 333, False), (384, 384, True)])
def test_fp8_blocks_small_shapes_every_element(Sq, Sk, causal):
    say(f"fp8 blocks B2 H3 Sq={Sq} Sk={Sk} causal={causal}")
    say(full_check(quantised(2, 3, Sq, Sk, seed=Sq * 7 + Sk, spread=3), causal, 8.0, f"{Sq}x{Sk} c{causal}"))


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_fp8_blocks_many_heads_every_element(tau):
    say(f"fp8 blocks B1 H64 S1000 causal tau={tau}")
    say(full_check(quantised(1, 64, 1000, 1000, seed=81, spread=2), True, tau, f"H64 S1000 tau={tau}"))


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_fp8_blocks_key_ramp_wide_v_ratios_every_element(tau):
    """The rescale-stress key ramp, and block magnitudes over 2^-6 .. 2^6, so
    some V blocks sit 2^-12 below the head's largest (their r P often falls
    below e4m3's normal range)."""
    say(f"fp8 blocks B1 H4 S1536 causal key ramp, spread 6, tau={tau}")
    say(full_check(quantised(1, 4, 1536, 1536, seed=83, key_ramp=6.0, spread=6), True, tau, f"ramp tau={tau}"))


def test_fp8_blocks_equal_factors_match_the_per_tensor_forward():
    """With every block's factor equal, the block form computes what the
    per-tensor form computes, up to float32 summation order."""
    say("fp8 blocks: equal factors vs per-tensor")
    q, k, v = (t.float() for t in make_inputs(1, 4, 640, 640, D, seed=85))
    codes, f = [], []
    for t in (q, k, v):
        c, fb = quantise_e4m3_blocks(t)
        codes.append(c)
        f.append(torch.full_like(fb, 0.02))
    o_b, l_b = run(codes[0], f[0], codes[1], f[1], codes[2], f[2], True)
    o_t, l_t = fa.forward_fp8(*(c.to(DEV) for c in codes), 0.02, 0.02, 0.02, causal=True)
    torch.cuda.synchronize()
    o_t, l_t = o_t.cpu().double().numpy(), l_t.cpu().double().numpy()
    assert np.abs(l_b - l_t).max() <= 1e-5 * max(1.0, np.abs(l_t).max())
    assert np.abs(o_b - o_t).max() <= 2.0 ** -7 * max(1.0, np.abs(o_t).max())


def test_fp8_blocks_long_causal_sampled():
    """The causal B1 H16 S8192 d128 shape with block spread 2, sampled heads
    and rows, each on its key prefix."""
    say("fp8 blocks B1 H16 S8192 causal, sampled")
    S = 8192
    q8, qf, k8, kf, v8, vf = quantised(1, 16, S, S, seed=3, spread=2)
    o, lse = run(q8, qf, k8, kf, v8, vf, True)
    scale = 1 / math.sqrt(D)
    rng = np.random.default_rng(3)
    rows = sorted(set(rng.choice(S, size=16, replace=False).tolist()) | {0, 1, 127, 128, S - 1})
    for h in (0, 9):
        for i in rows:
            nb = i // 128 + 1
            hq = lambda t: t[:, h:h + 1, i:i + 1]                       # noqa: E731
            hk = lambda t: t[:, h:h + 1, :i + 1]                        # noqa: E731
            qfi = qf[:, h:h + 1, i // 128:i // 128 + 1]
            kfi, vfi = kf[:, h:h + 1, :nb], vf[:, h:h + 1, :]
            # the kernel's ratio reference is the head's largest V factor over all blocks
            O, L = attention_fp8_blockscaled_reference(hq(q8), hk(k8), hk(v8), qfi, kfi, vfi[:, :, :nb], scale, False)
            bound, sb = fp8_blockscaled_bounds(hq(q8), hk(k8), hk(v8), qfi, kfi, vfi[:, :, :nb], scale, False)
            # widen the rounding term to the head's largest factor (the prefix's may be smaller)
            ratio = float(vfi.max() / vfi[:, :, :nb].max())
            check(o[:, h:h + 1, i:i + 1], lse[:, h:h + 1, i:i + 1], O, L, bound * ratio, sb, f"head {h} row {i}")
    say(f"sampled rows {len(rows)} x 2 heads ok")


def test_fp8_blocks_causal_prefix_independence_and_run_to_run_bitwise():
    say("fp8 blocks causal prefix independence, run to run")
    S, i = 320, 150
    q8, qf, k8, kf, v8, vf = quantised(1, 2, S, S, seed=87, spread=2)
    o1, l1 = run(q8, qf, k8, kf, v8, vf, True)
    o1b, l1b = run(q8, qf, k8, kf, v8, vf, True)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    k2, v2 = k8.clone(), v8.clone()
    k2[:, :, i + 1:] = 0x7E                                  # 448 ...
    v2[:, :, i + 1:] = 0xFE                                  # ... and -448 after row i
    o2, l2 = run(q8, qf, k2, kf, v2, vf, True)
    assert np.array_equal(o1[:, :, :i + 1], o2[:, :, :i + 1])
    assert np.array_equal(l1[:, :, :i + 1], l2[:, :, :i + 1])
    assert not np.array_equal(o1[:, :, i + 1:], o2[:, :, i + 1:])


@pytest.mark.parametrize("Sq,Sk,causal,tau", [(17, 17, True, 8.0), (200, 333, False, 8.0), (384, 384, True, 0.0),
                                              (1000, 1000, True, 8.0)])
def test_fp8_blocks_d64_every_element(Sq, Sk, causal, tau):
    say(f"fp8 blocks d64 B2 H3 Sq={Sq} Sk={Sk} causal={causal} tau={tau}")
    say(full_check(quantised(2, 3, Sq, Sk, seed=Sq * 13 + Sk, spread=3, d=64), causal, tau,
                   f"d64 {Sq}x{Sk} c{causal} tau={tau}"))
