"""GPU parity of the e4m3 forward (fa_fwd_fp8) against the oracle: exact
attention of the dequantised inputs, within the per-element bound of rounding
the unnormalised probabilities to e4m3 (oracle.fp8_output_bound) plus the
bf16 output rounding; LSE within the forward's LSE tolerance."""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_50_amd as fa
from oracle import (attention_fp8_reference, e4m3_decode, fp8_float32_bound, fp8_output_bound,
                    fp8_score_error_bound, summation_gamma)
from parity import LSE_REL, oracle_rows
from workloads import make_inputs, quantise_e4m3, quantise_e4m3_per_head

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def quantised(B, H, Sq, Sk, d, seed, key_ramp=0.0, amax=224.0):
    q, k, v = make_inputs(B, H, Sq, Sk, d, seed=seed, key_ramp=key_ramp)
    (q8, qs), (k8, ks), (v8, vs) = (quantise_e4m3(t.float(), amax) for t in (q, k, v))
    return q8, k8, v8, qs, ks, vs


def run(q8, k8, v8, qs, ks, vs, causal, tau=8.0):
    o, lse = fa.forward_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), qs, ks, vs, causal=causal, tau=tau)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def bounds(q8, k8, v8, qs, ks, vs, scale, causal):
    """Per-element bound of the kernel's O error: rounding P to e4m3 plus the
    float32 arithmetic (oracle.fp8_output_bound + oracle.fp8_float32_bound)."""
    return (fp8_output_bound(q8, k8, v8, qs, ks, vs, scale, causal)
            + fp8_float32_bound(q8, k8, v8, qs, ks, vs, scale, causal))


def row_bounds(q8, k8, v8, qs, ks, vs, scale, b, h, rows):
    """bounds() of causal rows i of slice (b, h), each on its key prefix."""
    return np.stack([bounds(q8[b:b + 1, h:h + 1, i:i + 1], k8[b:b + 1, h:h + 1, :i + 1],
                            v8[b:b + 1, h:h + 1, :i + 1], qs, ks, vs, scale, False)[0, 0, 0] for i in rows])


def check(o, lse, O, L, bound, what, score_bound=0.0):
    """O within the bound of rounding P plus the float32 arithmetic (bound)
    plus the bf16 output rounding; LSE within the forward's relative tolerance
    plus the float32 accumulation bound of the row's scores (score_bound,
    oracle.fp8_score_error_bound)."""
    err = np.abs(o - O)
    allowed = bound + 2.0 ** -8 * np.abs(O)
    lse_err = np.maximum(np.abs(lse - L) - score_bound, 0.0) / np.maximum(1.0, np.abs(L))
    stats = dict(o_max=float(err.max()), o_mean=float(err.mean()), bound_max=float(bound.max()),
                 worst_ratio=float((err / allowed).max()), lse_rel=float(lse_err.max()))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    assert np.all(err <= allowed), (what, stats)
    assert stats["lse_rel"] <= LSE_REL, (what, stats)
    return stats


@pytest.mark.parametrize("Sq,Sk,causal", [(1, 1, False), (17, 17, True), (128, 128, False), (257, 257, True),
                                          (200, 333, False), (384, 384, True)])
def test_fp8_small_shapes_every_element(Sq, Sk, causal):
    say(f"fp8 fwd B2 H3 Sq={Sq} Sk={Sk} causal={causal}")
    d = 128
    q8, k8, v8, qs, ks, vs = quantised(2, 3, Sq, Sk, d, seed=Sq * 7 + Sk)
    o, lse = run(q8, k8, v8, qs, ks, vs, causal)
    scale = 1 / math.sqrt(d)
    O, L = attention_fp8_reference(q8, k8, v8, qs, ks, vs, scale, causal)
    bound = bounds(q8, k8, v8, qs, ks, vs, scale, causal)
    say(check(o, lse, O, L, bound, f"{Sq}x{Sk} c{causal}"))


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_fp8_many_heads_every_element(tau):
    """Enough heads for several rounds of workgroups, ragged length."""
    say(f"fp8 fwd B1 H64 S1000 causal tau={tau}")
    d = 128
    q8, k8, v8, qs, ks, vs = quantised(1, 64, 1000, 1000, d, seed=31)
    o, lse = run(q8, k8, v8, qs, ks, vs, True, tau=tau)
    scale = 1 / math.sqrt(d)
    O, L = attention_fp8_reference(q8, k8, v8, qs, ks, vs, scale, True)
    bound = bounds(q8, k8, v8, qs, ks, vs, scale, True)
    say(check(o, lse, O, L, bound, f"H64 S1000 tau={tau}"))


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_fp8_key_ramp_every_element(tau):
    """Keys biased along the queries' mean direction, growing over the key
    index (six standard deviations of q.k by the last key): the row max rises
    tile after tile, so the conditional rescale fires often (tau 0: at every
    rise)."""
    say(f"fp8 fwd B1 H4 S1536 causal key ramp tau={tau}")
    d = 128
    q8, k8, v8, qs, ks, vs = quantised(1, 4, 1536, 1536, d, seed=41, key_ramp=6.0)
    o, lse = run(q8, k8, v8, qs, ks, vs, True, tau=tau)
    scale = 1 / math.sqrt(d)
    O, L = attention_fp8_reference(q8, k8, v8, qs, ks, vs, scale, True)
    bound = bounds(q8, k8, v8, qs, ks, vs, scale, True)
    say(check(o, lse, O, L, bound, f"ramp tau={tau}"))


def test_fp8_extreme_codes_and_zero_queries():
    """Tensors scaled so their largest magnitudes land on e4m3's largest
    finite value (448), and query rows of all-zero codes, whose attention is
    the plain mean of the visible V rows."""
    say("fp8 fwd B2 H2 S300 non-causal and causal, amax 448, zero query rows")
    d = 128
    q8, k8, v8, qs, ks, vs = quantised(2, 2, 300, 300, d, seed=43, amax=448.0)
    assert int((q8 & 0x7F).max()) == 0x7E and int((v8 & 0x7F).max()) == 0x7E
    q8[:, :, ::7] = 0
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        o, lse = run(q8, k8, v8, qs, ks, vs, causal)
        O, L = attention_fp8_reference(q8, k8, v8, qs, ks, vs, scale, causal)
        bound = bounds(q8, k8, v8, qs, ks, vs, scale, causal)
        say(check(o, lse, O, L, bound, f"amax 448 causal={causal}"))
        # zero query rows: uniform weights, so O is the mean of the visible V rows
        v = e4m3_decode(v8) * vs
        for i in range(0, 300, 7):
            n_vis = i + 1 if causal else 300
            mean = v[:, :, :n_vis].mean(axis=2)
            assert np.abs(O[:, :, i] - mean).max() < 1e-12
            assert np.abs(L[:, :, i] - math.log(n_vis)).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_per_head_descales_every_element(causal):
    """Heads of very different magnitudes, each quantised with its own factor
    (head_descales [3,B,H]); once with per-tensor factors 1, once with
    per-tensor factors 2, 0.5, 4 and the per-head factors divided by them
    (the two multiply)."""
    say(f"fp8 fwd per-head descales B2 H4 S300 causal={causal}")
    B, H, S, d = 2, 4, 300, 128
    q, k, v = make_inputs(B, H, S, S, d, seed=47)
    mag = torch.tensor([1.0, 8.0, 0.125, 2.0]).view(1, H, 1, 1)
    (q8, qh), (k8, kh), (v8, vh) = (quantise_e4m3_per_head(t.float() * mag) for t in (q, k, v))
    scale = 1 / math.sqrt(d)
    O, L = attention_fp8_reference(q8, k8, v8, qh.numpy(), kh.numpy(), vh.numpy(), scale, causal)
    bound = bounds(q8, k8, v8, qh.numpy(), kh.numpy(), vh.numpy(), scale, causal)
    # head 1 reaches scores of std ~64: float32 accumulation moves small-|LSE| rows
    sb = fp8_score_error_bound(q8, k8, qh.numpy(), kh.numpy(), scale, causal)
    for tensor_f in ((1.0, 1.0, 1.0), (2.0, 0.5, 4.0)):
        hd = torch.stack([qh / tensor_f[0], kh / tensor_f[1], vh / tensor_f[2]]).contiguous().to(DEV)
        o, lse = fa.forward_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), *tensor_f, causal=causal, head_descales=hd)
        torch.cuda.synchronize()
        say(check(o.cpu().double().numpy(), lse.cpu().double().numpy(), O, L, bound,
                  f"per-head causal={causal} tensor factors {tensor_f}", score_bound=sb))


def test_fp8_long_causal_sampled():
    """The causal B1 H16 S8192 d128 shape, sampled heads and rows (a causal
    row is the non-causal result over its key prefix)."""
    say("fp8 fwd B1 H16 S8192 causal, sampled")
    B, H, S, d = 1, 16, 8192, 128
    q8, k8, v8, qs, ks, vs = quantised(B, H, S, S, d, seed=3)
    o, lse = run(q8, k8, v8, qs, ks, vs, True)
    scale = 1 / math.sqrt(d)
    rng = np.random.default_rng(3)
    rows = sorted(set(rng.choice(S, size=24, replace=False).tolist()) | {0, 1, 255, 256, S - 1})
    deq = [torch.from_numpy(e4m3_decode(t) * s) for t, s in ((q8, qs), (k8, ks), (v8, vs))]
    for b, h in [(0, 0), (0, 9)]:
        O, L = oracle_rows(deq[0], deq[1], deq[2], scale, True, [(b, h)], rows)
        bound = row_bounds(q8, k8, v8, qs, ks, vs, scale, b, h, rows)
        say(check(o[b, h, rows], lse[b, h, rows], O[0], L[0], bound, f"head {h}"))


def test_fp8_error_does_not_drift_with_sequence_length():
    """Error of the e4m3 forward on sampled rows of causal B1 H2 d128 inputs at
    S = 1024 ... 8192: against exact attention of the dequantised inputs (the
    kernel's own error: within the bound at every length, and its mean no
    larger at 8192 than twice that at 1024, since the softmax and P V
    accumulate in fp32), and, reported beside it, against exact attention of
    the unquantised bf16 inputs (the end-to-end error of quantising Q, K, V)."""
    d, scale = 128, 1 / math.sqrt(128)
    rng = np.random.default_rng(11)
    means = {}
    for S in (1024, 2048, 4096, 8192):
        say(f"fp8 drift S={S}")
        q, k, v = make_inputs(1, 2, S, S, d, seed=50 + S // 1024)
        (q8, qs), (k8, ks), (v8, vs) = (quantise_e4m3(t.float()) for t in (q, k, v))
        o, lse = run(q8, k8, v8, qs, ks, vs, True)
        rows = sorted(set(rng.choice(S, size=32, replace=False).tolist()) | {S - 1})
        deq = [torch.from_numpy(e4m3_decode(t) * s) for t, s in ((q8, qs), (k8, ks), (v8, vs))]
        errs, errs_in = [], []
        for h in (0, 1):
            O, L = oracle_rows(deq[0], deq[1], deq[2], scale, True, [(0, h)], rows)
            bound = row_bounds(q8, k8, v8, qs, ks, vs, scale, 0, h, rows)
            check(o[0, h, rows], lse[0, h, rows], O[0], L[0], bound, f"S={S} head {h}")
            errs.append(np.abs(o[0, h, rows] - O[0]))
            Ob, _ = oracle_rows(q, k, v, scale, True, [(0, h)], rows)
            errs_in.append(np.abs(o[0, h, rows] - Ob[0]))
        e, ei = np.concatenate(errs), np.concatenate(errs_in)
        means[S] = float(e.mean())
        say(f"S={S}: kernel error vs dequantised inputs max {e.max():.4g} mean {e.mean():.4g}; "
            f"vs unquantised bf16 inputs max {ei.max():.4g} mean {ei.mean():.4g}")
    assert means[8192] <= 2.0 * means[1024], means


def test_fp8_longest_head_sampled():
    """The largest head the boundary accepts at d = 128 (8,387,583 keys),
    300 queries, non-causal, e4m3 inputs.  Sampled rows against the oracle's
    key-range attention of the dequantised inputs over 1M-key chunks, merged
    by log-sum-exp; the P-rounding bound from the same chunks: sum_j p_j |v_j|
    is the merged attention of |V|, and l_max = exp(LSE - max_j s_j)."""
    from oracle import attention_partial, dequantise, merge_partials
    d, Sq = 128, 300
    Sk = (1 << 31) // (d * 2) - 1024 - 1
    say(f"fp8 fwd longest head B1 H1 Sq={Sq} Sk={Sk}")
    q8, k8, v8, qs, ks, vs = quantised(1, 1, Sq, Sk, d, seed=62)
    o, lse = run(q8, k8, v8, qs, ks, vs, False)
    scale = 1 / math.sqrt(d)
    rows = [0, 131, 255, 256, 299]
    qq = dequantise(q8[:, :, rows], qs)
    O_c, L_c, A_c, smax, vabs, sabs, qkabs = [], [], [], -np.inf, 0.0, 0.0, 0.0
    for a in range(0, Sk, 1 << 20):
        kk, vv = dequantise(k8[:, :, a:a + (1 << 20)], ks), dequantise(v8[:, :, a:a + (1 << 20)], vs)
        n = kk.shape[2]
        Oc, Lc = attention_partial(qq, kk, vv, scale, 0, 0, n)
        Ac, _ = attention_partial(qq, kk, np.abs(vv), scale, 0, 0, n)
        O_c.append(Oc); L_c.append(Lc); A_c.append(Ac)
        sc = scale * np.einsum("bhic,bhjc->bhij", qq, kk)
        smax = np.maximum(smax, sc.max(axis=-1))
        sabs = np.maximum(sabs, np.abs(sc).max(axis=-1))
        qkabs = np.maximum(qkabs, np.einsum("bhic,bhjc->bhij", np.abs(qq), np.abs(kk)).max(axis=-1))
        vabs = vabs + np.abs(vv).sum(axis=2)
    O, L = merge_partials(np.stack(O_c), np.stack(L_c))
    A, _ = merge_partials(np.stack(A_c), np.stack(L_c))
    lmax = np.exp(L - smax)
    # fp8_output_bound and fp8_float32_bound from the same chunks
    u = 2.0 ** -24
    eps = d * u / (1 - d * u) * scale * qkabs + 8 * u * sabs
    f32 = (np.expm1(2 * eps) + 2 * summation_gamma(Sk) + 16 * u)[..., None] * A
    bound = 2.0 ** -4 * A + 2.0 ** -10 * vabs[:, :, None, :] / lmax[..., None] + f32
    say(check(o[:, :, rows], lse[:, :, rows], O, L, bound, "fp8 longest head"))


def test_fp8_causal_prefix_independence_bitwise():
    """Causal row i depends on keys 0..i only, bit for bit: replacing every
    later K and V row by e4m3's largest codes (which raises the row max of
    the later rows of the same waves, so their rescale branch is taken) leaves
    rows 0..i of O and LSE unchanged."""
    say("fp8 fwd causal prefix independence")
    S, d, i = 320, 128, 150
    q8, k8, v8, qs, ks, vs = quantised(1, 2, S, S, d, seed=13)
    o1, l1 = run(q8, k8, v8, qs, ks, vs, True)
    g = torch.Generator().manual_seed(14)
    k2, v2 = k8.clone(), v8.clone()
    sign = torch.randint(0, 2, k2[:, :, i + 1:].shape, generator=g).to(torch.uint8) << 7
    k2[:, :, i + 1:] = 0x7E | sign                     # +-448
    v2[:, :, i + 1:] = 0xFE                            # -448
    o2, l2 = run(q8, k2, v2, qs, ks, vs, True)
    assert np.array_equal(o1[:, :, :i + 1], o2[:, :, :i + 1])
    assert np.array_equal(l1[:, :, :i + 1], l2[:, :, :i + 1])
    assert not np.array_equal(o1[:, :, i + 1:], o2[:, :, i + 1:])


def test_fp8_run_to_run_bitwise():
    say("fp8 fwd run-to-run")
    q8, k8, v8, qs, ks, vs = quantised(1, 4, 1000, 1000, 128, seed=15)
    a = run(q8, k8, v8, qs, ks, vs, True)
    b = run(q8, k8, v8, qs, ks, vs, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---- d = 64 (64-byte rows: one 64-dim step for S^T, two 32-dim output blocks)
@pytest.mark.parametrize("Sq,Sk,causal", [(1, 1, False), (17, 17, True), (128, 128, False), (257, 257, True),
                                          (200, 333, False), (384, 384, True)])
def test_fp8_d64_small_shapes_every_element(Sq, Sk, causal):
    say(f"fp8 fwd d64 B2 H3 Sq={Sq} Sk={Sk} causal={causal}")
    d = 64
    q8, k8, v8, qs, ks, vs = quantised(2, 3, Sq, Sk, d, seed=Sq * 11 + Sk)
    o, lse = run(q8, k8, v8, qs, ks, vs, causal)
    scale = 1 / math.sqrt(d)
    O, L = attention_fp8_reference(q8, k8, v8, qs, ks, vs, scale, causal)
    bound = bounds(q8, k8, v8, qs, ks, vs, scale, causal)
    sb = fp8_score_error_bound(q8, k8, qs, ks, scale, causal)
    say(check(o, lse, O, L, bound, f"d64 {Sq}x{Sk} c{causal}", sb))


@pytest.mark.parametrize("tau", [0.0, 8.0])
def test_fp8_d64_many_heads_and_key_ramp_every_element(tau):
    """64 heads at S = 1000 (ragged last tile), and the rescale-stress key
    ramp at S = 1536, at d = 64."""
    d = 64
    scale = 1 / math.sqrt(d)
    for (B, H, S, ramp, seed) in [(1, 64, 1000, 0.0, 71), (1, 4, 1536, 6.0, 73)]:
        say(f"fp8 fwd d64 B{B} H{H} S{S} ramp={ramp} tau={tau}")
        q8, k8, v8, qs, ks, vs = quantised(B, H, S, S, d, seed=seed, key_ramp=ramp)
        o, lse = run(q8, k8, v8, qs, ks, vs, True, tau)
        O, L = attention_fp8_reference(q8, k8, v8, qs, ks, vs, scale, True)
        bound = bounds(q8, k8, v8, qs, ks, vs, scale, True)
        sb = fp8_score_error_bound(q8, k8, qs, ks, scale, True)
        say(check(o, lse, O, L, bound, f"d64 H{H} S{S} ramp={ramp} tau={tau}", sb))


def test_fp8_d64_causal_prefix_independence_and_run_to_run_bitwise():
    say("fp8 fwd d64 causal prefix independence, run to run")
    S, i, d = 320, 150, 64
    q8, k8, v8, qs, ks, vs = quantised(1, 2, S, S, d, seed=75)
    o1, l1 = run(q8, k8, v8, qs, ks, vs, True)
    o1b, l1b = run(q8, k8, v8, qs, ks, vs, True)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    k2, v2 = k8.clone(), v8.clone()
    k2[:, :, i + 1:] = 0x7E
    v2[:, :, i + 1:] = 0xFE
    o2, l2 = run(q8, k2, v2, qs, ks, vs, True)
    assert np.array_equal(o1[:, :, :i + 1], o2[:, :, :i + 1])
    assert np.array_equal(l1[:, :, :i + 1], l2[:, :, :i + 1])
    assert not np.array_equal(o1[:, :, i + 1:], o2[:, :, i + 1:])
