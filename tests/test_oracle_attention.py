"""Pins of the exact-attention oracle against things other than itself.

Brute-force scalar loops, a hand-worked example, closed forms for special
inputs, high-precision log-sum-exp, structural invariants (probabilities sum
to one, causal prefix independence) and finite differences for the gradients.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_forward, attention_backward, attention_probs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- brute force
def brute_forward(q, k, v, scale, causal):
    """Scalar loops with math.exp; one query row at a time."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    O = np.zeros((B, H, Sq, v.shape[3]))
    L = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                keys = [j for j in range(Sk) if (not causal or j <= i)]
                s = {j: scale * sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) for j in keys}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                tot = sum(w.values())
                for c in range(v.shape[3]):
                    O[b, h, i, c] = sum(w[j] * v[b, h, j, c] for j in keys) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


def brute_backward(q, k, v, do, scale, causal):
    """Gradients by the chain rule written per element (scalar loops)."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                keys = [j for j in range(Sk) if (not causal or j <= i)]
                s = {j: scale * sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) for j in keys}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                tot = sum(w.values())
                p = {j: w[j] / tot for j in keys}
                # dL/dP_ij = dO_i . v_j ; softmax Jacobian: dS_ij = P_ij (g_j - sum_k P_ik g_k)
                g = {j: sum(do[b, h, i, c] * v[b, h, j, c] for c in range(v.shape[3])) for j in keys}
                gbar = sum(p[j] * g[j] for j in keys)
                for j in keys:
                    ds = p[j] * (g[j] - gbar)
                    for c in range(d):
                        dq[b, h, i, c] += scale * ds * k[b, h, j, c]
                        dk[b, h, j, c] += scale * ds * q[b, h, i, c]
                    for c in range(v.shape[3]):
                        dv[b, h, j, c] += p[j] * do[b, h, i, c]
    return dq, dk, dv


@pytest.mark.parametrize("Sq,Sk,d,causal", [(1, 1, 1, False), (2, 3, 4, False), (3, 3, 4, True),
                                            (17, 17, 8, True), (17, 5, 8, False), (5, 17, 4, False)])
def test_forward_matches_brute_force(Sq, Sk, d, causal):
    rng = np.random.default_rng(100 + Sq * 7 + Sk + d)
    q = rng.standard_normal((1, 2, Sq, d))
    k = rng.standard_normal((1, 2, Sk, d))
    v = rng.standard_normal((1, 2, Sk, d))
    scale = 1 / math.sqrt(d)
    O, L = attention_forward(q, k, v, scale, causal)
    Ob, Lb = brute_forward(q, k, v, scale, causal)
    assert np.max(np.abs(O - Ob)) < 1e-12
    assert np.max(np.abs(L - Lb)) < 1e-12


@pytest.mark.parametrize("Sq,Sk,d,causal", [(2, 3, 4, False), (3, 3, 4, True), (17, 17, 8, True)])
def test_backward_matches_brute_force(Sq, Sk, d, causal):
    rng = np.random.default_rng(7 + Sq + Sk + d)
    q = rng.standard_normal((1, 1, Sq, d))
    k = rng.standard_normal((1, 1, Sk, d))
    v = rng.standard_normal((1, 1, Sk, d))
    do = rng.standard_normal((1, 1, Sq, d))
    scale = 0.7
    got = attention_backward(q, k, v, do, scale, causal)
    ref = brute_backward(q, k, v, do, scale, causal)
    for g, r in zip(got, ref):
        assert np.max(np.abs(g - r)) < 1e-12


def test_worked_example_by_hand():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_2x2.json")))
    q = np.array(ex["q"])[None, None]
    k = np.array(ex["k"])[None, None]
    v = np.array(ex["v"])[None, None]
    do = np.array(ex["dout"])[None, None]
    O, L = attention_forward(q, k, v, ex["scale"])
    np.testing.assert_allclose(O[0, 0], ex["O"], atol=1e-14)
    np.testing.assert_allclose(L[0, 0], ex["LSE"], atol=1e-14)
    dq, dk, dv = attention_backward(q, k, v, do, ex["scale"])
    np.testing.assert_allclose(dq[0, 0], ex["dQ"], atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], ex["dK"], atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], ex["dV"], atol=1e-14)


# -------------------------------------------------------------- closed forms
def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 5, 8))
    k = rng.standard_normal((1, 1, 1, 8))
    v = rng.standard_normal((1, 1, 1, 8))
    O, L = attention_forward(q, k, v, 0.3)
    np.testing.assert_allclose(O[0, 0], np.repeat(v[0, 0], 5, axis=0), atol=1e-15)
    np.testing.assert_allclose(L[0, 0], 0.3 * (q[0, 0] @ k[0, 0, 0]), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_uniform_weights(causal):
    rng = np.random.default_rng(2)
    S, d = 9, 4
    q = np.zeros((1, 1, S, d))
    k = rng.standard_normal((1, 1, S, d))
    v = rng.standard_normal((1, 1, S, d))
    O, L = attention_forward(q, k, v, 1.0, causal)
    for i in range(S):
        n = i + 1 if causal else S
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, :n].mean(axis=0), atol=1e-14)
        assert abs(L[0, 0, i] - math.log(n)) < 1e-14


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(3)
    d = 4
    k = rng.standard_normal((1, 1, 6, d))
    v = rng.standard_normal((1, 1, 6, d))
    q = 60.0 * k[:, :, 2:3] / np.linalg.norm(k[0, 0, 2])
    k = k.copy()
    k[0, 0, 2] *= 3.0  # key 2 wins by a wide margin
    O, _ = attention_forward(q, k, v, 1.0)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 2], atol=1e-12)


def test_lse_matches_high_precision():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 40
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 4, 16)) * 3
    k = rng.standard_normal((1, 1, 50, 16)) * 3
    v = rng.standard_normal((1, 1, 50, 16))
    _, L = attention_forward(q, k, v, 0.25)
    for i in range(4):
        s = [mpmath.mpf(0.25) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(q[0, 0, i], k[0, 0, j]))
             for j in range(50)]
        ref = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))
        assert abs(L[0, 0, i] - float(ref)) < 1e-13


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_are_a_distribution(causal):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 2, 33, 8)) * 4
    k = rng.standard_normal((2, 2, 33, 8)) * 4
    P = attention_probs(q, k, 0.5, causal)
    assert P.min() >= 0
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
    if causal:
        assert np.all(np.triu(P[0, 0], 1) == 0)
    # all-ones values must give all-ones output: the weights are normalised
    O, _ = attention_forward(q, k, np.ones((2, 2, 33, 8)), 0.5, causal)
    np.testing.assert_allclose(O, 1.0, atol=1e-13)


def test_causal_rows_depend_only_on_prefix():
    rng = np.random.default_rng(6)
    S, d = 24, 8
    q = rng.standard_normal((1, 1, S, d))
    k = rng.standard_normal((1, 1, S, d))
    v = rng.standard_normal((1, 1, S, d))
    O, L = attention_forward(q, k, v, 0.4, causal=True)
    i = 10
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] = 1e3 * rng.standard_normal((1, 1, S - i - 1, d))
    v2[:, :, i + 1:] = -7e2
    O2, L2 = attention_forward(q, k2, v2, 0.4, causal=True)
    assert np.array_equal(O[:, :, :i + 1], O2[:, :, :i + 1])
    assert np.array_equal(L[:, :, :i + 1], L2[:, :, :i + 1])
    assert not np.allclose(O[:, :, i + 1:], O2[:, :, i + 1:])


def test_non_causal_equals_causal_on_last_row():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 12, 4))
    k = rng.standard_normal((1, 1, 12, 4))
    v = rng.standard_normal((1, 1, 12, 4))
    O1, L1 = attention_forward(q, k, v, 1.0, causal=False)
    O2, L2 = attention_forward(q, k, v, 1.0, causal=True)
    np.testing.assert_allclose(O1[0, 0, -1], O2[0, 0, -1], atol=1e-14)
    assert not np.allclose(O1[0, 0, 0], O2[0, 0, 0])


# ----------------------------------------------------------------- gradients
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_finite_differences(causal):
    rng = np.random.default_rng(9)
    Sq, Sk, d = 5, 5, 3
    q = rng.standard_normal((1, 1, Sq, d))
    k = rng.standard_normal((1, 1, Sk, d))
    v = rng.standard_normal((1, 1, Sk, d))
    do = rng.standard_normal((1, 1, Sq, d))
    scale = 0.8
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        O, _ = attention_forward(q_, k_, v_, scale, causal)
        return float((O * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{a + "_": b for a, b in args_p.items()}) -
                        loss(**{a + "_": b for a, b in args_m.items()})) / (2 * h)
        rel = np.max(np.abs(num - g)) / max(1e-12, np.max(np.abs(g)))
        assert rel < 1e-6, (name, rel)


def test_row_identity_for_D():
    """sum_j P_ij dP_ij equals sum_c dO_ic O_ic (the two forms of D)."""
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 1, 7, 4))
    k = rng.standard_normal((1, 1, 9, 4))
    v = rng.standard_normal((1, 1, 9, 4))
    do = rng.standard_normal((1, 1, 7, 4))
    P = attention_probs(q, k, 1.0)[0, 0]
    O, _ = attention_forward(q, k, v, 1.0)
    dP = do[0, 0] @ v[0, 0].T
    np.testing.assert_allclose((P * dP).sum(1), (do[0, 0] * O[0, 0]).sum(1), atol=1e-13)


def test_mistake_in_a_copy_is_caught():
    """A planted mistake (dropped max subtraction with huge logits) must fail
    the brute-force comparison -- guards the test itself, on the CPU."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 1, 3, 2)) * 40
    k = rng.standard_normal((1, 1, 3, 2)) * 40
    v = rng.standard_normal((1, 1, 3, 2))
    with np.errstate(over="ignore", invalid="ignore"):
        s = q[0, 0] @ k[0, 0].T
        bad = (np.exp(s) / np.exp(s).sum(1, keepdims=True)) @ v[0, 0]
    Ob, _ = brute_forward(q, k, v, 1.0, False)
    assert not np.allclose(bad, Ob[0, 0], atol=1e-6)
