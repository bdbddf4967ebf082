"""Pins of the conditional-rescaling model (FA4 paper §3.1.4, Eq. 6).

The model must reproduce the exact oracle for every tau and gating
granularity (the pages' invariant that the final 1/l restores the exact
result), reduce to the eager online softmax at tau = 0, skip more as tau
grows, and keep every unnormalised probability below 2^tau.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_forward, conditional_rescale_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(seed, S=160, d=16, ramp=0.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, S, d))
    k = rng.standard_normal((1, 2, S, d))
    v = rng.standard_normal((1, 2, S, d))
    if ramp:
        u = q.mean(axis=2, keepdims=True)
        u /= np.linalg.norm(u, axis=-1, keepdims=True)
        k = k + (ramp * math.sqrt(d) * np.arange(S) / (S - 1))[None, None, :, None] * u
    return q, k, v


def test_tau_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "fa4_algorithm_constants.json")))["tau"]
    assert g["value"] == math.log2(g["factor_bound"])


@pytest.mark.parametrize("tau", [0.0, 8.0, 16.0, 64.0])
@pytest.mark.parametrize("group", [1, 32])
@pytest.mark.parametrize("causal", [False, True])
def test_conditional_rescaling_is_exact(tau, group, causal):
    q, k, v = _inputs(1, ramp=6.0)
    scale = 1 / math.sqrt(16)
    O, L = attention_forward(q, k, v, scale, causal)
    O2, L2, st = conditional_rescale_forward(q, k, v, scale, causal, tau=tau,
                                             block_n=32, group_rows=group)
    assert np.max(np.abs(O - O2)) < 1e-12
    assert np.max(np.abs(L - L2)) < 1e-12
    assert st["max_p"] <= 2.0 ** tau * (1 + 1e-12)
    assert st["min_l"] >= 1.0 - 1e-12


def test_tau_zero_is_eager_online_softmax():
    """At tau = 0 with row gating every rise of a row max is corrected."""
    q, k, v = _inputs(2, ramp=6.0)
    _, _, st = conditional_rescale_forward(q, k, v, 0.25, tau=0.0, block_n=16, group_rows=1)
    assert st["row_rescales"].sum() == st["rising_steps"] > 0


def test_rescale_count_non_increasing_in_tau():
    q, k, v = _inputs(3, S=256, ramp=6.0)
    counts = []
    for tau in (0.0, 1.0, 2.0, 4.0, 8.0, 16.0):
        _, _, st = conditional_rescale_forward(q, k, v, 0.25, tau=tau, block_n=16, group_rows=1)
        counts.append(int(st["row_rescales"].sum()))
    assert all(a >= b for a, b in zip(counts, counts[1:])), counts
    assert counts[0] > counts[-1]


def test_ramp_exercises_both_sides_of_tau():
    """With the key bias ramp some rows cross tau = 8 after their first block
    while most rises of the max stay below it."""
    q, k, v = _inputs(4, S=512, d=64, ramp=6.0)
    _, _, st = conditional_rescale_forward(q, k, v, 1 / 8, tau=8.0, block_n=64, group_rows=1)
    assert st["row_rescales"].sum() > 0
    assert st["rising_steps"] > 10 * st["row_rescales"].sum()


def test_stale_reference_gives_wrong_unnormalised_sum_without_final_division():
    """Guard: with skipped corrections the unnormalised accumulators differ
    from the eager ones, so exactness really comes from the final 1/l."""
    q, k, v = _inputs(5, ramp=6.0)
    _, _, st8 = conditional_rescale_forward(q, k, v, 0.25, tau=8.0, block_n=16)
    assert st8["max_p"] > 1.0     # some probability was taken against a stale max


def test_group_size_changes_event_count_only():
    """Wave-gated correction with per-row selection: the same rows are
    corrected whatever the group size; larger groups run the step in fewer
    (group, block) events than there are row corrections."""
    q, k, v = _inputs(6, S=256, ramp=6.0)
    O1, L1, s1 = conditional_rescale_forward(q, k, v, 0.25, causal=True, tau=4.0, block_n=32, group_rows=1)
    O32, L32, s32 = conditional_rescale_forward(q, k, v, 0.25, causal=True, tau=4.0, block_n=32, group_rows=32)
    assert np.array_equal(s1["row_rescales"], s32["row_rescales"])
    assert np.array_equal(O1, O32) and np.array_equal(L1, L32)
    assert s32["group_events"] <= s1["group_events"] == s1["row_rescales"].sum()
    # per-group counts: with one row per group they are the row counts; a
    # group corrects in a block iff one of its rows does, so its count lies
    # between its rows' largest count and their sum
    assert np.array_equal(s1["group_counts"], s1["row_rescales"])
    assert s32["group_counts"].sum() == s32["group_events"]
    rows = s1["row_rescales"].reshape(s1["row_rescales"].shape[:2] + (-1, 32))
    assert np.all(rows.max(-1) <= s32["group_counts"]) and np.all(s32["group_counts"] <= rows.sum(-1))
    assert s32["group_counts"].max() > 0
