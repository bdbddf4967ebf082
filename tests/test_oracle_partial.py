"""Pins of oracle.partial (attention over a key range, and the merge of such
parts) against things other than its own formulas: the full-attention oracle
over the union of the ranges, identities, and brute force on a tiny case."""
import math

import numpy as np
import pytest

from oracle import attention_forward, attention_partial, merge_partials


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _parts(q, k, v, scale, bounds, causal, q_offset=0):
    outs = [attention_partial(q, k, v, scale, q_offset, a, b, causal) for a, b in zip(bounds[:-1], bounds[1:])]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bounds", [(0, 40, 96), (0, 1, 33, 95, 96), (0, 17, 18, 50, 96)])
def test_merge_of_any_partition_is_full_attention(causal, bounds):
    rng = np.random.default_rng(len(bounds) * 7 + causal)
    q, k, v = (_rand((2, 3, 96, 16), rng, 1.5) for _ in range(3))
    O_ref, L_ref = attention_forward(q, k, v, 0.3, causal)
    O, L = merge_partials(*_parts(q, k, v, 0.3, bounds, causal))
    assert np.max(np.abs(O - O_ref)) < 1e-12
    assert np.max(np.abs(L - L_ref)) < 1e-12


def test_causal_query_block_with_offset():
    """A block of queries at global rows q0..q0+m-1 against key ranges: the
    merge equals those rows of the full causal attention."""
    rng = np.random.default_rng(5)
    S, q0, m = 80, 24, 30
    q, k, v = (_rand((1, 2, S, 8), rng) for _ in range(3))
    O_ref, L_ref = attention_forward(q, k, v, 0.5, True)
    qb = q[:, :, q0:q0 + m]
    O, L = merge_partials(*_parts(qb, k, v, 0.5, (0, 10, 40, 53, S), True, q_offset=q0))
    assert np.max(np.abs(O - O_ref[:, :, q0:q0 + m])) < 1e-12
    assert np.max(np.abs(L - L_ref[:, :, q0:q0 + m])) < 1e-12


def test_full_range_is_attention_forward():
    rng = np.random.default_rng(6)
    q = _rand((1, 2, 20, 8), rng)
    k, v = _rand((1, 2, 33, 8), rng), _rand((1, 2, 33, 8), rng)
    for causal in (False,):
        O, L = attention_partial(q, k, v, 0.7, 0, 0, 33, causal)
        O_ref, L_ref = attention_forward(q, k, v, 0.7, causal)
        assert np.max(np.abs(O - O_ref)) < 1e-13 and np.max(np.abs(L - L_ref)) < 1e-13
    q2 = _rand((1, 2, 33, 8), rng)
    O, L = attention_partial(q2, k, v, 0.7, 0, 0, 33, True)
    O_ref, L_ref = attention_forward(q2, k, v, 0.7, True)
    assert np.max(np.abs(O - O_ref)) < 1e-13 and np.max(np.abs(L - L_ref)) < 1e-13


def test_one_part_merge_is_identity_and_empty_parts_change_nothing():
    rng = np.random.default_rng(8)
    q, k, v = (_rand((1, 1, 16, 4), rng) for _ in range(3))
    O1, L1 = attention_partial(q, k, v, 1.0, 0, 0, 16, True)
    O, L = merge_partials(O1[None], L1[None])
    assert np.array_equal(O, O1) and np.array_equal(L, L1)
    # keys 10..15 for query rows 0..7 (global 0..7): every row is empty
    Oe, Le = attention_partial(q[:, :, :8], k, v, 1.0, 0, 10, 16, True)
    assert np.all(Oe == 0) and np.all(np.isneginf(Le))
    Oa, La = attention_partial(q[:, :, :8], k, v, 1.0, 0, 0, 10, True)
    Om, Lm = merge_partials(np.stack([Oa, Oe]), np.stack([La, Le]))
    assert np.array_equal(Om, Oa) and np.array_equal(Lm, La)
    # every part empty: O = 0, LSE = -inf
    Oz, Lz = merge_partials(np.stack([Oe, Oe]), np.stack([Le, Le]))
    assert np.all(Oz == 0) and np.all(np.isneginf(Lz))


def test_brute_force_tiny():
    """One query, keys 1..3 of four, scalar loops."""
    q = np.array([[[[0.5, -1.0]]]])
    k = np.array([[[[9.0, 9.0], [1.0, 0.0], [0.0, 1.0], [2.0, 2.0]]]])
    v = np.array([[[[7.0, 7.0], [1.0, 2.0], [3.0, -1.0], [0.5, 0.25]]]])
    scale = 0.8
    s = [scale * (q[0, 0, 0, 0] * k[0, 0, j, 0] + q[0, 0, 0, 1] * k[0, 0, j, 1]) for j in (1, 2, 3)]
    z = sum(math.exp(x) for x in s)
    o = [sum(math.exp(s[t]) * v[0, 0, j, c] for t, j in enumerate((1, 2, 3))) / z for c in (0, 1)]
    O, L = attention_partial(q, k, v, scale, 0, 1, 4)
    assert abs(L[0, 0, 0] - math.log(z)) < 1e-14
    assert max(abs(O[0, 0, 0, c] - o[c]) for c in (0, 1)) < 1e-14


def test_merge_uses_lse_not_row_max():
    """Parts whose score scales differ widely (one range dominates): a merge
    weighted by the parts' maxima instead of their LSEs would be off."""
    rng = np.random.default_rng(9)
    q = _rand((1, 1, 12, 8), rng)
    k = np.concatenate([_rand((1, 1, 20, 8), rng, 0.2), _rand((1, 1, 20, 8), rng, 3.0)], axis=2)
    v = _rand((1, 1, 40, 8), rng)
    O_ref, L_ref = attention_forward(q, k, v, 0.5, False)
    O, L = merge_partials(*_parts(q, k, v, 0.5, (0, 20, 40), False))
    assert np.max(np.abs(O - O_ref)) < 1e-12 and np.max(np.abs(L - L_ref)) < 1e-12
