"""Pins of the block-scaled e4m3 oracle (oracle/fp8_blocks.py): block
dequantisation against a scalar loop and the per-tensor form, the V ratios
against their definition, and the output bound against a brute-force
pipeline that rounds r_j P_j with torch's e4m3 conversion."""
import math

import numpy as np
import torch

from oracle import (attention_forward, attention_probs, dequantise, dequantise_blocks, e4m3_decode,
                    fp8_blockscaled_bounds, fp8_output_bound, v_ratios)
from workloads import quantise_e4m3_blocks


def _codes(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * 40).to(torch.float8_e4m3fn).view(torch.uint8)


def test_block_dequantisation_matches_scalar_loop():
    B, H, S, d, blk = 2, 2, 300, 4, 128               # ragged last block (300 = 2 * 128 + 44)
    codes = _codes((B, H, S, d), 1)
    f = np.exp2(np.random.default_rng(1).integers(-4, 5, size=(B, H, 3))).astype(np.float64)
    got = dequantise_blocks(codes, f, blk)
    v = e4m3_decode(codes)
    for b in range(B):
        for h in range(H):
            for i in range(S):
                assert np.array_equal(got[b, h, i], v[b, h, i] * f[b, h, i // blk])


def test_equal_factors_are_the_per_tensor_form():
    codes = _codes((1, 3, 200, 8), 2)
    f = np.full((1, 3, 2), 0.375)
    assert np.array_equal(dequantise_blocks(codes, f), dequantise(codes, 0.375))


def test_v_ratios():
    f = np.array([[[0.5, 2.0, 1.0]]])
    r = v_ratios(f, 300)
    assert r.shape == (1, 1, 300)
    assert np.all(r[0, 0, :128] == 0.25) and np.all(r[0, 0, 128:256] == 1.0) and np.all(r[0, 0, 256:] == 0.5)


def test_quantiser_blocks_round_trip():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(1, 2, 300, 16, generator=g) * torch.exp2(torch.randint(-3, 4, (1, 2, 300, 1), generator=g).float())
    codes, f = quantise_e4m3_blocks(x)
    assert f.shape == (1, 2, 3)
    back = dequantise_blocks(codes, f)
    # each element within half an e4m3 step of its block's grid (2^-4 relative, 2^-10 absolute in codes)
    fr = np.repeat(f.numpy().astype(np.float64), 128, axis=2)[:, :, :300, None]
    err = np.abs(back - x.double().numpy())
    assert np.all(err <= 2.0 ** -4 * np.abs(x.double().numpy()) + 2.0 ** -10 * fr + 1e-12)
    # every block reaches 224 (the factor is its max / 224)
    assert np.allclose(np.abs(e4m3_decode(codes)).reshape(1, 2, -1).max(-1), 224.0)


def test_bound_holds_for_brute_force_rounding_of_scaled_p():
    """Exact attention of block-scaled e4m3 inputs with r_j exp(s_j - max)
    rounded to e4m3 (torch's conversion) before P V, divided back by r_j and
    normalised by the unrounded sum stays within the bound, which is not
    vacuous; V blocks span 2^-6 .. 1 of the largest, so the subnormal term
    matters."""
    g = torch.Generator().manual_seed(7)
    B, H, S, d = 1, 2, 300, 16
    q8, qf = quantise_e4m3_blocks(torch.randn(B, H, S, d, generator=g) * 2)
    k8, kf = quantise_e4m3_blocks(torch.randn(B, H, S, d, generator=g) * 2)
    v = torch.randn(B, H, S, d, generator=g)
    v[:, :, :128] *= 2.0 ** -6
    v8, vf = quantise_e4m3_blocks(v)
    scale = 1 / math.sqrt(d)
    worst = 0.0
    for causal in (False, True):
        qd, kd, vd = dequantise_blocks(q8, qf), dequantise_blocks(k8, kf), dequantise_blocks(v8, vf)
        O, _ = attention_forward(qd, kd, vd, scale, causal)
        p = attention_probs(qd, kd, scale, causal)
        unnorm = p / p.max(axis=-1, keepdims=True)
        r = v_ratios(vf, S)[:, :, None, :]
        r8 = torch.from_numpy(unnorm * r).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        Oq = np.einsum("bhij,bhjc->bhic", r8 / r, vd) / unnorm.sum(-1, keepdims=True)
        bound, _ = fp8_blockscaled_bounds(q8, k8, v8, qf, kf, vf, scale, causal)
        err = np.abs(Oq - O)
        assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
        worst = max(worst, float((err / bound).max()))
    assert worst > 0.05


def test_equal_factors_give_the_per_tensor_rounding_bound():
    q8, k8, v8 = _codes((1, 2, 150, 8), 4), _codes((1, 2, 150, 8), 5), _codes((1, 2, 150, 8), 6)
    f = np.full((1, 2, 2), 0.01)
    bound, _ = fp8_blockscaled_bounds(q8, k8, v8, f, f, f, 0.3, True)
    per_tensor = fp8_output_bound(q8, k8, v8, 0.01, 0.01, 0.01, 0.3, True)
    assert np.all(bound >= per_tensor) and np.all(bound <= per_tensor * 1.01 + 1e-9)
