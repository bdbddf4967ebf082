"""The seeded generators are deterministic and follow the stated recipe."""
import math

import torch

from workloads import WORKLOADS, make_inputs


def test_deterministic_per_seed():
    a = make_inputs(1, 2, 64, 64, 16, seed=3, with_dout=True)
    b = make_inputs(1, 2, 64, 64, 16, seed=3, with_dout=True)
    c = make_inputs(1, 2, 64, 64, 16, seed=4, with_dout=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y) and x.dtype == torch.bfloat16 and x.is_contiguous()
    assert not torch.equal(a[0], c[0])


def test_head_subset_matches_full_draw():
    full = make_inputs(1, 4, 32, 32, 8, seed=9, key_ramp=6.0)
    sub = make_inputs(1, 4, 32, 32, 8, seed=9, key_ramp=6.0, heads=(1, 3))
    for x, y in zip(full, sub):
        assert torch.equal(x[:, 1:3], y)


def test_key_ramp_reaches_six_sigma_along_query_mean():
    B, H, S, d = 1, 1, 2048, 64
    q, k, _ = make_inputs(B, H, S, S, d, seed=5, key_ramp=6.0)
    q0, k0, _ = make_inputs(B, H, S, S, d, seed=5)
    u = q0.float().mean(dim=2)[0, 0]
    u = u / u.norm()
    shift = (k.float() - k0.float())[0, 0] @ u
    assert abs(shift[0].item()) < 0.05
    assert abs(shift[-1].item() - 6 * math.sqrt(d)) < 0.5


def test_config_flops():
    w = WORKLOADS[3]
    assert w.flops("fwd") == 4 * 16 * 8192 * 8192 * 128 / 2
    assert WORKLOADS[5].flops("bwd") == 10 * 16 * 4096 * 4096 * 128 / 2
