"""Pins of the MXFP4 oracle (oracle/mxfp4.py): the E2M1 and E8M0 decoders
against the formats' named values and torch's E8M0 type, block decoding
against a scalar loop, and the error bounds against a brute-force pipeline."""
import math

import numpy as np
import torch

from oracle import e4m3_decode
from oracle.mxfp4 import attention_mxfp4_reference, e2m1_decode, e8m0_decode, mx_decode, mxfp4_bounds
from workloads import quantise_e4m3, quantise_mxfp4


def test_e2m1_named_values():
    # OCP E2M1: zero, the subnormal 0.5, then 1, 1.5, 2, 3, 4 and the largest, 6
    assert e2m1_decode(np.arange(8)).tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    neg = e2m1_decode(np.arange(8, 16))
    assert np.array_equal(neg, -e2m1_decode(np.arange(8)))
    assert math.copysign(1.0, neg[0]) == -1.0                     # code 8 is -0
    assert np.all(np.diff(e2m1_decode(np.arange(8))) > 0)
    # every E2M1 value is exact in e4m3 (so the products of the kernel are exact)
    v = torch.tensor(e2m1_decode(np.arange(16)), dtype=torch.float32)
    assert torch.equal(v.to(torch.float8_e4m3fn).to(torch.float32), v)


def test_e8m0_against_torch():
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = e8m0_decode(codes)
    assert np.all((np.isnan(ref) & np.isnan(got)) | (ref == got))
    assert got[127] == 1.0 and np.isnan(got[255])


def test_block_decode_matches_scalar_loop():
    g = torch.Generator().manual_seed(3)
    packed = torch.randint(0, 256, (2, 3, 64), generator=g).to(torch.uint8)
    scales = torch.randint(100, 150, (2, 3, 4), generator=g).to(torch.uint8)
    got = mx_decode(packed, scales)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for a in range(2):
        for b in range(3):
            for e in range(128):
                byte = int(packed[a, b, e // 2])
                code = (byte >> 4) if e % 2 else (byte & 15)
                val = (-1.0 if code & 8 else 1.0) * mags[code & 7] * 2.0 ** (int(scales[a, b, e // 32]) - 127)
                assert got[a, b, e] == val


def test_quantiser_round_trip_within_half_a_step():
    """Input preparation: decoding the quantised codes recovers each element
    to within half an E2M1 step of its block (saturation aside)."""
    g = torch.Generator().manual_seed(4)
    x = torch.randn(4, 256, generator=g)
    packed, scales = quantise_mxfp4(x)
    y = mx_decode(packed, scales)
    step = np.repeat(e8m0_decode(scales), 32, axis=-1)         # 2^X: an E2M1 step is <= 2^X (at 4..6)
    clipped = np.abs(x.numpy()) > 6 * step
    err = np.abs(y - x.numpy())
    assert np.all(err[~clipped] <= step[~clipped] + 1e-12)


def test_bounds_hold_for_brute_force_pipeline():
    """float32 scores of the decoded MXFP4 Q, K; P = exp(s - max) in float32
    rounded to e4m3 (torch) before P V on the e4m3 V; normalised by the float32
    sum: within mxfp4_bounds of exact attention of the decoded tensors, and
    the bound is not vacuous."""
    g = torch.Generator().manual_seed(9)
    B, H, S, d = 1, 2, 96, 64
    q4, qs = quantise_mxfp4(torch.randn(B, H, S, d, generator=g) * 2)
    k4, ks = quantise_mxfp4(torch.randn(B, H, S, d, generator=g) * 2)
    v8, vs = quantise_e4m3(torch.randn(B, H, S, d, generator=g))
    scale = 1 / math.sqrt(d)
    q, k = (torch.from_numpy(mx_decode(a, b)).float() for a, b in ((q4, qs), (k4, ks)))
    v = torch.from_numpy(e4m3_decode(v8) * vs).float()
    for causal in (False, True):
        O, _ = attention_mxfp4_reference(q4, qs, k4, ks, v8, vs, scale, causal)
        s = (q @ k.transpose(-1, -2)) * scale
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
        p = torch.exp(s - s.amax(dim=-1, keepdim=True))
        o = (p.to(torch.float8_e4m3fn).to(torch.float32) @ v) / p.sum(dim=-1, keepdim=True)
        bound, _ = mxfp4_bounds(q4, qs, k4, ks, v8, vs, scale, causal)
        err = np.abs(o.double().numpy() - O)
        assert np.all(err <= bound)
        assert err.max() > 0.05 * bound.max()
