"""Pins of the e4m3 oracle (oracle/fp8.py) against the format's definition,
a library conversion of the same format, and a brute-force rounding of P."""
import math

import numpy as np
import torch

from oracle import attention_forward, attention_probs, e4m3_decode, fp8_output_bound


def test_named_values():
    # OCP e4m3fn: zero, smallest subnormal 2^-9, largest subnormal 7 * 2^-9,
    # smallest normal 2^-6, one, 1.5, largest 448, NaN
    codes = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0xFE, 0x7F, 0xFF], dtype=np.uint8)
    v = e4m3_decode(codes)
    assert v[0] == 0.0 and v[1] == 0.0 and math.copysign(1.0, v[1]) == -1.0
    assert v[2] == 2.0 ** -9 and v[3] == 7 * 2.0 ** -9 and v[4] == 2.0 ** -6
    assert v[5] == 1.0 and v[6] == 1.5 and v[7] == 448.0 and v[8] == -448.0
    assert np.isnan(v[9]) and np.isnan(v[10])


def test_all_codes_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    pos = got[:127]
    assert np.all(np.diff(pos) > 0)   # monotone over the positive finite codes


def _quantise(x, amax=224.0):
    ds = float(x.abs().max()) / amax
    return (x / ds).to(torch.float8_e4m3fn).view(torch.uint8), ds


def test_bound_holds_for_brute_force_rounding_of_p():
    """Exact attention of e4m3 inputs with P = exp(s - max) rounded to e4m3
    (torch's conversion) before P V and normalised by the unrounded sum stays
    within fp8_output_bound, which is also not vacuous."""
    g = torch.Generator().manual_seed(7)
    B, H, S, d = 1, 2, 96, 16
    q8, qs = _quantise(torch.randn(B, H, S, d, generator=g) * 2)
    k8, ks = _quantise(torch.randn(B, H, S, d, generator=g) * 2)
    v8, vs = _quantise(torch.randn(B, H, S, d, generator=g))
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        q, k, v = e4m3_decode(q8) * qs, e4m3_decode(k8) * ks, e4m3_decode(v8) * vs
        O, _ = attention_forward(q, k, v, scale, causal)
        p = attention_probs(q, k, scale, causal)
        pmax = p.max(axis=-1, keepdims=True)
        unnorm = p / pmax                                   # exp(s - max), max = 1
        r8 = torch.from_numpy(unnorm).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        Oq = np.einsum("bhij,bhjc->bhic", r8, v) / unnorm.sum(-1, keepdims=True)
        bound = fp8_output_bound(q8, k8, v8, qs, ks, vs, scale, causal)
        err = np.abs(Oq - O)
        assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
        assert err.max() > 0.05 * bound.max()
