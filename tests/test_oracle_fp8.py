"""Pins of the e4m3 oracle (oracle/fp8.py) against the format's definition,
a library conversion of the same format, and a brute-force rounding of P."""
import math

import numpy as np
import torch

from oracle import (attention_forward, attention_probs, dequantise, e4m3_decode, fp8_output_bound,
                    fp8_score_error_bound)


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


def test_per_slice_descales_apply_slice_by_slice():
    """A [B,H] descale scales slice (b, h) -- not a row or a dim -- by its own
    factor: the result equals the per-tensor form applied to each slice."""
    g = torch.Generator().manual_seed(9)
    codes = torch.randint(0, 256, (2, 3, 5, 4), generator=g).to(torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                  # no NaN codes
    f = np.array([[0.5, 2.0, 3.0], [0.25, 8.0, 1.5]])
    got = dequantise(codes, f)
    for b in range(2):
        for h in range(3):
            assert np.array_equal(got[b, h], dequantise(codes[b:b + 1, h:h + 1], f[b, h])[0, 0])
    assert np.array_equal(dequantise(codes, 2.0), 2.0 * e4m3_decode(codes))


def test_score_bound_holds_for_float32_sums():
    """Scores summed in float32 -- term by term in order, and by torch's
    float32 matmul -- differ from the exact ones by no more than
    fp8_score_error_bound / scale per row; the bound is the worst case (it
    assumes every rounding error adds up), so a typical error is a small
    fraction of it, but not a vanishing one."""
    g = torch.Generator().manual_seed(5)
    B, H, S, d = 1, 2, 24, 128
    q8, qs = _quantise(torch.randn(B, H, S, d, generator=g) * 8)
    k8, ks = _quantise(torch.randn(B, H, S, d, generator=g) * 8)
    q, k = dequantise(q8, qs), dequantise(k8, ks)
    exact = np.einsum("bhic,bhjc->bhij", q, k)
    for causal in (False, True):
        bound = fp8_score_error_bound(q8, k8, qs, ks, 1.0, causal)
        seq = np.zeros_like(exact, dtype=np.float32)
        q32, k32 = q.astype(np.float32), k.astype(np.float32)
        for c in range(d):
            seq = (seq + q32[..., :, None, c] * k32[..., None, :, c]).astype(np.float32)
        lib = torch.from_numpy(q32) @ torch.from_numpy(k32).transpose(-1, -2)
        vis = np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
        for got in (seq.astype(np.float64), lib.double().numpy()):
            err = np.where(vis, np.abs(got - exact), 0.0).max(axis=-1)
            assert np.all(err <= bound)
        err_seq = np.where(vis, np.abs(seq.astype(np.float64) - exact), 0.0).max(axis=-1)
        assert np.max(err_seq / bound) > 5e-3     # 1.4e-2 here: a worst-case bound


def test_summation_bound_holds_for_float32_sums():
    """summation_gamma(n - 1) * sum |x| bounds the error of float32 sums of n
    terms -- sequential (cumsum), pairwise (numpy) and torch's reduction --
    of positive and of signed terms up to 4 M of them; the sequential sums of
    positive terms reach a few percent of it (it is not vacuous)."""
    from oracle import summation_gamma
    rng = np.random.default_rng(0)
    worst = 0.0
    for n in (2, 100, 1000, 10_000, 1 << 20, 1 << 22):
        for kind in ("pos", "signed"):
            x = (rng.random(n) if kind == "pos" else rng.standard_normal(n)).astype(np.float32)
            exact = float(np.sum(x.astype(np.float64)))
            bound = float(summation_gamma(n - 1)) * float(np.sum(np.abs(x.astype(np.float64))))
            sums = (np.cumsum(x, dtype=np.float32)[-1], np.sum(x, dtype=np.float32), torch.from_numpy(x).sum().item())
            for s in sums:
                assert abs(float(s) - exact) <= bound, (n, kind)
            if kind == "pos" and n >= 1000:
                worst = max(worst, abs(float(sums[0]) - exact) / bound)
    assert worst > 0.02, worst


def test_float32_pipeline_within_both_bounds():
    """A float32 rendering of the e4m3 forward's arithmetic (scores summed in
    float32, P = 2^(s c - m) in float32 rounded to e4m3 for P V, float32 row
    sum and P V sums, one division) differs from exact attention of the
    dequantised inputs by no more than fp8_output_bound + fp8_float32_bound."""
    from oracle import fp8_float32_bound
    g = torch.Generator().manual_seed(17)
    B, H, S, d = 1, 2, 130, 64
    q8, qs = _quantise(torch.randn(B, H, S, d, generator=g) * 3)
    k8, ks = _quantise(torch.randn(B, H, S, d, generator=g) * 3)
    v8, vs = _quantise(torch.randn(B, H, S, d, generator=g))
    scale = 1 / math.sqrt(d)
    q, k, v = (torch.from_numpy(dequantise(t, f)).float() for t, f in ((q8, qs), (k8, ks), (v8, vs)))
    for causal in (False, True):
        O, _ = attention_forward(q.double(), k.double(), v.double(), scale, causal)
        s = (q @ k.transpose(-1, -2)) * torch.tensor(scale * 1.4426950408889634, dtype=torch.float32)
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
        m = s.amax(dim=-1, keepdim=True)
        p = torch.exp2(s - m)
        p8 = p.to(torch.float8_e4m3fn).to(torch.float32)
        o = (p8 @ v) / p.sum(dim=-1, keepdim=True)
        err = np.abs(o.double().numpy() - O)
        allowed = (fp8_output_bound(q8, k8, v8, qs, ks, vs, scale, causal)
                   + fp8_float32_bound(q8, k8, v8, qs, ks, vs, scale, causal))
        assert np.all(err <= allowed)
        assert err.max() > 0.05 * allowed.max()
