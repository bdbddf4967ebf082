"""GPU parity of fa_fwd_partial and fa_merge (split-KV / ring-attention
pieces) against the CPU oracle, through the C ABI."""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_50_amd as fa
from oracle import attention_forward, attention_partial, merge_partials
from parity import LSE_REL, O_MAX, O_MEAN, check_forward, oracle_rows
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_partial(o, lse, O, L, what):
    """float32 partial output: same O / LSE tolerances as the forward; rows
    with no visible key must be exactly O = 0, LSE = -inf."""
    o, lse = o.double().numpy(), lse.double().numpy()
    empty = np.isneginf(L)
    assert np.array_equal(np.isneginf(lse), empty), what
    assert np.all(o[empty] == 0.0), what
    seen = ~empty
    err = np.abs(o[seen] - O[seen])
    assert np.all(np.isfinite(o)), what
    assert err.max(initial=0.0) <= O_MAX and (err.mean() if err.size else 0.0) <= O_MEAN, (what, err.max())
    lerr = np.abs(lse[seen] - L[seen]) / np.maximum(1.0, np.abs(L[seen]))
    assert lerr.max(initial=0.0) <= LSE_REL, (what, lerr.max())
    return float(err.max(initial=0.0))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq,Sk,q_off,kb,ke,causal", [
    (100, 300, 0, 0, 300, False), (100, 300, 0, 37, 250, False), (77, 300, 0, 250, 300, False),
    (128, 512, 200, 0, 64, True), (128, 512, 200, 64, 230, True), (128, 512, 200, 230, 512, True),
    (300, 300, 0, 0, 300, True), (300, 300, 0, 129, 300, True), (513, 1024, 511, 700, 1024, True),
    # an even number of 128-row query blocks: the causal launch pairs block 3 with 0 and 2 with
    # 1 in one workgroup each; with keys 300.. rows 0-255 see none, so the second block of
    # each pair is one with no visible key (the early exit between two blocks)
    (512, 1024, 0, 300, 1024, True), (512, 512, 0, 0, 512, True),
])
def test_partial_every_element(d, Sq, Sk, q_off, kb, ke, causal):
    say(f"partial d={d} Sq={Sq} Sk={Sk} q_off={q_off} keys {kb}..{ke} causal={causal}")
    q, _, _ = make_inputs(2, 3, Sq, Sq, d, seed=Sq + d)
    _, k, v = make_inputs(2, 3, Sk, Sk, d, seed=Sk * 3 + d)
    o, lse = fa.forward_partial(q.to(DEV), k.to(DEV), v.to(DEV), q_off, kb, ke, causal=causal)
    torch.cuda.synchronize()
    O, L = attention_partial(q, k, v, 1 / math.sqrt(d), q_off, kb, ke, causal)
    say(check_partial(o.cpu(), lse.cpu(), O, L, f"d{d} {Sq}x{Sk} q_off={q_off} {kb}..{ke} c{causal}"))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tau,emu", [(0.0, 0.25), (64.0, 0.25), (0.0, 1.0), (64.0, 1.0), (8.0, 0.5)])
@pytest.mark.parametrize("Sq,Sk,q_off,kb,ke,causal", [
    (300, 1024, 0, 37, 900, False), (300, 1024, 500, 200, 1024, True), (1000, 1000, 0, 0, 1000, True),
])
def test_partial_tau_and_emulation_every_element(d, tau, emu, Sq, Sk, q_off, kb, ke, causal):
    """The key-range forward at tau 0 (eager rescale), 64 (almost never) and
    8, with software exponentials on a quarter, half or all of the scores;
    keys carry the rescale-stress ramp so row maxima keep rising."""
    say(f"partial d={d} tau={tau} emu={emu} Sq={Sq} Sk={Sk} q_off={q_off} keys {kb}..{ke} causal={causal}")
    q, _, _ = make_inputs(1, 4, Sq, Sq, d, seed=Sq + d + 7)
    _, k, v = make_inputs(1, 4, Sk, Sk, d, seed=Sk + d + 9, key_ramp=6.0)
    o, lse = fa.forward_partial(q.to(DEV), k.to(DEV), v.to(DEV), q_off, kb, ke, causal=causal, tau=tau,
                                emu_frac=emu)
    torch.cuda.synchronize()
    O, L = attention_partial(q, k, v, 1 / math.sqrt(d), q_off, kb, ke, causal)
    say(check_partial(o.cpu(), lse.cpu(), O, L, f"d{d} tau={tau} emu={emu} {Sq}x{Sk} q_off={q_off} {kb}..{ke}"))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 3, 5])
def test_merge_every_element(d, n):
    """Seeded synthetic parts (including empty rows in some parts and rows
    empty in every part) through fa_merge and the oracle merge."""
    say(f"merge d={d} n={n}")
    g = torch.Generator().manual_seed(100 * n + d)
    B, H, S = 2, 3, 129
    op = torch.randn((n, B, H, S, d), generator=g)
    lp = torch.randn((n, B, H, S), generator=g) * 4.0 + 2.0
    drop = torch.rand((n, B, H, S), generator=g) < 0.3
    lp[drop] = -math.inf
    op[drop] = 0.0
    lp[:, :, :, 5] = -math.inf            # row 5: empty in every part
    op[:, :, :, 5] = 0.0
    o, lse = fa.merge(op.to(DEV), lp.to(DEV))
    torch.cuda.synchronize()
    O, L = merge_partials(op, lp)
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    empty = np.isneginf(L)
    assert np.array_equal(np.isneginf(lse), empty) and np.all(o[empty] == 0.0)
    err = np.abs(o - O)
    floor = 2.0 ** -8 * np.abs(O)                       # bf16 rounding of the output
    assert np.all(err <= floor + 1e-6), err.max()
    lerr = np.abs(lse[~empty] - L[~empty]) / np.maximum(1.0, np.abs(L[~empty]))
    assert lerr.max() <= 1e-6


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_partials_then_merge_equal_full_attention(d, causal):
    say(f"split-kv end to end d={d} causal={causal}")
    S = 700
    q, k, v = make_inputs(1, 4, S, S, d, seed=31 + d + causal)
    bounds = [0, 1, 190, 333, 334, 640, S]
    parts = [fa.forward_partial(q.to(DEV), k.to(DEV), v.to(DEV), 0, a, b, causal=causal)
             for a, b in zip(bounds[:-1], bounds[1:])]
    o, lse = fa.merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
    torch.cuda.synchronize()
    O, L = attention_forward(q, k, v, 1 / math.sqrt(d), causal)
    say(check_forward(o.cpu(), lse.cpu(), O, L, f"split-kv d{d} c{causal}"))


def test_split_kv_causal_long_sampled():
    """The benchmark's configuration: causal B1 H16 S8192 d128 as 4 key ranges
    plus the merge, sampled heads and rows against the oracle."""
    w = WORKLOADS[3]
    say(f"split-kv {w.name}")
    q, k, v = (t.to(DEV) for t in workload_inputs(w)[:3])
    bounds = [w.Sk * i // 4 for i in range(5)]
    parts = [fa.forward_partial(q, k, v, 0, a, b, causal=True) for a, b in zip(bounds[:-1], bounds[1:])]
    o, lse = fa.merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    rows = sorted(set(rng.choice(w.Sq, size=32, replace=False).tolist()) |
                  {0, 1, 2047, 2048, 2049, 4095, 4096, 6143, 6144, w.Sq - 1})
    bh = [(0, 0), (0, 11)]
    qc, kc, vc = (t.cpu() for t in (q, k, v))
    O, L = oracle_rows(qc, kc, vc, w.scale, True, bh, rows)
    oc, lc = o.cpu(), lse.cpu()
    og = torch.stack([oc[b, h, rows] for b, h in bh])
    lg = torch.stack([lc[b, h, rows] for b, h in bh])
    say(check_forward(og, lg, O, L, "split-kv S8192"))
