"""GPU parity of fa_bwd_ds (the five-product backward: dS written by the
dK/dV kernel, dQ = scale dS K from it) against the CPU oracle, called through
the C ABI.  As for fa_bwd, the GPU backward consumes the GPU forward's O and
LSE and the oracle recomputes everything in float64 (max |err| <= 2e-2).

The dK/dV kernel of this form is fa_bwd's with the dS stores added, so dK and
dV must equal fa_bwd's bit for bit; dQ is summed in another order and must
agree with fa_bwd's to bf16 rounding."""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_50_amd as fa
from oracle import attention_backward
from parity import check_grads, oracle_backward_heads
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def both(q, k, v, do, causal, det=False, fill=None):
    """(fa_bwd_ds outputs, fa_bwd outputs) on the GPU forward's O and LSE."""
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal)
    B, H, Sq, d = q.shape
    ws = None
    if fill is not None:
        n = fa.fa_bwd_ds_workspace_bytes(B, H, Sq, k.shape[2], d, causal, det)
        ws = torch.full((n,), fill, dtype=torch.uint8, device=DEV)
    got = fa.backward_ds(qd, kd, vd, o, lse, dod, causal=causal, deterministic=det, workspace=ws)
    ref = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, deterministic=det)
    torch.cuda.synchronize()
    return [t.cpu() for t in got], [t.cpu() for t in ref]


def agree_with_split(got, split, what):
    assert torch.equal(got[1], split[1]), (what, "dK differs from fa_bwd's")
    assert torch.equal(got[2], split[2]), (what, "dV differs from fa_bwd's")
    a, b = got[0].double(), split[0].double()
    # both dQ are fp32 sums of bf16 dS times K, rounded to bf16 once: dS
    # elements formed in two fp32 orders may round to neighbouring bf16
    # values, so beside the final rounding (2^-7 relative covers two ulps) a
    # small share of the tensor's scale is allowed; a misplaced row or key
    # is off by the scale itself
    tol = 2.0 ** -7 * b.abs() + 2.0 ** -8 * float(b.abs().max())
    assert bool(((a - b).abs() <= tol).all()), (what, float((a - b).abs().max()))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq,Sk,causal", [(1, 1, False), (17, 17, True), (64, 200, False), (128, 128, True),
                                          (257, 257, True), (200, 333, False), (384, 384, True)])
def test_small_shapes_every_element(d, Sq, Sk, causal):
    say(f"bwd_ds small d={d} Sq={Sq} Sk={Sk} causal={causal}")
    q, k, v, do = make_inputs(2, 2, Sq, Sk, d, seed=Sq * 31 + Sk + d, with_dout=True)
    got, split = both(q, k, v, do, causal)
    ref = attention_backward(q, k, v, do, 1 / math.sqrt(d), causal)
    say(check_grads(got, ref, f"d{d} {Sq}x{Sk} c{causal}"))
    agree_with_split(got, split, f"d{d} {Sq}x{Sk} c{causal}")


@pytest.mark.parametrize("d,Sq,Sk,causal", [(128, 1000, 1000, True), (64, 1000, 1000, True),
                                            (128, 333, 1100, False), (64, 700, 129, False)])
def test_ragged_multi_slab_every_element(d, Sq, Sk, causal):
    """Several 128-row dS slabs, a ragged last slab and key tile."""
    say(f"bwd_ds ragged d={d} Sq={Sq} Sk={Sk} causal={causal}")
    q, k, v, do = make_inputs(1, 3, Sq, Sk, d, seed=7 * Sq + Sk + d, with_dout=True)
    got, split = both(q, k, v, do, causal, det=True)
    ref = attention_backward(q, k, v, do, 1 / math.sqrt(d), causal)
    say(check_grads(got, ref, f"d{d} {Sq}x{Sk} c{causal}"))
    agree_with_split(got, split, f"d{d} {Sq}x{Sk} c{causal}")


@pytest.mark.parametrize("fill", [0x00, 0xFF])
def test_workspace_contents_do_not_matter(fill):
    """A workspace of NaN bf16 (0xFFFF) or zeros gives the same bits: the dQ
    kernel reads only the dS the dK/dV kernel wrote (causal: no slab part
    above the diagonal)."""
    say(f"bwd_ds workspace fill {fill:#x}")
    q, k, v, do = make_inputs(1, 2, 555, 555, 128, seed=77, with_dout=True)
    a, _ = both(q, k, v, do, True, fill=fill)
    b, _ = both(q, k, v, do, True, fill=0x7F)
    for x, y in zip(a, b):
        assert torch.isfinite(x.float()).all()
        assert torch.equal(x, y)


def test_config5_sampled_heads_and_run_to_run():
    """The causal B1 H16 S4096 d128 backward: two whole heads against the
    oracle, dK and dV equal to fa_bwd's, dQ close to it, three runs equal."""
    w = WORKLOADS[5]
    say(f"bwd_ds {w.name}")
    q, k, v, do = workload_inputs(w)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=w.causal)
    runs = []
    for _ in range(3):
        runs.append([t.cpu() for t in fa.backward_ds(qd, kd, vd, o, lse, dod, causal=w.causal)])
        torch.cuda.synchronize()
    split = [t.cpu() for t in fa.backward(qd, kd, vd, o, lse, dod, causal=w.causal)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
    agree_with_split(runs[0], split, w.name)
    heads = [(0, 0), (0, 13)]
    refs = oracle_backward_heads(q, k, v, do, w.scale, w.causal, heads)
    for (b, h), ref in zip(heads, refs):
        g = [t[b:b + 1, h:h + 1] for t in runs[0]]
        say(h, check_grads(g, ref, f"{w.name} head {h}"))
    for t in runs[0]:
        assert torch.isfinite(t.float()).all()


def test_non_causal_long_whole_head():
    """Non-causal B1 H4 S4096 d64: one whole head against the oracle (every
    key tile of every slab in play), the rest against fa_bwd."""
    say("bwd_ds non-causal S4096 d64")
    q, k, v, do = make_inputs(1, 4, 4096, 4096, 64, seed=123, with_dout=True)
    got, split = both(q, k, v, do, False)
    agree_with_split(got, split, "non-causal S4096 d64")
    (ref,) = oracle_backward_heads(q, k, v, do, 1 / 8.0, False, [(0, 2)])
    say(check_grads([t[:, 2:3] for t in got], ref, "non-causal S4096 d64 head 2"))


@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_phases_separately_equal_one_call(d, causal):
    """fa_bwd_ds_phase(PREPARE), then DKDV, then DQ writes the same bits as
    one fa_bwd_ds call; PREPARE touches no output, DKDV only dK and dV."""
    say(f"bwd_ds phases d={d} causal={causal}")
    q, k, v, do = (t.to(DEV) for t in make_inputs(1, 3, 333, 333, d, seed=60 + d, with_dout=True))
    o, lse = fa.forward(q, k, v, causal=causal)
    ref = fa.backward_ds(q, k, v, o, lse, do, causal=causal)
    nbytes = fa.fa_bwd_ds_workspace_bytes(1, 3, 333, 333, d, causal, False)
    ws = torch.full((nbytes,), 0x55, dtype=torch.uint8, device=DEV)
    outs = [torch.full_like(q, 7.0) for _ in range(3)]
    fa.fa_bwd_ds_phase(fa.FA_BWD_PREPARE, q, k, v, o, lse, do, *outs, ws, causal=causal)
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in outs), "PREPARE wrote an output"
    fa.fa_bwd_ds_phase(fa.FA_BWD_DKDV, q, k, v, o, lse, do, *outs, ws, causal=causal)
    torch.cuda.synchronize()
    assert bool((outs[0] == 7.0).all()), "DKDV wrote dQ"
    assert torch.equal(outs[1], ref[1]) and torch.equal(outs[2], ref[2])
    fa.fa_bwd_ds_phase(fa.FA_BWD_DQ, q, k, v, o, lse, do, *outs, ws, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)


def test_keys_past_sk_with_very_negative_scores():
    """Non-causal, Sk = 200 (the last 128-key block has 56 keys past Sk, read
    as zero rows), every score about -141 (LSE about -136): a key past Sk
    would have P = exp(0 - LSE) = inf.  Its dS must not reach dQ (inf times
    its zero K row is NaN): every gradient finite (on a NaN-filled
    workspace), dK and dV equal to the split form's, dQ equal to it to
    rounding, all within the gradient tolerance of the oracle.  (dQ is a
    cancellation of K's large common component here, about 2e-3, so its
    error relative to its own size is a few percent in both forms.)"""
    say("bwd_ds keys past Sk, scores about -141")
    B, H, Sq, Sk, d = 1, 2, 130, 200, 128
    g = torch.Generator().manual_seed(7)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = (40.0 * u + 0.3 * torch.randn(B, H, Sq, d, generator=g)).to(torch.bfloat16)
    k = (-40.0 * u + 0.3 * torch.randn(B, H, Sk, d, generator=g)).to(torch.bfloat16)
    v = (0.1 * torch.randn(B, H, Sk, d, generator=g)).to(torch.bfloat16)
    do = (0.1 * torch.randn(B, H, Sq, d, generator=g)).to(torch.bfloat16)
    got, split = both(q, k, v, do, False, fill=0xFF)
    for t in got:
        assert torch.isfinite(t.float()).all()
    agree_with_split(got, split, "keys past Sk")
    ref = attention_backward(q, k, v, do, 1 / math.sqrt(d), False)
    say(check_grads(got, ref, "keys past Sk"))


def test_largest_slice_sampled():
    """Causal B1 H1 Sq = Sk = 32640, d = 64: one (b, h) slice of dS is just
    under 2^31 bytes, the largest fa_bwd_ds accepts (32-bit offsets at their
    limit).  dK and dV must equal the split form's bit for bit; dQ rows
    (each depends on its own row only) are checked against the oracle on
    sampled rows, including the first and last."""
    S, d = 32640, 64
    say(f"bwd_ds largest slice S={S} d={d}")
    assert fa.fa_bwd_ds_workspace_bytes(1, 1, S, S, d, True, False) > 0
    assert fa.fa_bwd_ds_workspace_bytes(1, 1, S + 1, S + 1, d, True, False) == 0
    q, k, v, do = make_inputs(1, 1, S, S, d, seed=171, with_dout=True)
    got, split = both(q, k, v, do, True)
    assert torch.equal(got[1], split[1]) and torch.equal(got[2], split[2])
    for t in got:
        assert torch.isfinite(t.float()).all()
    rng = np.random.default_rng(171)
    rows = sorted(set(rng.choice(S, size=12, replace=False).tolist()) | {0, 1, 127, 128, S - 1})
    scale = 1 / math.sqrt(d)
    worst = 0.0
    for i in rows:
        sl = lambda t, n: t[:, :, :n].double().numpy()                      # noqa: E731
        qi = lambda t: t[:, :, i:i + 1].double().numpy()                     # noqa: E731
        ref = attention_backward(qi(q), sl(k, i + 1), sl(v, i + 1), qi(do), scale, False)
        err = float(np.abs(got[0][:, :, i:i + 1].double().numpy() - ref[0]).max())
        worst = max(worst, err)
        assert err <= 2e-2, (i, err)
    say(f"{len(rows)} sampled dQ rows, worst {worst:.3g}")
