"""GPU parity of fa_bwd against the CPU oracle (called through the C ABI).

The GPU backward consumes the GPU forward's O and LSE (as a training step
does); the oracle recomputes everything in float64, so the forward's
rounding is part of the error budget (max |err| <= 2e-2).
"""
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


def run_bwd(q, k, v, do, causal, deterministic, reps=1):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal)
    outs = []
    for _ in range(reps):
        dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, deterministic=deterministic)
        torch.cuda.synchronize()
        outs.append((dq.cpu(), dk.cpu(), dv.cpu()))
    return outs


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq,Sk,causal", [(1, 1, False), (17, 17, True), (64, 200, False), (128, 128, True),
                                          (257, 257, True), (200, 333, False), (384, 384, True)])
@pytest.mark.parametrize("det", [False, True])
def test_small_shapes_every_element(d, Sq, Sk, causal, det):
    say(f"bwd small d={d} Sq={Sq} Sk={Sk} causal={causal} det={det}")
    q, k, v, do = make_inputs(2, 2, Sq, Sk, d, seed=Sq * 31 + Sk + d, with_dout=True)
    (got,) = run_bwd(q, k, v, do, causal, det)
    ref = attention_backward(q, k, v, do, 1 / math.sqrt(d), causal)
    check_grads(got, ref, f"d{d} {Sq}x{Sk} c{causal} det{det}")


@pytest.mark.parametrize("det", [True, False])
def test_config5_sampled_heads(det):
    w = WORKLOADS[5]
    say(f"bwd {w.name} det={det}")
    q, k, v, do = workload_inputs(w)
    (got,) = run_bwd(q, k, v, do, w.causal, det)
    heads = [(0, 0), (0, 13)]
    refs = oracle_backward_heads(q, k, v, do, w.scale, w.causal, heads)
    for (b, h), ref in zip(heads, refs):
        g = [t[b:b + 1, h:h + 1] for t in got]
        st = check_grads(g, ref, f"{w.name} head {h}")
        say(h, st)
    for t in got:
        assert torch.isfinite(t.float()).all()


def test_config5_deterministic_bit_identical_three_runs():
    w = WORKLOADS[5]
    say(f"bwd {w.name} deterministic x3")
    q, k, v, do = workload_inputs(w)
    runs = run_bwd(q, k, v, do, w.causal, True, reps=3)
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


def test_deterministic_non_causal_bit_identical():
    say("bwd non-causal deterministic x3")
    q, k, v, do = make_inputs(2, 4, 1024, 1024, 64, seed=21, with_dout=True)
    runs = run_bwd(q, k, v, do, False, True, reps=3)
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


def test_workspace_reuse_and_dirty_workspace():
    """The workspace contents on entry do not matter."""
    say("bwd dirty workspace")
    q, k, v, do = (t.to(DEV) for t in make_inputs(1, 2, 300, 300, 128, seed=5, with_dout=True))
    o, lse = fa.forward(q, k, v, causal=True)
    nbytes = fa.fa_bwd_workspace_bytes(1, 2, 300, 300, 128, True, True)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)
    a = fa.backward(q, k, v, o, lse, do, causal=True, deterministic=True, workspace=ws)
    b = fa.backward(q, k, v, o, lse, do, causal=True, deterministic=True, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True)])
def test_phases_separately_equal_fa_bwd(d, causal):
    """fa_bwd_phase(PREPARE), then DQ, then DKDV (also DKDV before DQ) writes
    the same bits as one fa_bwd call, which forms the row terms inside the dQ
    kernel (workspace included); DQ and DKDV each touch only their outputs."""
    say(f"bwd phases d={d} causal={causal}")
    q, k, v, do = (t.to(DEV) for t in make_inputs(1, 3, 333, 333, d, seed=40 + d, with_dout=True))
    o, lse = fa.forward(q, k, v, causal=causal)
    ref = fa.backward(q, k, v, o, lse, do, causal=causal)
    nbytes = fa.fa_bwd_workspace_bytes(1, 3, 333, 333, d, causal, False)
    ws_fused = torch.full((nbytes,), 0x55, dtype=torch.uint8, device=DEV)
    fused = [torch.empty_like(q) for _ in range(3)]
    fa.fa_bwd(q, k, v, o, lse, do, *fused, ws_fused, causal=causal)
    ws_prep = torch.full((nbytes,), 0x55, dtype=torch.uint8, device=DEV)
    fa.fa_bwd_phase(fa.FA_BWD_PREPARE, q, k, v, o, lse, do, *fused, ws_prep, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(ws_fused, ws_prep), "row terms of the fused dQ kernel differ from the prep kernel's"
    for a, b in zip(fused, ref):
        assert torch.equal(a, b)
    for order in ((fa.FA_BWD_DQ, fa.FA_BWD_DKDV), (fa.FA_BWD_DKDV, fa.FA_BWD_DQ)):
        ws = torch.full((nbytes,), 0x55, dtype=torch.uint8, device=DEV)
        outs = [torch.full_like(q, 7.0) for _ in range(3)]
        fa.fa_bwd_phase(fa.FA_BWD_PREPARE, q, k, v, o, lse, do, *outs, ws, causal=causal)
        torch.cuda.synchronize()
        assert all(bool((t == 7.0).all()) for t in outs), "PREPARE wrote an output"
        fa.fa_bwd_phase(order[0], q, k, v, o, lse, do, *outs, ws, causal=causal)
        torch.cuda.synchronize()
        first = (0,) if order[0] == fa.FA_BWD_DQ else (1, 2)
        for i in range(3):
            if i in first:
                assert torch.equal(outs[i], ref[i])
            else:
                assert bool((outs[i] == 7.0).all())
        fa.fa_bwd_phase(order[1], q, k, v, o, lse, do, *outs, ws, causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)
