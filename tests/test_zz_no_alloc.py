"""fa_bwd_noalloc (the backward for callers that cannot allocate: its
workspace is the library's fixed device scratch) against fa_bwd on the same
inputs, through the C ABI: bit-identical gradients (the same kernels), which
also meet the oracle's gradient tolerance; two calls in a row, the second on
a smaller input, so a stale scratch from the first call would show."""
import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_50_amd as fa
from parity import check_grads, oracle_backward_heads
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def grads_both_ways(B, H, S, d, causal, seed):
    q, k, v, do = make_inputs(B, H, S, S, d, seed=seed, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal)
    ref = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, deterministic=True)
    got = [torch.empty_like(t) for t in (qd, kd, vd)]
    fa.fa_bwd_noalloc(qd, kd, vd, o, lse, dod, *got, causal=causal, deterministic=True)
    torch.cuda.synchronize()
    return (q, k, v, do), [t.cpu() for t in ref], [t.cpu() for t in got]


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_noalloc_matches_fa_bwd_twice_second_smaller(d, causal):
    for B, H, S, seed in ((2, 8, 1000, 81), (1, 3, 300, 82)):
        say(f"noalloc bwd d={d} causal={causal} B{B} H{H} S{S}")
        inputs, ref, got = grads_both_ways(B, H, S, d, causal, seed)
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(r, g), (name, B, H, S)
        q, k, v, do = inputs
        oracle = oracle_backward_heads(q, k, v, do, 1 / math.sqrt(d), causal, [(0, 0), (B - 1, H - 1)])
        for (b, h), r in zip([(0, 0), (B - 1, H - 1)], oracle):
            say(check_grads([t[b:b + 1, h:h + 1] for t in got], r, f"noalloc ({b},{h})"))


def test_noalloc_refuses_beyond_scratch():
    """B * H * Sq above FA_NOALLOC_MAX_ROWS is refused before any launch."""
    S = fa.FA_NOALLOC_MAX_ROWS // 16 + 64
    q = torch.zeros((1, 16, S, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((1, 16, S), dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, lse, q, q, q, q, causal=True)
    assert e.value.status == fa.FA_ERR_SCRATCH
