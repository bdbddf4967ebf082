"""The C-ABI library loads on a CPU-only host, exports every symbol that
include/fa.h declares, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import exact_attention_50_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_exp2_probe", "fa_status_str",
            "fa_fwd_realised_emu_frac", "fa_fwd_fp8"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(5):
        assert fa.fa_status_str(s) and fa.fa_status_str(s) != "unknown status"
    assert fa.fa_status_str(99) == "unknown status"


FAKE = 1 << 20   # aligned, never dereferenced: validation fails first


def _fwd(L, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Sq=16, Sk=16, d=64, causal=0, scale=0.125,
         tau=8.0, emu=0.0):
    vp = ctypes.c_void_p
    return L.fa_fwd(vp(q), vp(k), vp(v), vp(o), vp(lse), B, H, Sq, Sk, d, causal, scale, tau, emu, vp(0))


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_INVALID), (dict(lse=0), fa.FA_ERR_INVALID), (dict(o=FAKE + 2), fa.FA_ERR_INVALID),
    (dict(B=0), fa.FA_ERR_INVALID), (dict(Sk=-1), fa.FA_ERR_INVALID), (dict(scale=0.0), fa.FA_ERR_INVALID),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID), (dict(tau=-1.0), fa.FA_ERR_INVALID),
    (dict(tau=65.0), fa.FA_ERR_INVALID), (dict(emu=1.5), fa.FA_ERR_INVALID), (dict(causal=2), fa.FA_ERR_INVALID),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(causal=1, Sq=16, Sk=32), fa.FA_ERR_UNSUPPORTED),
    # one head past 31-bit byte offsets: (8M + 1024) rows x 128 dims x 2 bytes
    (dict(d=128, Sq=16, Sk=(1 << 23)), fa.FA_ERR_UNSUPPORTED),
    (dict(d=128, Sq=16, Sk=(1 << 31) // 256 - 1024), fa.FA_ERR_UNSUPPORTED),   # one past the largest head
])
def test_fwd_rejects_before_any_launch(L, kw, status):
    assert _fwd(L, **kw) == status


def _fwd8(L, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, qs=1.0, ks=1.0, vs=1.0, hd=0, B=1, H=1, Sq=16, Sk=16,
          d=128, causal=0, scale=0.125, tau=8.0):
    vp = ctypes.c_void_p
    return L.fa_fwd_fp8(vp(q), vp(k), vp(v), qs, ks, vs, vp(hd), vp(o), vp(lse), B, H, Sq, Sk, d, causal, scale,
                        tau, vp(0))


@pytest.mark.parametrize("kw,status", [
    (dict(v=0), fa.FA_ERR_INVALID), (dict(k=FAKE + 8), fa.FA_ERR_INVALID), (dict(H=0), fa.FA_ERR_INVALID),
    (dict(qs=0.0), fa.FA_ERR_INVALID), (dict(vs=-1.0), fa.FA_ERR_INVALID), (dict(ks=float("inf")), fa.FA_ERR_INVALID),
    (dict(tau=8.5), fa.FA_ERR_INVALID), (dict(scale=-1.0), fa.FA_ERR_INVALID), (dict(causal=3), fa.FA_ERR_INVALID),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(causal=1, Sq=16, Sk=8), fa.FA_ERR_UNSUPPORTED),
    (dict(hd=FAKE + 2), fa.FA_ERR_INVALID), (dict(hd=FAKE + 4, d=32), fa.FA_ERR_UNSUPPORTED),
    # each factor valid on its own, their product (folded into one float
    # score factor) overflows or underflows
    (dict(qs=1e30, ks=1e30), fa.FA_ERR_INVALID), (dict(qs=1e-30, ks=1e-20), fa.FA_ERR_INVALID),
])
def test_fwd_fp8_rejects_before_any_launch(L, kw, status):
    assert _fwd8(L, **kw) == status


def test_partial_and_merge_validation(L):
    vp = ctypes.c_void_p

    def part(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Sq=16, Sk=32, d=64, q_off=0, kb=0, ke=32,
                 causal=0, scale=0.125, tau=8.0, emu=0.0)
        a.update(kw)
        return L.fa_fwd_partial(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), vp(a["lse"]), a["B"], a["H"],
                                a["Sq"], a["Sk"], a["d"], a["q_off"], a["kb"], a["ke"], a["causal"], a["scale"],
                                a["tau"], a["emu"], vp(0))
    assert part(kb=5, ke=5) == fa.FA_ERR_INVALID        # empty range
    assert part(kb=-1) == fa.FA_ERR_INVALID
    assert part(ke=33) == fa.FA_ERR_INVALID             # past Sk
    assert part(q_off=-3) == fa.FA_ERR_INVALID
    assert part(o=0) == fa.FA_ERR_INVALID
    assert part(causal=2) == fa.FA_ERR_INVALID
    assert part(d=80) == fa.FA_ERR_UNSUPPORTED
    # causal bounds are formed as q_offset + row block end + one tile in
    # 32-bit ints: offsets that would overflow them are refused
    assert part(q_off=(1 << 31) - 16 - 512) == fa.FA_ERR_UNSUPPORTED
    assert part(q_off=(1 << 31) - 16 - 1, causal=1) == fa.FA_ERR_UNSUPPORTED

    def merge(**kw):
        a = dict(op=FAKE, lp=FAKE, n=2, B=1, H=1, Sq=16, d=64, o=FAKE, lse=FAKE)
        a.update(kw)
        return L.fa_merge(vp(a["op"]), vp(a["lp"]), a["n"], a["B"], a["H"], a["Sq"], a["d"], vp(a["o"]),
                          vp(a["lse"]), vp(0))
    assert merge(n=0) == fa.FA_ERR_INVALID
    assert merge(op=0) == fa.FA_ERR_INVALID
    assert merge(o=FAKE + 4) == fa.FA_ERR_INVALID
    assert merge(Sq=0) == fa.FA_ERR_INVALID
    assert merge(d=96) == fa.FA_ERR_UNSUPPORTED


def test_bwd_validation_and_workspace(L):
    vp = ctypes.c_void_p
    ws = fa.fa_bwd_workspace_bytes(1, 2, 100, 100, 64, True, True)
    assert ws >= 2 * 100 * 4 and ws % 256 == 0
    assert fa.fa_bwd_workspace_bytes(0, 2, 100, 100, 64, True, True) == 0
    assert fa.fa_bwd_workspace_bytes(1, 2, 100, 100, 80, True, True) == 0
    args = [vp(FAKE)] * 9 + [1, 2, 100, 100, 64, 1, 0.125, 1, vp(FAKE)]
    # workspace too small
    assert L.fa_bwd(*args, ws - 1, vp(0)) == fa.FA_ERR_INVALID
    # null output
    bad = list(args)
    bad[7] = vp(0)
    assert L.fa_bwd(*bad, ws, vp(0)) == fa.FA_ERR_INVALID
    # deterministic flag out of range
    bad = list(args)
    bad[16] = 3
    assert L.fa_bwd(*bad, ws, vp(0)) == fa.FA_ERR_INVALID


def test_bwd_ds_validation_and_workspace(L):
    """The five-product backward's workspace is the row terms plus one bf16
    dS^T slab of (Sk rounded up to 128) x 128 per (b, h, block of 128 query
    rows); it validates like fa_bwd and refuses slices whose dS reaches
    2^31 bytes."""
    vp = ctypes.c_void_p
    rows = fa.fa_bwd_workspace_bytes(2, 3, 300, 200, 64, False, False)
    ws = fa.fa_bwd_ds_workspace_bytes(2, 3, 300, 200, 64, False, False)
    assert ws == rows + 2 * 3 * 3 * 256 * 128 * 2
    assert fa.fa_bwd_ds_workspace_bytes(2, 3, 300, 200, 128, True, True) == ws
    assert fa.fa_bwd_ds_workspace_bytes(1, 16, 4096, 4096, 128, True, False) == \
        fa.fa_bwd_workspace_bytes(1, 16, 4096, 4096, 128, True, False) + 16 * 4096 * 4096 * 2
    assert fa.fa_bwd_ds_workspace_bytes(1, 1, 32640, 32640, 128, True, False) > 0
    assert fa.fa_bwd_ds_workspace_bytes(1, 1, 32641, 32641, 128, True, False) == 0
    assert fa.fa_bwd_ds_workspace_bytes(1, 2, 100, 100, 80, True, True) == 0
    assert fa.fa_bwd_ds_workspace_bytes(0, 2, 100, 100, 64, True, True) == 0
    ws = fa.fa_bwd_ds_workspace_bytes(1, 2, 100, 100, 64, True, False)
    args = [vp(FAKE)] * 9 + [1, 2, 100, 100, 64, 1, 0.125, 0, vp(FAKE)]
    assert L.fa_bwd_ds(*args, ws - 1, vp(0)) == fa.FA_ERR_INVALID
    for i in (0, 5, 8):
        bad = list(args)
        bad[i] = vp(0)
        assert L.fa_bwd_ds(*bad, ws, vp(0)) == fa.FA_ERR_INVALID
    bad = list(args)
    bad[17] = vp(0)                                # null workspace
    assert L.fa_bwd_ds(*bad, ws, vp(0)) == fa.FA_ERR_INVALID
    bad = list(args)
    bad[16] = 2
    assert L.fa_bwd_ds(*bad, ws, vp(0)) == fa.FA_ERR_INVALID
    bad = list(args)
    bad[13] = 96
    assert L.fa_bwd_ds(*bad, ws, vp(0)) == fa.FA_ERR_UNSUPPORTED
    bad = list(args)
    bad[12] = 64                                   # causal with Sq != Sk
    assert L.fa_bwd_ds(*bad, ws, vp(0)) == fa.FA_ERR_UNSUPPORTED
    big = [vp(FAKE)] * 9 + [1, 1, 32641, 32641, 128, 1, 0.125, 0, vp(FAKE)]
    assert L.fa_bwd_ds(*big, 1 << 40, vp(0)) == fa.FA_ERR_UNSUPPORTED
    # the phase entry point: an empty or unknown mask is refused, the rest
    # validated as above
    for ph in (0, 8, -1):
        assert L.fa_bwd_ds_phase(ph, *args, ws, vp(0)) == fa.FA_ERR_INVALID
    assert L.fa_bwd_ds_phase(fa.FA_BWD_DQ, *args, ws - 1, vp(0)) == fa.FA_ERR_INVALID
    assert L.fa_bwd_ds_phase(fa.FA_BWD_ALL, *big, 1 << 40, vp(0)) == fa.FA_ERR_UNSUPPORTED


def test_realised_emu_share(L):
    assert fa.fa_fwd_realised_emu_frac(128, 0.0) == 0.0
    assert abs(fa.fa_fwd_realised_emu_frac(128, 0.10) - 0.10) < 0.02
    assert fa.fa_fwd_realised_emu_frac(64, 0.25) == 0.25
    assert fa.fa_fwd_realised_emu_frac(128, 1.0) == 1.0
    assert fa.fa_fwd_realised_emu_frac(128, 2.0) < 0
    assert fa.fa_fwd_realised_emu_frac(40, 0.1) < 0


def test_exp2_probe_empty_is_noop(L):
    vp = ctypes.c_void_p
    assert L.fa_exp2_probe(vp(0), vp(0), vp(0), 0, vp(0)) == fa.FA_OK
    assert L.fa_exp2_probe(vp(0), vp(0), vp(0), -1, vp(0)) == fa.FA_ERR_INVALID
    assert L.fa_exp2_probe(vp(0), vp(FAKE), vp(FAKE), 5, vp(0)) == fa.FA_ERR_INVALID


def test_bwd_phase_mask_validation(L):
    vp = ctypes.c_void_p
    ws = fa.fa_bwd_workspace_bytes(1, 2, 100, 100, 64, True, True)
    args = [vp(FAKE)] * 9 + [1, 2, 100, 100, 64, 1, 0.125, 1, vp(FAKE), ws, vp(0)]
    for bad_mask in (0, 8, -1):
        assert L.fa_bwd_phase(bad_mask, *args) == fa.FA_ERR_INVALID
    bad = list(args)
    bad[13] = 96   # d
    assert L.fa_bwd_phase(fa.FA_BWD_DQ, *bad) == fa.FA_ERR_UNSUPPORTED


def test_bwd_noalloc_validation(L):
    """The allocation-free backward validates like fa_bwd and refuses requests
    beyond its fixed scratch (B * H * Sq > FA_NOALLOC_MAX_ROWS) before any
    HIP call."""
    vp = ctypes.c_void_p

    def call(B=1, H=2, Sq=100, Sk=100, d=64, causal=1, scale=0.125, det=1, null=None, mis=None):
        ptrs = [FAKE] * 9
        if null is not None:
            ptrs[null] = 0
        if mis is not None:
            ptrs[mis] = FAKE + 8
        return L.fa_bwd_noalloc(*[vp(p) for p in ptrs], B, H, Sq, Sk, d, causal, scale, det, vp(0))
    assert call(null=0) == fa.FA_ERR_INVALID
    assert call(null=8) == fa.FA_ERR_INVALID
    assert call(mis=4) == fa.FA_ERR_INVALID
    assert call(scale=0.0) == fa.FA_ERR_INVALID
    assert call(det=2) == fa.FA_ERR_INVALID
    assert call(d=96) == fa.FA_ERR_UNSUPPORTED
    assert call(Sk=50) == fa.FA_ERR_UNSUPPORTED          # causal, Sq != Sk
    limit = fa.FA_NOALLOC_MAX_ROWS
    assert call(B=2, H=16, Sq=limit // 32 + 1, Sk=limit // 32 + 1) == fa.FA_ERR_SCRATCH
    assert call(B=1, H=1, Sq=limit + 1, Sk=limit + 1, causal=0) == fa.FA_ERR_SCRATCH
    assert "scratch" in fa.fa_status_str(fa.FA_ERR_SCRATCH)


def test_fwd_mxfp4_rejects_before_any_launch(L):
    vp = ctypes.c_void_p

    def call(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, v=FAKE, vd=1.0, o=FAKE, lse=FAKE, B=1, H=1, Sq=16, Sk=16, d=128,
             causal=0, scale=0.125, tau=8.0):
        return L.fa_fwd_mxfp4(vp(q), vp(qs), vp(k), vp(ks), vp(v), vd, vp(o), vp(lse), B, H, Sq, Sk, d, causal,
                              scale, tau, vp(0))
    assert call(qs=0) == fa.FA_ERR_INVALID
    assert call(k=0) == fa.FA_ERR_INVALID
    assert call(ks=FAKE + 2) == fa.FA_ERR_INVALID          # scales must be 4-byte aligned
    assert call(q=FAKE + 8) == fa.FA_ERR_INVALID
    assert call(vd=0.0) == fa.FA_ERR_INVALID
    assert call(vd=float("inf")) == fa.FA_ERR_INVALID
    assert call(tau=9.0) == fa.FA_ERR_INVALID
    assert call(scale=-1.0) == fa.FA_ERR_INVALID
    assert call(scale=1e-40) == fa.FA_ERR_INVALID           # scale * log2(e) below the normal range
    assert call(causal=2) == fa.FA_ERR_INVALID
    assert call(d=64) == fa.FA_ERR_UNSUPPORTED
    assert call(causal=1, Sk=32) == fa.FA_ERR_UNSUPPORTED


def test_fwd_fp8_blocks_rejects_before_any_launch(L):
    vp = ctypes.c_void_p

    def call(q=FAKE, k=FAKE, v=FAKE, qf=FAKE, kf=FAKE, vf=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Sq=16, Sk=16, d=128,
             causal=0, scale=0.125, tau=8.0):
        return L.fa_fwd_fp8_blocks(vp(q), vp(k), vp(v), vp(qf), vp(kf), vp(vf), vp(o), vp(lse), B, H, Sq, Sk, d,
                                   causal, scale, tau, vp(0))
    assert call(vf=0) == fa.FA_ERR_INVALID
    assert call(qf=FAKE + 2) == fa.FA_ERR_INVALID          # factors must be 4-byte aligned
    assert call(v=FAKE + 8) == fa.FA_ERR_INVALID
    assert call(lse=0) == fa.FA_ERR_INVALID
    assert call(tau=8.5) == fa.FA_ERR_INVALID
    assert call(scale=float("nan")) == fa.FA_ERR_INVALID
    assert call(scale=1e-40) == fa.FA_ERR_INVALID
    assert call(B=0) == fa.FA_ERR_INVALID
    assert call(causal=3) == fa.FA_ERR_INVALID
    assert call(d=96) == fa.FA_ERR_UNSUPPORTED
    assert call(causal=1, Sk=48) == fa.FA_ERR_UNSUPPORTED
