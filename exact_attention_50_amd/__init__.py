"""Python binding of libfa, the gfx950 fused exact-attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa.h.  PyTorch provides device
memory and the current stream.  The functions named like the C entry points
(``fa_fwd``, ``fa_bwd``, ...) take torch tensors and pass their device
pointers through; ``forward`` / ``backward`` additionally allocate outputs.

There is no fallback: if libfa.so is missing or a call fails, an exception is
raised.
"""
import ctypes
import math
import os

__all__ = [
    "FAError", "lib", "LIB_PATH", "fa_status_str",
    "fa_fwd", "fa_fwd_realised_emu_frac", "fa_fwd_rescale_count", "fa_fwd_partial", "fa_merge", "fa_exp2_probe",
    "fa_fwd_fp8", "fa_fwd_fp8_blocks", "fa_fwd_mxfp4",
    "fa_bwd", "fa_bwd_phase", "fa_bwd_workspace_bytes", "fa_bwd_noalloc",
    "fa_bwd_ds", "fa_bwd_ds_phase", "fa_bwd_ds_workspace_bytes",
    "forward", "forward_partial", "merge", "forward_fp8", "forward_fp8_blocks", "forward_mxfp4",
    "backward", "backward_ds",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_SCRATCH = 0, 1, 2, 3, 4
FA_NOALLOC_MAX_ROWS = 1 << 21
FA_BWD_PREPARE, FA_BWD_DQ, FA_BWD_DKDV, FA_BWD_ALL = 1, 2, 4, 7

_lib = None


class FAError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {fa_status_str(status)} (status {status})")
        self.status = status


def lib():
    """Load libfa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "or python -m exact_attention_50_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, f, vp]
    L.fa_fwd.restype = i
    L.fa_fwd_rescale_count.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, vp, vp]
    L.fa_fwd_rescale_count.restype = i
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, vp, i, i, i, i, i, i, f, f, vp]
    L.fa_fwd_fp8.restype = i
    L.fa_fwd_fp8_blocks.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, vp]
    L.fa_fwd_fp8_blocks.restype = i
    L.fa_fwd_mxfp4.argtypes = [vp, vp, vp, vp, vp, f, vp, vp, i, i, i, i, i, i, f, f, vp]
    L.fa_fwd_mxfp4.restype = i
    L.fa_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, f, f, vp]
    L.fa_fwd_partial.restype = i
    L.fa_merge.argtypes = [vp, vp, i, i, i, i, i, vp, vp, vp]
    L.fa_merge.restype = i
    L.fa_fwd_realised_emu_frac.argtypes = [i, f]
    L.fa_fwd_realised_emu_frac.restype = f
    L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.fa_bwd_workspace_bytes.restype = sz
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.fa_bwd.restype = i
    L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.fa_bwd_noalloc.restype = i
    L.fa_bwd_phase.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.fa_bwd_phase.restype = i
    L.fa_bwd_ds_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.fa_bwd_ds_workspace_bytes.restype = sz
    L.fa_bwd_ds.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.fa_bwd_ds.restype = i
    L.fa_bwd_ds_phase.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.fa_bwd_ds_phase.restype = i
    L.fa_exp2_probe.argtypes = [vp, vp, vp, ctypes.c_longlong, vp]
    L.fa_exp2_probe.restype = i
    L.fa_status_str.argtypes = [i]
    L.fa_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def fa_status_str(status):
    return lib().fa_status_str(int(status)).decode()


def fa_fwd_realised_emu_frac(d, emu_frac):
    return float(lib().fa_fwd_realised_emu_frac(int(d), float(emu_frac)))


def fa_bwd_workspace_bytes(B, H, Sq, Sk, d, causal, deterministic):
    return int(lib().fa_bwd_workspace_bytes(B, H, Sq, Sk, d, int(bool(causal)), int(bool(deterministic))))


# ------------------------------------------------------------------ helpers
def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_bf16(name, t, shape):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected a contiguous bf16 CUDA tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device} contiguous={t.is_contiguous()}")


def _check_f32(name, t, shape):
    import torch
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected a contiguous float32 CUDA tensor of shape {tuple(shape)}")


# --------------------------------------------------------- C-named wrappers
def fa_fwd(q, k, v, o, lse, causal=False, scale=None, tau=8.0, emu_frac=0.0):
    """Enqueue the forward on the current stream; fills o and lse in place."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    _check_bf16("q", q, (B, H, Sq, d))
    _check_bf16("k", k, (B, H, Sk, d))
    _check_bf16("v", v, (B, H, Sk, d))
    _check_bf16("o", o, (B, H, Sq, d))
    _check_f32("lse", lse, (B, H, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq, Sk, d, int(bool(causal)),
                      float(scale), float(tau), float(emu_frac), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")


FA_RESCALE_SLOT_ROWS = 32


def fa_fwd_rescale_count(q, k, v, o, lse, events, causal=False, scale=None, tau=8.0):
    """The instrumented forward (hardware exponentials): fills o and lse as
    fa_fwd does and adds, per (b, h) and 32-row wavefront slot, the
    wavefront-level corrections taken after each wavefront's first key tile
    to events (int32 CUDA [B, H, ceil(Sq / 32)])."""
    import torch
    B, H, Sq, d = q.shape
    slots = -(-Sq // FA_RESCALE_SLOT_ROWS)
    Sk = k.shape[2]
    _check_bf16("q", q, (B, H, Sq, d))
    _check_bf16("k", k, (B, H, Sk, d))
    _check_bf16("v", v, (B, H, Sk, d))
    _check_bf16("o", o, (B, H, Sq, d))
    _check_f32("lse", lse, (B, H, Sq))
    if events.dtype != torch.int32 or not events.is_cuda or not events.is_contiguous() or \
            tuple(events.shape) != (B, H, slots):
        raise ValueError(f"events: expected a contiguous int32 CUDA tensor of shape {(B, H, slots)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_rescale_count(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq, Sk, d,
                                    int(bool(causal)), float(scale), float(tau), _ptr(events), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_rescale_count")


def _check_e4m3(name, t, shape):
    import torch
    if (t.dtype not in (torch.uint8, torch.float8_e4m3fn) or not t.is_cuda or not t.is_contiguous()
            or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name}: expected a contiguous e4m3 (float8_e4m3fn or uint8) CUDA tensor of shape "
                         f"{tuple(shape)}, got {t.dtype} {tuple(t.shape)} on {t.device}")


def fa_fwd_fp8(q8, k8, v8, o, lse, q_descale=1.0, k_descale=1.0, v_descale=1.0, causal=False, scale=None, tau=8.0,
               head_descales=None):
    """Enqueue the e4m3 forward on the current stream; fills the bf16 o and
    the float32 lse in place.  q8, k8, v8 hold e4m3 bytes (float8_e4m3fn or
    uint8); the attention is computed on q_descale * q8, k_descale * k8,
    v_descale * v8, each factor times the (batch, head) slice's factor in
    head_descales (None, or a float32 CUDA tensor [3, B, H]: Q, K, V)."""
    B, H, Sq, d = q8.shape
    Sk = k8.shape[2]
    _check_e4m3("q8", q8, (B, H, Sq, d))
    _check_e4m3("k8", k8, (B, H, Sk, d))
    _check_e4m3("v8", v8, (B, H, Sk, d))
    _check_bf16("o", o, (B, H, Sq, d))
    _check_f32("lse", lse, (B, H, Sq))
    if head_descales is not None:
        _check_f32("head_descales", head_descales, (3, B, H))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), float(q_descale), float(k_descale), float(v_descale),
                          None if head_descales is None else _ptr(head_descales),
                          _ptr(o), _ptr(lse), B, H, Sq, Sk, d, int(bool(causal)), float(scale), float(tau),
                          _stream(q8))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")


FA_FP8_SCALE_BLOCK = 128


def fa_fwd_fp8_blocks(q8, k8, v8, q_factors, k_factors, v_factors, o, lse, causal=False, scale=None, tau=8.0):
    """Enqueue the e4m3 forward with per-block factors on the current
    stream; fills the bf16 o and the float32 lse in place.  q8, k8, v8 hold
    e4m3 bytes; q_factors is a float32 CUDA tensor [B, H, ceil(Sq / 128)],
    k_factors and v_factors [B, H, ceil(Sk / 128)]: the factor of each block
    of 128 consecutive rows."""
    B, H, Sq, d = q8.shape
    Sk = k8.shape[2]
    nq, nk = -(-Sq // FA_FP8_SCALE_BLOCK), -(-Sk // FA_FP8_SCALE_BLOCK)
    _check_e4m3("q8", q8, (B, H, Sq, d))
    _check_e4m3("k8", k8, (B, H, Sk, d))
    _check_e4m3("v8", v8, (B, H, Sk, d))
    _check_f32("q_factors", q_factors, (B, H, nq))
    _check_f32("k_factors", k_factors, (B, H, nk))
    _check_f32("v_factors", v_factors, (B, H, nk))
    _check_bf16("o", o, (B, H, Sq, d))
    _check_f32("lse", lse, (B, H, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_fp8_blocks(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_factors), _ptr(k_factors), _ptr(v_factors),
                                 _ptr(o), _ptr(lse), B, H, Sq, Sk, d, int(bool(causal)), float(scale), float(tau),
                                 _stream(q8))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8_blocks")


def _check_u8(name, t, shape):
    import torch
    if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected a contiguous uint8 CUDA tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def fa_fwd_mxfp4(q4, q_scales, k4, k_scales, v8, o, lse, v_descale=1.0, causal=False, scale=None, tau=8.0):
    """Enqueue the MXFP4-Q/K, e4m3-V forward: q4 [B,H,Sq,d/2] and k4
    [B,H,Sk,d/2] packed E2M1 bytes, q_scales [B,H,Sq,d/32] and k_scales
    [B,H,Sk,d/32] E8M0 bytes, v8 e4m3 [B,H,Sk,d]; fills the bf16 o and
    float32 lse in place."""
    B, H, Sq, d2 = q4.shape
    d = 2 * d2
    Sk = k4.shape[2]
    _check_u8("q4", q4, (B, H, Sq, d2))
    _check_u8("k4", k4, (B, H, Sk, d2))
    _check_u8("q_scales", q_scales, (B, H, Sq, d // 32))
    _check_u8("k_scales", k_scales, (B, H, Sk, d // 32))
    _check_e4m3("v8", v8, (B, H, Sk, d))
    _check_bf16("o", o, (B, H, Sq, d))
    _check_f32("lse", lse, (B, H, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_mxfp4(_ptr(q4), _ptr(q_scales), _ptr(k4), _ptr(k_scales), _ptr(v8), float(v_descale),
                            _ptr(o), _ptr(lse), B, H, Sq, Sk, d, int(bool(causal)), float(scale), float(tau),
                            _stream(q4))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_mxfp4")


def forward_mxfp4(q4, q_scales, k4, k_scales, v8, v_descale=1.0, causal=False, scale=None, tau=8.0):
    """Returns (O bf16 [B,H,Sq,d], LSE float32 [B,H,Sq]) of the MXFP4 forward."""
    import torch
    B, H, Sq, d2 = q4.shape
    o = torch.empty((B, H, Sq, 2 * d2), dtype=torch.bfloat16, device=q4.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q4.device)
    fa_fwd_mxfp4(q4, q_scales, k4, k_scales, v8, o, lse, v_descale, causal=causal, scale=scale, tau=tau)
    return o, lse


def fa_fwd_partial(q, k, v, o_part, lse_part, q_offset, k_begin, k_end, causal=False, scale=None, tau=8.0,
                   emu_frac=0.0):
    """Enqueue the forward over keys k_begin..k_end-1; fills the float32
    o_part [B,H,Sq,d] and lse_part [B,H,Sq] in place."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    _check_bf16("q", q, (B, H, Sq, d))
    _check_bf16("k", k, (B, H, Sk, d))
    _check_bf16("v", v, (B, H, Sk, d))
    _check_f32("o_part", o_part, (B, H, Sq, d))
    _check_f32("lse_part", lse_part, (B, H, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, H, Sq, Sk, d,
                              int(q_offset), int(k_begin), int(k_end), int(bool(causal)), float(scale), float(tau),
                              float(emu_frac), _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_partial")


def fa_merge(o_parts, lse_parts, o, lse):
    """Enqueue the merge of n partial results: o_parts float32 [n,B,H,Sq,d],
    lse_parts float32 [n,B,H,Sq]; fills the bf16 o and float32 lse."""
    n, B, H, Sq, d = o_parts.shape
    _check_f32("o_parts", o_parts, (n, B, H, Sq, d))
    _check_f32("lse_parts", lse_parts, (n, B, H, Sq))
    _check_bf16("o", o, (B, H, Sq, d))
    _check_f32("lse", lse, (B, H, Sq))
    st = lib().fa_merge(_ptr(o_parts), _ptr(lse_parts), n, B, H, Sq, d, _ptr(o), _ptr(lse), _stream(o))
    if st != FA_OK:
        raise FAError(st, "fa_merge")


def fa_bwd_phase(phases, q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=False, scale=None,
                 deterministic=False):
    """Enqueue the backward kernels selected by the FA_BWD_* bit mask."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    for name, t, s in (("q", q, (B, H, Sq, d)), ("k", k, (B, H, Sk, d)), ("v", v, (B, H, Sk, d)),
                       ("o", o, (B, H, Sq, d)), ("dout", dout, (B, H, Sq, d)), ("dq", dq, (B, H, Sq, d)),
                       ("dk", dk, (B, H, Sk, d)), ("dv", dv, (B, H, Sk, d))):
        _check_bf16(name, t, s)
    _check_f32("lse", lse, (B, H, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fa_bwd_phase(int(phases), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                            _ptr(dk), _ptr(dv), B, H, Sq, Sk, d, int(bool(causal)), float(scale),
                            int(bool(deterministic)), _ptr(workspace), ws_bytes, _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_phase")


def fa_bwd_ds_workspace_bytes(B, H, Sq, Sk, d, causal, deterministic):
    return int(lib().fa_bwd_ds_workspace_bytes(B, H, Sq, Sk, d, int(bool(causal)), int(bool(deterministic))))


def _bwd_call(name, q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, scale, deterministic, phases=None):
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    for n, t, s in (("q", q, (B, H, Sq, d)), ("k", k, (B, H, Sk, d)), ("v", v, (B, H, Sk, d)),
                    ("o", o, (B, H, Sq, d)), ("dout", dout, (B, H, Sq, d)), ("dq", dq, (B, H, Sq, d)),
                    ("dk", dk, (B, H, Sk, d)), ("dv", dv, (B, H, Sk, d))):
        _check_bf16(n, t, s)
    _check_f32("lse", lse, (B, H, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = workspace.numel() * workspace.element_size()
    head = () if phases is None else (int(phases),)
    st = getattr(lib(), name)(*head, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                              _ptr(dv), B, H, Sq, Sk, d, int(bool(causal)), float(scale), int(bool(deterministic)),
                              _ptr(workspace), ws_bytes, _stream(q))
    if st != FA_OK:
        raise FAError(st, name)


def fa_bwd_ds(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=False, scale=None, deterministic=False):
    """Enqueue the five-product backward (dS through the workspace) on the
    current stream; fills dq, dk, dv in place."""
    _bwd_call("fa_bwd_ds", q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, scale, deterministic)


def fa_bwd_ds_phase(phases, q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=False, scale=None,
                    deterministic=False):
    """Enqueue some of fa_bwd_ds's launches (FA_BWD_PREPARE, then FA_BWD_DKDV,
    then FA_BWD_DQ) on the current stream."""
    _bwd_call("fa_bwd_ds_phase", q, k, v, o, lse, dout, dq, dk, dv, workspace, causal, scale, deterministic,
              phases=phases)


def backward_ds(q, k, v, o, lse, dout, causal=False, scale=None, deterministic=False, workspace=None):
    """Five-product backward; returns (dQ, dK, dV) bf16."""
    import torch
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    if workspace is None:
        nbytes = fa_bwd_ds_workspace_bytes(B, H, Sq, Sk, d, causal, deterministic)
        if nbytes == 0:
            raise FAError(FA_ERR_UNSUPPORTED, "fa_bwd_ds_workspace_bytes")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    fa_bwd_ds(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=causal, scale=scale, deterministic=deterministic)
    return dq, dk, dv


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=False, scale=None, deterministic=False):
    """Enqueue the backward on the current stream; fills dq, dk, dv in place."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    for name, t, s in (("q", q, (B, H, Sq, d)), ("k", k, (B, H, Sk, d)), ("v", v, (B, H, Sk, d)),
                       ("o", o, (B, H, Sq, d)), ("dout", dout, (B, H, Sq, d)), ("dq", dq, (B, H, Sq, d)),
                       ("dk", dk, (B, H, Sk, d)), ("dv", dv, (B, H, Sk, d))):
        _check_bf16(name, t, s)
    _check_f32("lse", lse, (B, H, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, H, Sq, Sk, d, int(bool(causal)), float(scale), int(bool(deterministic)),
                      _ptr(workspace), ws_bytes, _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=False, scale=None, deterministic=False):
    """fa_bwd without a caller workspace (the library's fixed scratch; no
    device allocation): fills dq, dk, dv in place."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    for name, t, s in (("q", q, (B, H, Sq, d)), ("k", k, (B, H, Sk, d)), ("v", v, (B, H, Sk, d)),
                       ("o", o, (B, H, Sq, d)), ("dout", dout, (B, H, Sq, d)), ("dq", dq, (B, H, Sq, d)),
                       ("dk", dk, (B, H, Sk, d)), ("dv", dv, (B, H, Sk, d))):
        _check_bf16(name, t, s)
    _check_f32("lse", lse, (B, H, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                              _ptr(dv), B, H, Sq, Sk, d, int(bool(causal)), float(scale), int(bool(deterministic)),
                              _stream(q))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_noalloc")


def fa_exp2_probe(x, y_hw, y_emu):
    """Hardware and software 2^x of a float32 CUDA tensor, written in place."""
    n = x.numel()
    for name, t in (("x", x), ("y_hw", y_hw), ("y_emu", y_emu)):
        _check_f32(name, t, (n,))
    st = lib().fa_exp2_probe(_ptr(x), _ptr(y_hw), _ptr(y_emu), n, _stream(x))
    if st != FA_OK:
        raise FAError(st, "fa_exp2_probe")


# ------------------------------------------------------ allocating helpers
def forward_fp8(q8, k8, v8, q_descale=1.0, k_descale=1.0, v_descale=1.0, causal=False, scale=None, tau=8.0,
                head_descales=None):
    """Returns (O bf16 [B,H,Sq,d], LSE float32 [B,H,Sq]) of the e4m3 forward."""
    import torch
    B, H, Sq, d = q8.shape
    o = torch.empty((B, H, Sq, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q8.device)
    fa_fwd_fp8(q8, k8, v8, o, lse, q_descale, k_descale, v_descale, causal=causal, scale=scale, tau=tau,
               head_descales=head_descales)
    return o, lse


def forward_fp8_blocks(q8, k8, v8, q_factors, k_factors, v_factors, causal=False, scale=None, tau=8.0):
    """Returns (O bf16 [B,H,Sq,d], LSE float32 [B,H,Sq]) of the e4m3 forward
    with per-block factors."""
    import torch
    B, H, Sq, d = q8.shape
    o = torch.empty((B, H, Sq, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q8.device)
    fa_fwd_fp8_blocks(q8, k8, v8, q_factors, k_factors, v_factors, o, lse, causal=causal, scale=scale, tau=tau)
    return o, lse


def forward(q, k, v, causal=False, scale=None, tau=8.0, emu_frac=0.0):
    """Returns (O bf16 [B,H,Sq,d], LSE float32 [B,H,Sq])."""
    import torch
    B, H, Sq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, causal=causal, scale=scale, tau=tau, emu_frac=emu_frac)
    return o, lse


def forward_partial(q, k, v, q_offset, k_begin, k_end, causal=False, scale=None, tau=8.0, emu_frac=0.0):
    """Returns (O_part float32 [B,H,Sq,d], LSE_part float32 [B,H,Sq])."""
    import torch
    B, H, Sq, d = q.shape
    o = torch.empty((B, H, Sq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    fa_fwd_partial(q, k, v, o, lse, q_offset, k_begin, k_end, causal=causal, scale=scale, tau=tau, emu_frac=emu_frac)
    return o, lse


def merge(o_parts, lse_parts):
    """Returns (O bf16 [B,H,Sq,d], LSE float32 [B,H,Sq])."""
    import torch
    n, B, H, Sq, d = o_parts.shape
    o = torch.empty((B, H, Sq, d), dtype=torch.bfloat16, device=o_parts.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=o_parts.device)
    fa_merge(o_parts, lse_parts, o, lse)
    return o, lse


def backward(q, k, v, o, lse, dout, causal=False, scale=None, deterministic=False, workspace=None):
    """Returns (dQ, dK, dV) bf16."""
    import torch
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    if workspace is None:
        nbytes = fa_bwd_workspace_bytes(B, H, Sq, Sk, d, causal, deterministic)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=causal, scale=scale,
           deterministic=deterministic)
    return dq, dk, dv
