"""Seeded synthetic inputs for the attention workloads.

This module only draws inputs; it holds none of the attention arithmetic and
is shared by the tests, the benchmark and the smoke check (the CPU oracle and
the HIP library never import it).

Recipe (the pages measure on synthetic kernel sweeps with unstated shapes, so
no public dataset is involved):
  * one CPU ``torch.Generator`` per workload, seeded by the workload's seed;
  * draw order Q, K, V, then dO for the backward workload;
  * each tensor is float32 N(0, 1) rounded to bf16 (round-to-nearest-even by
    ``Tensor.to``), layout [B, H, S, d] contiguous;
  * the rescale-stress workload adds, before rounding, a per-key bias along
    the unit mean direction u of the (b, h) slice's queries:
    k_j += (ramp * sqrt(d) * j / (Sk - 1)) * u, with ramp = 6 -- six standard
    deviations of the raw score q.k (whose deviation is sqrt(d)) at the last
    key, so row maxima keep rising and some rows cross tau = 8 (log2 units).
"""
import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    d: int
    causal: bool
    seed: int
    kind: str = "fwd"               # "fwd" or "bwd" (bwd also runs fwd for O, LSE)
    key_ramp: float = 0.0           # in standard deviations of q.k
    emu_fracs: tuple = (0.0,)
    extra: dict = field(default_factory=dict)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    def flops(self, pass_="fwd"):
        """Counted FLOPs: forward 4*B*H*Sq*Sk*d, backward 10*B*H*Sq*Sk*d;
        causal counts half."""
        per_pair = 4 if pass_ == "fwd" else 10
        f = per_pair * self.B * self.H * self.Sq * self.Sk * self.d
        return f / 2 if self.causal else f


WORKLOADS = {
    1: Workload("tiny-fwd-noncausal-B1H2S256d64", 1, 2, 256, 256, 64, False, seed=1),
    2: Workload("fwd-noncausal-B2H16S2048d128", 2, 16, 2048, 2048, 128, False, seed=2),
    3: Workload("fwd-causal-B1H16S8192d128", 1, 16, 8192, 8192, 128, True, seed=3),
    4: Workload("fwd-causal-rescale-stress-B4H32S4096d64", 4, 32, 4096, 4096, 64, True, seed=4,
                key_ramp=6.0, emu_fracs=(0.0, 0.10, 0.25)),
    5: Workload("bwd-causal-B1H16S4096d128", 1, 16, 4096, 4096, 128, True, seed=5, kind="bwd"),
}

# Supplementary shapes, reported beside the configurations above and labelled
# as extra: the non-causal forward at S = 8192, d = 128.
EXTRA_WORKLOADS = {
    6: Workload("extra-fwd-noncausal-B1H16S8192d128", 1, 16, 8192, 8192, 128, False, seed=6),
}


def make_inputs(B, H, Sq, Sk, d, seed, key_ramp=0.0, with_dout=False, heads=None):
    """Draw bf16 Q, K, V (and dO) on the CPU.

    ``heads``: optional (h0, h1) to return only that head range of the full
    draw (the full tensors are drawn so a subset matches the full workload).
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((B, H, Sq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Sk, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Sk, d), generator=g, dtype=torch.float32)
    do = torch.randn((B, H, Sq, d), generator=g, dtype=torch.float32) if with_dout else None
    if key_ramp:
        u = q.mean(dim=2, keepdim=True)
        u = u / u.norm(dim=-1, keepdim=True)
        ramp = key_ramp * math.sqrt(d) * torch.arange(Sk, dtype=torch.float32) / max(1, Sk - 1)
        k = k + ramp[None, None, :, None] * u
    out = [q, k, v] + ([do] if with_dout else [])
    if heads is not None:
        out = [t[:, heads[0]:heads[1]] for t in out]
    out = [t.to(torch.bfloat16).contiguous() for t in out]
    return tuple(out)


def workload_inputs(w, heads=None):
    return make_inputs(w.B, w.H, w.Sq, w.Sk, w.d, w.seed, key_ramp=w.key_ramp,
                       with_dout=(w.kind == "bwd"), heads=heads)


def quantise_e4m3(x, amax=224.0):
    """e4m3 codes (uint8, torch's round-to-nearest float8_e4m3fn conversion)
    and the per-tensor dequantisation factor of a float tensor: x is divided
    by max|x| / amax first, so its largest magnitude lands on amax (half of
    e4m3's 448, leaving room for rounding)."""
    descale = float(x.abs().max()) / amax if float(x.abs().max()) > 0 else 1.0
    codes = (x.float() / descale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, descale


def quantise_e4m3_per_head(x, amax=224.0):
    """As quantise_e4m3, with one dequantisation factor per (batch, head)
    slice of x [B,H,S,d]: returns uint8 codes and float32 factors [B,H]."""
    m = x.float().abs().amax(dim=(2, 3))
    descale = torch.where(m > 0, m / amax, torch.ones_like(m))
    codes = (x.float() / descale[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, descale


_E2M1_MAGS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantise_mxfp4(x, block=32):
    """MXFP4 codes of a float tensor [..., d] (d a multiple of 2 * block/2):
    per block of `block` consecutive elements of a row, the shared exponent
    X = floor(log2(max |x|)) - 2 (the OCP microscaling rule for E2M1, whose
    largest exponent is 2), stored as the E8M0 byte X + 127; each element
    x / 2^X goes to the nearest E2M1 value (ties to the even code), saturating
    at +-6.  Returns (packed uint8 [..., d/2], element 2j in the low nibble of
    byte j; scales uint8 [..., d/block])."""
    xf = x.float()
    shp = xf.shape
    blocks = xf.reshape(shp[:-1] + (shp[-1] // block, block))
    amax = blocks.abs().amax(dim=-1, keepdim=True)
    X = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.full_like(amax, -127.0))
    X = X.clamp(-127, 127)
    y = (blocks / torch.exp2(X)).reshape(shp)
    mags = torch.tensor(_E2M1_MAGS, dtype=torch.float32)
    dist = (y.abs().clamp(max=6.0)[..., None] - mags).abs()
    # nearest magnitude; on a tie the even code (mantissa bit 0) wins
    dist = dist + 1e-6 * (torch.arange(8) & 1).float()
    idx = dist.argmin(dim=-1)
    codes = (idx | torch.where(y < 0, 8, 0)).to(torch.uint8)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).to(torch.uint8).contiguous()
    scales = (X.squeeze(-1) + 127).to(torch.uint8).contiguous()
    return packed, scales


def quantise_e4m3_blocks(x, block=128, amax=224.0):
    """e4m3 codes of x [B,H,S,d] with one dequantisation factor per block of
    `block` consecutive rows of each (batch, head) slice (the last block may
    be shorter): each block is divided by its max|x| / amax (1 for an
    all-zero block) and converted with torch's round-to-nearest
    float8_e4m3fn.  Returns (uint8 codes, float32 factors [B,H,ceil(S/block)])."""
    B, H, S, d = x.shape
    nb = (S + block - 1) // block
    xf = x.float()
    pad = torch.zeros((B, H, nb * block - S, d), dtype=torch.float32)
    blocks = torch.cat([xf, pad], dim=2).reshape(B, H, nb, block, d)
    m = blocks.abs().amax(dim=(3, 4))
    f = torch.where(m > 0, m / amax, torch.ones_like(m))
    codes = (blocks / f[:, :, :, None, None]).reshape(B, H, nb * block, d)[:, :, :S]
    return codes.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), f.contiguous()
