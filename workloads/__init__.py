"""Seeded synthetic inputs for chunkwise context-parallel linear attention.

This module only draws random tensors with the shapes, dtypes and value
distributions of the five workloads below. It holds none of the method's
arithmetic: no cumulative decays, no states, no sequence-id expansion. Both the
CPU oracle and the GPU path consume exactly what it returns (CPU tensors; the
GPU side copies them to the device).

Workloads (every one uses chunk length C = 64):

* ``identity_fwd``  -- plain causal linear attention (no decay), forward only.
  B=1, H=1, T=256, d_k=d_v=16, fp32; q, k, v ~ N(0,1)/sqrt(16); 4 shards of 64.
* ``scalar_fwd``    -- scalar per-head decay, forward only. B=2, H=8, T=4096,
  d=64, bf16 q/k/v ~ N(0,1)/8; log-decay g = -softplus(N(0,1)) fp32 per
  (b,t,h); 8 shards of 512.
* ``diag_fwdbwd``   -- per-key-dimension gated decay, forward+backward. B=4,
  H=16, T=8192, d=128, bf16 q/k/v ~ N(0,1)/sqrt(128); log-decay per
  (b,t,h,d_k) = logsigmoid(N(0,1))/16 fp32; dO bf16 ~ N(0,1); 8 shards of 1024.
* ``packed_fwdbwd`` -- one packed stream of 32768 tokens, H=16, d=128, bf16;
  sequence lengths uniform integers in [128, 4096] drawn until the stream is
  full, the last one truncated; scalar decay as in ``scalar_fwd``; q/k/v
  ~ N(0,1)/sqrt(128); dO ~ N(0,1); 16 shards of 2048.
* ``long_fwdbwd``   -- one GPU's share of a 1,048,576-token sequence: B=1,
  H=32, T=131072, d=128; q bf16 ~ N(0,1); k bf16 = per-token L2-normalised
  N(0,1) (normalised in fp32, then rounded); v bf16 ~ N(0,1); scalar decay
  g = -softplus(N(0,1)+2); incoming state S_in fp32 ~ N(0, 0.1^2) per head;
  dO ~ N(0,1); 16 shards of 8192.

Draw order per workload (generator seeded ``1000 + index``, index 1..5 in the
order above): sequence lengths (packed only), q, k, v, g-noise, dO, S_in. All
draws are fp32; transforms are applied in fp32; bf16 tensors are then rounded
to nearest even by ``Tensor.to(torch.bfloat16)``.

``make(name, **overrides)`` returns a ``Workload`` whose shapes may be shrunk
(``B``, ``T``, ``H``, ``d``, ``num_shards``) for fast tests while keeping the
distributions; ``decay_scale`` multiplies g (weak-decay coverage variants); ``dtype`` overrides
the storage dtype of q/k/v/dO (same fp32 draws, different rounding).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch
import torch.nn.functional as F

CHUNK = 64


@dataclasses.dataclass(frozen=True)
class Spec:
    index: int
    B: int
    T: int
    H: int
    d: int
    dtype: torch.dtype
    decay: str            # "none" | "scalar" | "diag"
    num_shards: int
    backward: bool
    packed: bool = False
    initial_state: bool = False


SPECS = {
    "identity_fwd": Spec(1, 1, 256, 1, 16, torch.float32, "none", 4, False),
    "scalar_fwd": Spec(2, 2, 4096, 8, 64, torch.bfloat16, "scalar", 8, False),
    "diag_fwdbwd": Spec(3, 4, 8192, 16, 128, torch.bfloat16, "diag", 8, True),
    "packed_fwdbwd": Spec(4, 1, 32768, 16, 128, torch.bfloat16, "scalar", 16, True, packed=True),
    "long_fwdbwd": Spec(5, 1, 131072, 32, 128, torch.bfloat16, "scalar", 16, True, initial_state=True),
}


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    d: int                               # d_k (q, k, g per key dim)
    dtype: torch.dtype
    decay: str
    num_shards: int
    chunk: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: Optional[torch.Tensor]
    dO: Optional[torch.Tensor]
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[object]         # packed only: int32 [N+1] (B == 1), or a list of B of them

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def dv(self) -> int:
        return self.v.shape[-1]


def _lengths(gen: torch.Generator, T: int, lo: int, hi: int) -> torch.Tensor:
    """Uniform integer lengths in [lo, hi] until they cover T; last one truncated."""
    out = []
    total = 0
    while total < T:
        n = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
        n = min(n, T - total)
        out.append(n)
        total += n
    cu = [0]
    for n in out:
        cu.append(cu[-1] + n)
    return torch.tensor(cu, dtype=torch.int32)


def _packing(gen: torch.Generator, B: int, T: int, lo: int, hi: int):
    """One packed stream (B == 1) or one packing per batch row, each of T tokens."""
    if B == 1:
        return _lengths(gen, T, lo, hi)
    return [_lengths(gen, T, lo, hi) for _ in range(B)]


def make(name: str, *, B: Optional[int] = None, T: Optional[int] = None,
         H: Optional[int] = None, d: Optional[int] = None, dv: Optional[int] = None,
         num_shards: Optional[int] = None, decay_scale: float = 1.0,
         seed_offset: int = 0, len_range: Optional[tuple] = None,
         with_initial_state: Optional[bool] = None,
         backward: Optional[bool] = None, dtype: Optional[torch.dtype] = None,
         packed: Optional[bool] = None) -> Workload:
    spec = SPECS[name]
    B = spec.B if B is None else B
    T = spec.T if T is None else T
    H = spec.H if H is None else H
    d = spec.d if d is None else d
    dv = d if dv is None else dv        # value head dim (d_v); d is d_k
    P = spec.num_shards if num_shards is None else num_shards
    bwd = spec.backward if backward is None else backward
    init = spec.initial_state if with_initial_state is None else with_initial_state
    gen = torch.Generator().manual_seed(1000 + spec.index + seed_offset)

    cu = None
    if spec.packed if packed is None else packed:
        lo, hi = (128, 4096) if len_range is None else len_range
        cu = _packing(gen, B, T, lo, hi)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32)

    if name == "long_fwdbwd":
        q = randn(B, T, H, d)
        k = randn(B, T, H, d)
        k = k / k.norm(dim=-1, keepdim=True)
        v = randn(B, T, H, dv)
    else:
        scale = {"identity_fwd": 1.0 / math.sqrt(16), "scalar_fwd": 1.0 / 8}.get(
            name, 1.0 / math.sqrt(128))
        q = randn(B, T, H, d) * scale
        k = randn(B, T, H, d) * scale
        v = randn(B, T, H, dv) * scale

    g = None
    if spec.decay == "scalar":
        noise = randn(B, T, H)
        if name == "long_fwdbwd":
            g = -F.softplus(noise + 2.0)
        else:
            g = -F.softplus(noise)
    elif spec.decay == "diag":
        g = F.logsigmoid(randn(B, T, H, d)) / 16.0
    if g is not None and decay_scale != 1.0:
        g = g * decay_scale

    dO = randn(B, T, H, dv) if bwd else None
    S0 = randn(B, H, d, dv) * 0.1 if init else None

    dt = spec.dtype if dtype is None else dtype
    return Workload(
        name=name, B=B, T=T, H=H, d=d, dtype=dt, decay=spec.decay, num_shards=P,
        chunk=CHUNK,
        q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
        g=None if g is None else g.contiguous(),
        dO=None if dO is None else dO.to(dt).contiguous(),
        initial_state=None if S0 is None else S0.contiguous(),
        cu_seqlens=cu)


# ---- Mamba2 (SSD) inputs --------------------------------------------------------------------
# Shapes of a Mamba2 layer: x [B,T,H,P] (P = N unless given), dt [B,T,H], A [H], and B, C
# [B,T,G,N] shared by the H/G heads of a group. Distributions follow Mamba2's
# parameter initialisation: dt log-uniform in [1e-3, 1e-1] (as dt after its
# softplus), A = -U[1, 16] per head; x ~ N(0,1); B, C ~ N(0,1) / N^(1/4) so that
# C_t . B_s is of order one; dy ~ N(0,1); h_init ~ N(0, 0.1^2).

@dataclasses.dataclass(frozen=True)
class SsdSpec:
    index: int
    B: int
    T: int
    H: int
    G: int
    N: int
    dtype: torch.dtype
    num_shards: int


SSD_SPECS = {
    "ssd_fwdbwd": SsdSpec(6, 2, 4096, 8, 2, 64, torch.bfloat16, 8),
}


@dataclasses.dataclass
class SsdWorkload:
    name: str
    B: int
    T: int
    H: int
    G: int
    N: int
    dtype: torch.dtype
    num_shards: int
    x: torch.Tensor
    dt: torch.Tensor
    A: torch.Tensor
    Bm: torch.Tensor
    Cm: torch.Tensor
    dy: torch.Tensor
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[object]         # as Workload.cu_seqlens

    @property
    def tokens(self) -> int:
        return self.B * self.T


def make_ssd(name: str = "ssd_fwdbwd", *, B: Optional[int] = None, T: Optional[int] = None,
             H: Optional[int] = None, G: Optional[int] = None, N: Optional[int] = None,
             P: Optional[int] = None,
             num_shards: Optional[int] = None, packed: bool = False, len_range: tuple = (64, 1024),
             with_initial_state: bool = False, dtype: Optional[torch.dtype] = None,
             seed_offset: int = 0) -> SsdWorkload:
    spec = SSD_SPECS[name]
    B = spec.B if B is None else B
    T = spec.T if T is None else T
    H = spec.H if H is None else H
    G = spec.G if G is None else G
    N = spec.N if N is None else N
    hd = N if P is None else P          # head dim of x and y (Mamba2's P); N is the state size
    P = spec.num_shards if num_shards is None else num_shards
    gen = torch.Generator().manual_seed(1000 + spec.index + seed_offset)
    cu = _packing(gen, B, T, len_range[0], len_range[1]) if packed else None

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32)

    def rand(*shape):
        return torch.rand(*shape, generator=gen, dtype=torch.float32)

    x = randn(B, T, H, hd)
    dt = torch.exp(math.log(1e-3) + rand(B, T, H) * (math.log(1e-1) - math.log(1e-3)))
    A = -(1.0 + 15.0 * rand(H))
    Bm = randn(B, T, G, N) / N ** 0.25
    Cm = randn(B, T, G, N) / N ** 0.25
    dy = randn(B, T, H, hd)
    h0 = randn(B, H, N, hd) * 0.1 if with_initial_state else None
    dtp = spec.dtype if dtype is None else dtype
    return SsdWorkload(name=name, B=B, T=T, H=H, G=G, N=N, dtype=dtp, num_shards=P,
                       x=x.to(dtp).contiguous(), dt=dt.contiguous(), A=A.contiguous(),
                       Bm=Bm.to(dtp).contiguous(), Cm=Cm.to(dtp).contiguous(), dy=dy.to(dtp).contiguous(),
                       initial_state=None if h0 is None else h0.contiguous(), cu_seqlens=cu)


# ---- gated delta rule inputs ------------------------------------------------------------------
# A gated-DeltaNet layer's shapes: q, k L2-normalised per head (the usual setting,
# keeping I - beta k k^T a contraction), v ~ N(0, 1), beta = sigmoid(N(0, 1)) and a
# per-head log-decay g = logsigmoid(N(0, 1) + 3) (about -0.05 per token).
@dataclasses.dataclass
class DeltaSpec:
    index: int
    B: int
    T: int
    H: int
    d: int
    dtype: torch.dtype
    num_shards: int


DELTA_SPECS = {
    "delta_fwdbwd": DeltaSpec(7, 2, 8192, 16, 64, torch.bfloat16, 8),
    "delta_d128_fwdbwd": DeltaSpec(8, 2, 8192, 16, 128, torch.bfloat16, 8),
}


@dataclasses.dataclass
class DeltaWorkload:
    name: str
    B: int
    T: int
    H: int
    d: int
    dtype: torch.dtype
    num_shards: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    dO: torch.Tensor
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[object]

    @property
    def tokens(self) -> int:
        return self.B * self.T


def make_delta(name: str = "delta_fwdbwd", *, B: Optional[int] = None, T: Optional[int] = None,
               H: Optional[int] = None, d: Optional[int] = None, num_shards: Optional[int] = None,
               packed: bool = False, len_range: tuple = (64, 1024), with_initial_state: bool = False,
               dtype: Optional[torch.dtype] = None, seed_offset: int = 0) -> DeltaWorkload:
    spec = DELTA_SPECS[name]
    B = spec.B if B is None else B
    T = spec.T if T is None else T
    H = spec.H if H is None else H
    d = spec.d if d is None else d
    P = spec.num_shards if num_shards is None else num_shards
    gen = torch.Generator().manual_seed(1000 + spec.index + seed_offset)
    cu = _packing(gen, B, T, len_range[0], len_range[1]) if packed else None

    def randn(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32)

    q = F.normalize(randn(B, T, H, d), dim=-1)
    k = F.normalize(randn(B, T, H, d), dim=-1)
    v = randn(B, T, H, d)
    beta = torch.sigmoid(randn(B, T, H))
    g = F.logsigmoid(randn(B, T, H) + 3.0)
    dO = randn(B, T, H, d)
    S0 = randn(B, H, d, d) * 0.1 if with_initial_state else None
    dt = spec.dtype if dtype is None else dtype
    return DeltaWorkload(name=name, B=B, T=T, H=H, d=d, dtype=dt, num_shards=P,
                         q=q.to(dt).contiguous(), k=k.to(dt).contiguous(), v=v.to(dt).contiguous(),
                         g=g.contiguous(), beta=beta.contiguous(), dO=dO.to(dt).contiguous(),
                         initial_state=None if S0 is None else S0.contiguous(), cu_seqlens=cu)
