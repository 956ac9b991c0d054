"""PyTorch-facing calls of the chunkwise CP linear-attention library.

PyTorch provides device memory and the current HIP stream; every step of the
computation runs in libcpla's kernels. The split mirrors the Megatron-Core page
``core.ssm.context_parallel.chunkwise``: ``forward`` = cp_forward_prepare +
cp_forward_apply over all simulated shards (``chunkwise_cp_forward`` on one
GPU), ``backward`` = cp_backward_prepare + cp_backward_apply
(``chunkwise_cp_backward``); ``Context`` plays the part of ``CPSavedContext``
(tensors only, plus a plain problem description).
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import CplaError, Packed, Problem, SsdProblem, check

_DTYPE = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


# ---- argument checks ------------------------------------------------------------------
# The C ABI takes plain device pointers and cannot see a tensor's size, dtype or
# device, so every tensor is checked here against the shapes the call implies
# before any pointer is handed over: a wrong one raises instead of reaching a
# kernel. Shapes and dtypes are checked first, the device last.

def _expect(name: str, t, shape, dtype, device=None, optional: bool = False):
    if t is None:
        if optional:
            return
        raise CplaError(1, f"{name} is required")
    if not torch.is_tensor(t):
        raise CplaError(1, f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise CplaError(2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise CplaError(3, f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise CplaError(1, f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise CplaError(1, f"{name} is on {t.device}, expected {device}")


def _expect_gpu(first: str, tensors: dict):
    """Every given tensor on the GPU that holds the first one."""
    dev = tensors[first].device
    if dev.type != "cuda":
        raise CplaError(1, f"{first} must be on a GPU (got {dev}); the library has no host path")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise CplaError(1, f"{name} is on {t.device}, expected {dev}")


def _check_packed(packed, B: int, T: int, P: int, device):
    if packed is None:
        return
    _expect("packed.seq_idx", packed.seq_idx, (B, T), torch.int32, device)
    _expect("packed.preceding_rank_start", packed.preceding_rank_start, (B, P), torch.int32, device)
    _expect("packed.following_rank_stop", packed.following_rank_stop, (B, P), torch.int32, device)


# ---- packed-sequence metadata (host, in the library) --------------------------------

def shard_len(T: int, P: int, r: int) -> int:
    """Tokens of shard r when T tokens are divided among P shards the way
    torch.chunk divides them (the library's division; see include/cpla.h)."""
    if P <= 0 or T <= 0 or not 0 <= r < P:
        return 0
    size = -(-T // P)
    return max(0, min(size, T - r * size))


def seq_idx_from_cu_seqlens(cu_seqlens, T: int) -> np.ndarray:
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    out = np.empty(T, dtype=np.int32)
    check(_lib.lib().cpla_seq_idx_from_cu_seqlens(_i32p(cu), len(cu) - 1, T, _i32p(out)))
    return out


def packed_rank_slices(global_seq_idx: np.ndarray, cp_size: int):
    s = np.ascontiguousarray(global_seq_idx, dtype=np.int32)
    prs = np.empty(cp_size, dtype=np.int32)
    frs = np.empty(cp_size, dtype=np.int32)
    check(_lib.lib().cpla_packed_rank_slices(_i32p(s), len(s), cp_size, _i32p(prs), _i32p(frs)))
    return prs, frs


def build_packed_sequence_cp_metadata(global_seq_idx, cp_rank: int, cp_size: int) -> dict:
    s = np.ascontiguousarray(np.asarray(global_seq_idx), dtype=np.int32)
    L = shard_len(len(s), cp_size, cp_rank)
    local = np.empty(max(L, 1), dtype=np.int32)
    cu = np.empty(max(L, 1) + 1, dtype=np.int32)
    n = ctypes.c_int32()
    prs = ctypes.c_int32()
    frs = ctypes.c_int32()
    pi = ctypes.POINTER(ctypes.c_int32)
    check(_lib.lib().build_packed_sequence_cp_metadata(
        _i32p(s), len(s), cp_rank, cp_size, _i32p(local), _i32p(cu), ctypes.cast(ctypes.byref(n), pi),
        ctypes.cast(ctypes.byref(prs), pi), ctypes.cast(ctypes.byref(frs), pi)))
    return {"local_seq_idx": local[:L].copy(), "local_cu_seqlens": cu[:n.value + 1].copy(),
            "preceding_rank_start": prs.value, "following_rank_stop": frs.value}


@dataclasses.dataclass
class PackedMeta:
    seq_idx: torch.Tensor                 # device int32 [B, T]: each batch row packed on its own
    preceding_rank_start: torch.Tensor    # device int32 [B, P]
    following_rank_stop: torch.Tensor     # device int32 [B, P]

    def c(self) -> Packed:
        return Packed(self.seq_idx.data_ptr(), self.preceding_rank_start.data_ptr(),
                      self.following_rank_stop.data_ptr())


def _cu_rows(cu_seqlens, B: int):
    """cu_seqlens of every batch row: one 1-D cu_seqlens (B == 1), or one per row
    (a sequence of B of them, or a 2-D array when the rows hold equally many)."""
    if torch.is_tensor(cu_seqlens):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    if isinstance(cu_seqlens, np.ndarray):
        rows = [cu_seqlens] if cu_seqlens.ndim == 1 else list(cu_seqlens)
    else:
        items = list(cu_seqlens)
        rows = [np.asarray(items)] if items and np.ndim(items[0]) == 0 else [
            c.detach().cpu().numpy() if torch.is_tensor(c) else np.asarray(c) for c in items]
    if len(rows) != B:
        raise CplaError(2, f"cu_seqlens describes {len(rows)} packed rows for B={B}")
    return rows


def packed_meta(cu_seqlens, T: int, num_shards: int, device, B: int = 1) -> PackedMeta:
    """Device metadata for B packed rows of T tokens (``cu_seqlens`` as ``_cu_rows`` reads it)."""
    seqs, prss, frss = [], [], []
    for cu in _cu_rows(cu_seqlens, B):
        s = seq_idx_from_cu_seqlens(cu, T)
        prs, frs = packed_rank_slices(s, num_shards)
        seqs.append(s)
        prss.append(prs)
        frss.append(frs)
    dev = torch.device(device)
    return PackedMeta(*(torch.from_numpy(np.stack(x)).to(dev) for x in (seqs, prss, frss)))


# ---- forward / backward ----------------------------------------------------------------

@dataclasses.dataclass
class Context:
    problem: Problem
    decay: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: Optional[torch.Tensor]
    packed: Optional[PackedMeta]
    fwd_summary: torch.Tensor
    shard_in_state: torch.Tensor
    final_state: torch.Tensor
    chunk_states: Optional[torch.Tensor]
    has_initial_state: bool
    w: Optional[torch.Tensor] = None     # per-token input weights (scalar decay)


def _decay_of(g: Optional[torch.Tensor], q: torch.Tensor) -> int:
    if g is None:
        return _lib.DECAY_NONE
    if g.dim() == 3:
        return _lib.DECAY_SCALAR
    if g.dim() == 4 and g.shape[-1] == q.shape[-1]:
        return _lib.DECAY_DIAG
    raise ValueError(f"g must be [B,T,H] or [B,T,H,dk], got {tuple(g.shape)}")


def make_problem(q, v, num_shards: int, decay: int, chunk: int = 64, rank_range=None) -> Problem:
    """The problem of q [B,T,Hq,dk] and v [B,T,H,dv]; Hq < H (a divisor of H) shares
    each q and k head among H / Hq consecutive heads (qk_heads = Hq)."""
    B, T, Hq, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    if q.dtype not in _DTYPE:
        raise CplaError(3, f"dtype {q.dtype} unsupported")
    rb, re = (0, num_shards) if rank_range is None else rank_range
    return Problem(B, T, H, dk, dv, num_shards, chunk, rb, re, _DTYPE[q.dtype], decay, 0 if Hq == H else Hq)


def check_decay_range(g: torch.Tensor, num_shards: int, dk: Optional[int] = None) -> None:
    """Raise CplaError (INVALID) if a diagonal log-decay g [B,T,H,dk] leaves the range
    the kernels support (a chunk's running sum per key dim below
    CPLA_DIAG_GAMMA_MIN); synchronises the current stream. Scalar decays have no
    such limit."""
    if g is None or g.dim() != 4:
        return
    B, T, H, d = g.shape
    _expect("g", g, (B, T, H, d), torch.float32)
    _expect_gpu("g", dict(g=g))
    p = Problem(B, T, H, d, d, num_shards, 64, 0, num_shards, _lib.BF16, _lib.DECAY_DIAG)
    count = torch.empty(4, dtype=torch.int32, device=g.device)
    check(_lib.lib().cpla_check_decay_range(ctypes.byref(p), _ptr(g), _ptr(count), _stream()))


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor] = None, *,
            num_shards: int, initial_state: Optional[torch.Tensor] = None, cu_seqlens=None,
            packed: Optional[PackedMeta] = None, save_for_backward: bool = True, chunk: int = 64,
            out: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None):
    """o [B,T,H,dv] (dtype of q) and a Context for ``backward``. ``w`` [B,T,H] fp32:
    per-token input weights (scalar decay): S_t = exp(g_t) S_{t-1} + w_t k_t v_t^T.
    q and k may have fewer heads than v, a divisor Hq of H: head h then reads their
    head h // (H // Hq) (Mamba2's B and C shared by a group of heads)."""
    if not torch.is_tensor(q) or q.dim() != 4 or not torch.is_tensor(v) or v.dim() != 4:
        raise CplaError(2, "q and v must be [B,T,H,d] tensors")
    if q.dtype not in _DTYPE:
        raise CplaError(3, f"dtype {q.dtype} unsupported")
    B, T, Hq, dk = q.shape
    H, dv = v.shape[2], v.shape[-1]
    if Hq <= 0 or H % Hq != 0:
        raise CplaError(2, f"q and k have {Hq} heads, which does not divide the {H} heads of v")
    _expect("q", q, (B, T, Hq, dk), q.dtype)
    _expect("k", k, (B, T, Hq, dk), q.dtype)
    _expect("v", v, (B, T, H, dv), q.dtype)
    if g is not None and g.dim() == 4:
        _expect("g", g, (B, T, H, dk), torch.float32)
    else:
        _expect("g", g, (B, T, H), torch.float32, optional=True)
    _expect("initial_state", initial_state, (B, H, dk, dv), torch.float32, optional=True)
    _expect("w", w, (B, T, H), torch.float32, optional=True)
    _expect("out", out, (B, T, H, dv), q.dtype, optional=True)
    _expect_gpu("q", dict(q=q, k=k, v=v, g=g, initial_state=initial_state, w=w, out=out))
    _check_packed(packed, B, T, num_shards, q.device)
    decay = _decay_of(g, q)
    p = make_problem(q, v, num_shards, decay, chunk)
    if cu_seqlens is not None and packed is None:
        packed = packed_meta(cu_seqlens, q.shape[1], num_shards, q.device, q.shape[0])
    L = _lib.lib()
    W = L.cpla_summary_width(ctypes.byref(p))
    dev = q.device
    fsum = torch.empty((num_shards, B, H, W), device=dev, dtype=torch.float32)
    s_in = torch.empty((num_shards, B, H, dk, dv), device=dev, dtype=torch.float32)
    fin = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
    cs = None
    if save_for_backward:
        n_chunks = L.cpla_chunk_states_bytes(ctypes.byref(p)) // (B * H * dk * dv * 4)
        cs = torch.empty((B, H, n_chunks, dk, dv), device=dev, dtype=torch.float32)
    o = torch.empty(v.shape, device=dev, dtype=q.dtype) if out is None else out
    pk = ctypes.byref(packed.c()) if packed is not None else None
    st = _stream()
    if w is None:
        check(L.cp_forward_prepare(ctypes.byref(p), pk, _ptr(k), _ptr(v), _ptr(g), _ptr(fsum), st))
        check(L.cp_forward_apply(ctypes.byref(p), pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(fsum),
                                 _ptr(initial_state), _ptr(o), _ptr(s_in), _ptr(fin), _ptr(cs), st))
    else:
        check(L.cp_forward_prepare_weighted(ctypes.byref(p), pk, _ptr(k), _ptr(v), _ptr(g), _ptr(w), _ptr(fsum), st))
        check(L.cp_forward_apply_weighted(ctypes.byref(p), pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(w),
                                          _ptr(fsum), _ptr(initial_state), _ptr(o), _ptr(s_in), _ptr(fin), _ptr(cs),
                                          st))
    ctx = Context(p, decay, q, k, v, g, packed, fsum, s_in, fin, cs, initial_state is not None, w)
    return o, ctx


def backward(dO: torch.Tensor, ctx: Context, d_final_state: Optional[torch.Tensor] = None,
             want_intermediates: bool = False, grad_dtype: Optional[torch.dtype] = None):
    """(dq, dk, dv, dg, d_initial_state); dg is None without decay, d_initial_state
    None with packed sequences. With input weights (``w`` given to ``forward``) a
    sixth element dw [B,T,H] fp32 follows, and ``grad_dtype=torch.float32`` gives dq,
    dk, dv in fp32 (bf16 inputs, scalar decay). dq and dk are per head [B,T,H,dk]
    also where q and k are shared by groups of heads."""
    if ctx.chunk_states is None:
        raise CplaError(1, "forward was run with save_for_backward=False")
    B, T, _, dk = ctx.q.shape
    H, dv = ctx.v.shape[2], ctx.v.shape[-1]
    _expect("dO", dO, (B, T, H, dv), ctx.q.dtype, ctx.q.device)
    _expect("d_final_state", d_final_state, (B, H, dk, dv), torch.float32, ctx.q.device, optional=True)
    L = _lib.lib()
    p = ctx.problem
    P = p.num_shards
    dev = dO.device
    W = L.cpla_summary_width(ctypes.byref(p))
    bsum = torch.empty((P, B, H, W), device=dev, dtype=torch.float32)
    s_out = torch.empty((P, B, H, dk, dv), device=dev, dtype=torch.float32)
    gdt = ctx.q.dtype if grad_dtype is None else grad_dtype
    if gdt != ctx.q.dtype and ctx.w is None:
        raise CplaError(3, "fp32 gradients are available through the weighted backward only")
    dq = torch.empty((B, T, H, dk), device=dev, dtype=gdt)
    dk_ = torch.empty((B, T, H, dk), device=dev, dtype=gdt)
    dv_ = torch.empty(ctx.v.shape, device=dev, dtype=gdt)
    dg = None if ctx.g is None else torch.empty_like(ctx.g)
    dS0 = None
    if ctx.packed is None:
        dS0 = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
    pk = ctypes.byref(ctx.packed.c()) if ctx.packed is not None else None
    st = _stream()
    check(L.cp_backward_prepare(ctypes.byref(p), pk, _ptr(ctx.q), _ptr(ctx.g), _ptr(dO), _ptr(bsum), st))
    if ctx.w is None:
        check(L.cp_backward_apply(ctypes.byref(p), pk, _ptr(ctx.q), _ptr(ctx.k), _ptr(ctx.v), _ptr(ctx.g),
                                  _ptr(dO), _ptr(ctx.chunk_states), _ptr(bsum), _ptr(d_final_state), _ptr(dq),
                                  _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(s_out), _ptr(dS0), st))
        res = (dq, dk_, dv_, dg, dS0)
    else:
        dw = torch.empty_like(ctx.w)
        check(L.cp_backward_apply_weighted(ctypes.byref(p), pk, _ptr(ctx.q), _ptr(ctx.k), _ptr(ctx.v), _ptr(ctx.g),
                                           _ptr(ctx.w), _ptr(dO), _ptr(ctx.chunk_states), _ptr(bsum),
                                           _ptr(d_final_state), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(dw),
                                           _ptr(s_out), _ptr(dS0), _DTYPE[gdt], st))
        res = (dq, dk_, dv_, dg, dS0, dw)
    if want_intermediates:
        return res, {"bwd_summary": bsum, "shard_out_grad": s_out}
    return res


class ChunkwiseLinearAttention(torch.autograd.Function):
    """Autograd adapter: o = f(q, k, v, g, S_init) with shards simulated on one GPU."""

    @staticmethod
    def forward(fctx, q, k, v, g, initial_state, num_shards, cu_seqlens):
        if q.dim() == 4 and v.dim() == 4 and q.shape[2] != v.shape[2]:
            raise CplaError(2, "the autograd adapter takes q and k per head (their gradients are per head)")
        o, c = forward(q, k, v, g, num_shards=num_shards, initial_state=initial_state, cu_seqlens=cu_seqlens)
        fctx.cpla = c
        return o

    @staticmethod
    def backward(fctx, dO):
        dq, dk, dv, dg, dS0 = backward(dO.contiguous(), fctx.cpla)
        if not fctx.cpla.has_initial_state:
            dS0 = None
        return dq, dk, dv, dg, dS0, None, None


def chunkwise_linear_attention(q, k, v, g=None, initial_state=None, *, num_shards: int = 1, cu_seqlens=None):
    return ChunkwiseLinearAttention.apply(q, k, v, g, initial_state, num_shards, cu_seqlens)


# ---- Mamba2 (SSD) parametrisation ---------------------------------------------------------
# Mamba2's selective state space runs through the weighted scalar-decay path:
# cpla_ssd_inputs writes g = A dt; the CP calls read q = C and k = B in place (one
# head of them per group of heads) and take v = x and input weights w = dt;
# cpla_ssd_input_grads takes the gradients back (see include/cpla.h). dx is the dv
# of the CP backward.

@dataclasses.dataclass
class SsdContext:
    problem: SsdProblem
    dt: torch.Tensor
    A: torch.Tensor
    la: Context


def _ssd_problem(x, B) -> SsdProblem:
    Bt, T, H, P = x.shape
    if x.dtype not in _DTYPE:
        raise CplaError(3, f"dtype {x.dtype} unsupported")
    return SsdProblem(Bt, T, H, B.shape[2], B.shape[3], P, _DTYPE[x.dtype])


def ssd_forward(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, *,
                num_shards: int, initial_state: Optional[torch.Tensor] = None, cu_seqlens=None,
                packed: Optional[PackedMeta] = None):
    """y [Bt,T,H,P] (dtype of x) and an SsdContext for ``ssd_backward``. x [Bt,T,H,P];
    dt [Bt,T,H] and A [H] fp32; B, C [Bt,T,G,N] like x; initial_state [Bt,H,N,P] fp32."""
    if not torch.is_tensor(x) or x.dim() != 4 or not torch.is_tensor(B) or B.dim() != 4:
        raise CplaError(2, "x and B must be [Bt,T,H,P] and [Bt,T,G,N] tensors")
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _expect("x", x, (Bt, T, H, P), x.dtype)
    _expect("dt", dt, (Bt, T, H), torch.float32)
    _expect("A", A, (H,), torch.float32)
    _expect("B", B, (Bt, T, G, N), x.dtype)
    _expect("C", C, (Bt, T, G, N), x.dtype)
    _expect("initial_state", initial_state, (Bt, H, N, P), torch.float32, optional=True)
    _expect_gpu("x", dict(x=x, dt=dt, A=A, B=B, C=C, initial_state=initial_state))
    sp = _ssd_problem(x, B)
    g = torch.empty(dt.shape, device=x.device, dtype=torch.float32)
    check(_lib.lib().cpla_ssd_inputs(ctypes.byref(sp), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), None, None,
                                     _ptr(g), _stream()))
    y, la = forward(C, B, x, g, num_shards=num_shards, initial_state=initial_state, cu_seqlens=cu_seqlens,
                    packed=packed, w=dt)
    return y, SsdContext(sp, dt, A, la)


def ssd_backward(dy: torch.Tensor, ctx: SsdContext, d_final_state: Optional[torch.Tensor] = None):
    """(dx, d_dt, dA, dB, dC, d_initial_state); d_initial_state is None with packed
    sequences."""
    _expect("dy", dy, tuple(ctx.la.v.shape), ctx.la.v.dtype, ctx.la.v.device)
    dq, dk, dv, dg, dS0, dw = backward(dy, ctx.la, d_final_state, grad_dtype=torch.float32)
    sp = ctx.problem
    dev = dy.device
    xdt = ctx.la.v.dtype
    dx = torch.empty(ctx.la.v.shape, device=dev, dtype=xdt)
    ddt = torch.empty(ctx.dt.shape, device=dev, dtype=torch.float32)
    dA = torch.empty(ctx.A.shape, device=dev, dtype=torch.float32)
    Bshape = (sp.B, sp.T, sp.G, sp.N)
    dB = torch.empty(Bshape, device=dev, dtype=xdt)
    dC = torch.empty(Bshape, device=dev, dtype=xdt)
    check(_lib.lib().cpla_ssd_input_grads(ctypes.byref(sp), _ptr(ctx.dt), _ptr(ctx.A), _ptr(dq), _ptr(dk),
                                          _ptr(dv), _ptr(dg), _ptr(dw), _ptr(dx), _ptr(ddt), _ptr(dA), _ptr(dB),
                                          _ptr(dC), _stream()))
    return dx, ddt, dA, dB, dC, dS0


class Mamba2SSD(torch.autograd.Function):
    """Autograd adapter: y = SSD(x, dt, A, B, C, h_init) with shards simulated on one GPU."""

    @staticmethod
    def forward(fctx, x, dt, A, B, C, initial_state, num_shards, cu_seqlens):
        y, c = ssd_forward(x, dt, A, B, C, num_shards=num_shards, initial_state=initial_state,
                           cu_seqlens=cu_seqlens)
        fctx.cpla = c
        return y

    @staticmethod
    def backward(fctx, dy):
        dx, ddt, dA, dB, dC, dS0 = ssd_backward(dy.contiguous(), fctx.cpla)
        if not fctx.cpla.la.has_initial_state:
            dS0 = None
        return dx, ddt, dA, dB, dC, dS0, None, None


def mamba2_ssd(x, dt, A, B, C, initial_state=None, *, num_shards: int = 1, cu_seqlens=None):
    return Mamba2SSD.apply(x, dt, A, B, C, initial_state, num_shards, cu_seqlens)


# ---- the gated delta rule (dense transition) ---------------------------------------------

@dataclasses.dataclass
class DeltaContext:
    problem: Problem
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    packed: Optional[PackedMeta]
    fwd_summary: torch.Tensor
    shard_in_state: torch.Tensor
    final_state: torch.Tensor
    workspace: torch.Tensor             # the local context of the four calls (fp32 scratch)
    has_initial_state: bool


def delta_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, *,
                  num_shards: int, initial_state: Optional[torch.Tensor] = None, cu_seqlens=None,
                  packed: Optional[PackedMeta] = None):
    """Gated delta rule o [B,T,H,d] and a DeltaContext: S_t = exp(g_t)(I - beta_t k_t k_t^T) S_{t-1}
    + beta_t k_t v_t^T, o_t = S_t^T q_t; g, beta [B,T,H] fp32."""
    if not torch.is_tensor(q) or q.dim() != 4 or not torch.is_tensor(v) or v.dim() != 4:
        raise CplaError(2, "q and v must be [B,T,H,d] tensors")
    if q.dtype not in _DTYPE:
        raise CplaError(3, f"dtype {q.dtype} unsupported")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _expect("q", q, (B, T, H, dk), q.dtype)
    _expect("k", k, (B, T, H, dk), q.dtype)
    _expect("v", v, (B, T, H, dv), q.dtype)
    _expect("g", g, (B, T, H), torch.float32)
    _expect("beta", beta, (B, T, H), torch.float32)
    _expect("initial_state", initial_state, (B, H, dk, dv), torch.float32, optional=True)
    _expect_gpu("q", dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=initial_state))
    _check_packed(packed, B, T, num_shards, q.device)
    p = make_problem(q, v, num_shards, _lib.DECAY_DELTA)
    if cu_seqlens is not None and packed is None:
        packed = packed_meta(cu_seqlens, q.shape[1], num_shards, q.device, q.shape[0])
    L = _lib.lib()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    nb = L.cpla_delta_workspace_bytes(ctypes.byref(p))
    if nb < 0:
        check(L.cp_forward_prepare_delta(ctypes.byref(p), None, None, None, None, None, None, None, None))
    dev = q.device
    W = L.cpla_summary_width(ctypes.byref(p))
    ws = torch.empty((nb // 4,), device=dev, dtype=torch.float32)
    fsum = torch.empty((num_shards, B, H, W), device=dev, dtype=torch.float32)
    s_in = torch.empty((num_shards, B, H, dk, dv), device=dev, dtype=torch.float32)
    fin = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
    o = torch.empty(v.shape, device=dev, dtype=q.dtype)
    pk = ctypes.byref(packed.c()) if packed is not None else None
    st = _stream()
    check(L.cp_forward_prepare_delta(ctypes.byref(p), pk, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(fsum),
                                     _ptr(ws), st))
    check(L.cp_forward_apply_delta(ctypes.byref(p), pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(fsum),
                                   _ptr(initial_state), _ptr(o), _ptr(s_in), _ptr(fin), _ptr(ws), st))
    return o, DeltaContext(p, q, k, v, g, beta, packed, fsum, s_in, fin, ws, initial_state is not None)


def delta_backward(dO: torch.Tensor, ctx: DeltaContext, d_final_state: Optional[torch.Tensor] = None,
                   want_intermediates: bool = False):
    """(dq, dk, dv, dg, dbeta, d_initial_state); d_initial_state is None with packed sequences."""
    B, T, H, dk = ctx.q.shape
    dv = ctx.v.shape[-1]
    _expect("dO", dO, (B, T, H, dv), ctx.q.dtype, ctx.q.device)
    _expect("d_final_state", d_final_state, (B, H, dk, dv), torch.float32, ctx.q.device, optional=True)
    L = _lib.lib()
    p = ctx.problem
    P = p.num_shards
    dev = dO.device
    W = L.cpla_summary_width(ctypes.byref(p))
    bsum = torch.empty((P, B, H, W), device=dev, dtype=torch.float32)
    s_out = torch.empty((P, B, H, dk, dv), device=dev, dtype=torch.float32)
    dq, dk_, dv_ = torch.empty_like(ctx.q), torch.empty_like(ctx.k), torch.empty_like(ctx.v)
    dg, db = torch.empty_like(ctx.g), torch.empty_like(ctx.beta)
    dS0 = None if ctx.packed is not None else torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
    pk = ctypes.byref(ctx.packed.c()) if ctx.packed is not None else None
    st = _stream()
    check(L.cp_backward_prepare_delta(ctypes.byref(p), pk, _ptr(ctx.q), _ptr(ctx.k), _ptr(ctx.g), _ptr(ctx.beta),
                                      _ptr(dO), _ptr(ctx.fwd_summary), _ptr(bsum), _ptr(ctx.workspace), st))
    check(L.cp_backward_apply_delta(ctypes.byref(p), pk, _ptr(ctx.q), _ptr(ctx.k), _ptr(ctx.v), _ptr(ctx.g),
                                    _ptr(ctx.beta), _ptr(dO), _ptr(bsum), _ptr(d_final_state), _ptr(dq), _ptr(dk_),
                                    _ptr(dv_), _ptr(dg), _ptr(db), _ptr(s_out), _ptr(dS0), _ptr(ctx.workspace), st))
    res = (dq, dk_, dv_, dg, db, dS0)
    if want_intermediates:
        return res, {"bwd_summary": bsum, "shard_out_grad": s_out}
    return res


class GatedDeltaRule(torch.autograd.Function):
    """Autograd adapter for the gated delta rule, shards simulated on one GPU."""

    @staticmethod
    def forward(fctx, q, k, v, g, beta, initial_state, num_shards, cu_seqlens):
        o, c = delta_forward(q, k, v, g, beta, num_shards=num_shards, initial_state=initial_state,
                             cu_seqlens=cu_seqlens)
        fctx.cpla = c
        return o

    @staticmethod
    def backward(fctx, dO):
        dq, dk, dv, dg, db, dS0 = delta_backward(dO.contiguous(), fctx.cpla)
        if not fctx.cpla.has_initial_state:
            dS0 = None
        return dq, dk, dv, dg, db, dS0, None, None


def gated_delta_rule(q, k, v, g, beta, initial_state=None, *, num_shards: int = 1, cu_seqlens=None):
    return GatedDeltaRule.apply(q, k, v, g, beta, initial_state, num_shards, cu_seqlens)
