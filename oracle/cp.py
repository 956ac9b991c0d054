"""The chunkwise CP method run through shard summaries, in fp64 (oracle; test use only).

Megatron-Core API page ``core.ssm.context_parallel.chunkwise``:

* ``cp_forward_prepare``: each contiguous shard's summary with ZERO incoming
  state: ``delta_S`` is the shard's final state started from zero, and ``M`` the
  map from the incoming state to the outgoing one, so that
  ``S_out = M S_in + delta_S`` (classes ``CPForward*Summary``);
* ``chunkwise_cp_forward`` / ``cp_forward_apply``: compose the selected causal
  prefix of summaries to get the shard's incoming state, then run the shard;
* ``cp_backward_prepare``: gamma = gradient w.r.t. the shard's incoming state
  with ZERO outgoing-state gradient, so ``dS_in = M^T dS_out + gamma``
  (classes ``CPBackward*Summary``);
* ``chunkwise_cp_backward`` / ``cp_backward_apply``: compose the selected
  reverse-causal suffix to get the gradient arriving at the shard's end, then
  finish the shard's input gradients.

M is diagonal here (a vector over the key dimension, one scalar, or 1), so
M^T = M. Readings: a shard that contains a packed-sequence start (its first
token included) forgets its incoming state, so its M is exactly 0; with packed
sequences rank r composes from zero over ranks [preceding_rank_start, r) and
the suffix from zero over (r, following_rank_stop); without packing the prefix
starts at rank 0 from S_init and the suffix ends at the last rank from
dS_final. Shards follow torch.chunk: ceil(T / P) tokens each, the last
non-empty one shorter when P does not divide T, and trailing shards empty when
the stream is too short (the graceful division the mixle page relies on, in
place of failing fast); an empty shard's map is the identity. With one
packing per batch row (``seq_idx`` [B, T]) the rows are independent problems,
each with its own rank slices, and are run one after the other.
"""
from __future__ import annotations

import numpy as np

from . import recurrence as rec
from .metadata import rank_slices


def _np(x):
    return rec._np(x)


def shard_bounds(T, P):
    """[start, end) of every shard: torch.chunk's split of T tokens into P parts."""
    if P <= 0 or T <= 0:
        raise ValueError("T and the number of shards must be positive")
    s = -(-T // P)
    return [(min(r * s, T), min((r + 1) * s, T)) for r in range(P)]


def _local_resets(global_starts, bounds):
    a, e = bounds
    return global_starts[a:e].copy()


def transitions(g, decay, B, T, H, dk, P, global_starts):
    """M_r for every shard: [P, B, H, m] with m = dk (diag) or 1."""
    m = dk if decay == "diag" else 1
    out = np.zeros((P, B, H, m))
    for r, (a, e) in enumerate(shard_bounds(T, P)):
        if global_starts[a:e].any():
            continue  # forgets its incoming state: M = 0
        if decay == "none":
            out[r] = 1.0
        elif decay == "scalar":
            out[r, :, :, 0] = np.exp(_np(g)[:, a:e, :].sum(axis=1))
        else:
            out[r] = np.exp(_np(g)[:, a:e, :, :].sum(axis=1))
    return out


def _shard(x, bounds):
    a, e = bounds
    return None if x is None else _np(x)[:, a:e]


def forward_summaries(k, v, g, decay, P, seq_idx=None):
    """(M [P,B,H,m], delta_S [P,B,H,dk,dv]) — each shard run alone from a zero state."""
    k, v = _np(k), _np(v)
    B, T, H, dk = k.shape
    dv = v.shape[3]
    starts = rec.starts_from_seq_idx(seq_idx, T)
    dS = np.zeros((P, B, H, dk, dv))
    for r, bd in enumerate(shard_bounds(T, P)):
        zq = np.zeros((B, bd[1] - bd[0], H, dk))
        _, fin = rec.forward(zq, _shard(k, bd), _shard(v, bd), _shard(g, bd), decay,
                             resets=_local_resets(starts, bd))
        dS[r] = fin
    return transitions(g, decay, B, T, H, dk, P, starts), dS


def backward_summaries(q, dO, g, decay, P, dv, seq_idx=None):
    """(M [P,B,H,m], gamma [P,B,H,dk,dv]) — each shard's adjoint with zero outgoing gradient."""
    q, dO = _np(q), _np(dO)
    B, T, H, dk = q.shape
    starts = rec.starts_from_seq_idx(seq_idx, T)
    gam = np.zeros((P, B, H, dk, dv))
    for r, bd in enumerate(shard_bounds(T, P)):
        L = bd[1] - bd[0]
        z = np.zeros((B, L, H, dk))
        zv = np.zeros((B, L, H, dv))
        *_, dS0 = rec.backward(_shard(q, bd), z, zv, _shard(g, bd), decay, _shard(dO, bd),
                               resets=_local_resets(starts, bd))
        gam[r] = dS0
    return transitions(g, decay, B, T, H, dk, P, starts), gam


def _scale(M, S):
    """diag(M) S for M [B,H,m] (m = dk or 1) and S [B,H,dk,dv]."""
    return M[..., :, None] * S


def slices(P, seq_idx=None):
    """Per-rank (prefix start, suffix stop). Unpacked: (0, P) for every rank."""
    if seq_idx is None:
        return np.zeros(P, dtype=np.int32), np.full(P, P, dtype=np.int32)
    return rank_slices(seq_idx, P)


def compose_prefix(M, dS, initial_state=None, prs=None):
    """Incoming state of every shard: [P,B,H,dk,dv], plus the stream's final state."""
    P = M.shape[0]
    zero = np.zeros_like(dS[0])
    if prs is None:
        prs = np.zeros(P, dtype=np.int32)
    S_in = np.zeros_like(dS)
    for r in range(P):
        S = _np(initial_state).copy() if (initial_state is not None and prs[r] == 0) else zero.copy()
        for j in range(int(prs[r]), r):
            S = _scale(M[j], S) + dS[j]
        S_in[r] = S
    final = _scale(M[P - 1], S_in[P - 1]) + dS[P - 1]
    return S_in, final


def compose_suffix(M, gam, d_final_state=None, frs=None):
    """Gradient arriving at the end of every shard: [P,B,H,dk,dv], plus dS_init."""
    P = M.shape[0]
    zero = np.zeros_like(gam[0])
    if frs is None:
        frs = np.full(P, P, dtype=np.int32)
    dS_out = np.zeros_like(gam)
    for r in range(P):
        dS = _np(d_final_state).copy() if (d_final_state is not None and frs[r] == P) else zero.copy()
        for j in range(int(frs[r]) - 1, r, -1):
            dS = _scale(M[j], dS) + gam[j]
        dS_out[r] = dS
    d_init = _scale(M[0], dS_out[0]) + gam[0]
    return dS_out, d_init


def _per_row(seq_idx):
    return seq_idx is not None and np.ndim(seq_idx) == 2


def _row(x, b):
    return None if x is None else _np(x)[b:b + 1]


def _stack(parts, shard_major):
    """Concatenate per-row results: batch axis 1 for the per-shard arrays named
    in ``shard_major``, axis 0 otherwise."""
    out = {}
    for key, first in parts[0].items():
        if first is None:
            out[key] = None
        elif isinstance(first, dict):
            out[key] = _stack([p[key] for p in parts], shard_major)
        else:
            out[key] = np.concatenate([p[key] for p in parts], axis=1 if key in shard_major else 0)
    return out


_SHARD_MAJOR = ("M", "delta_S", "S_in", "gamma", "dS_out")


def cp_forward(q, k, v, g, decay, P, initial_state=None, seq_idx=None):
    """The method end to end: prepare (summaries), compose, apply. Returns o,
    final state, and the intermediates (M, delta_S, S_in)."""
    q, k, v = _np(q), _np(k), _np(v)
    B, T, H, dk = q.shape
    if _per_row(seq_idx):
        return _stack([cp_forward(_row(q, b), _row(k, b), _row(v, b), _row(g, b), decay, P,
                                  _row(initial_state, b), np.asarray(seq_idx)[b]) for b in range(B)],
                      _SHARD_MAJOR)
    starts = rec.starts_from_seq_idx(seq_idx, T)
    M, dS = forward_summaries(k, v, g, decay, P, seq_idx)
    prs, _ = slices(P, seq_idx)
    S_in, final = compose_prefix(M, dS, initial_state, prs)
    o = np.zeros((B, T, H, v.shape[3]))
    for r, bd in enumerate(shard_bounds(T, P)):
        o_r, _ = rec.forward(_shard(q, bd), _shard(k, bd), _shard(v, bd), _shard(g, bd), decay,
                             initial_state=S_in[r], resets=_local_resets(starts, bd))
        o[:, bd[0]:bd[1]] = o_r
    return {"o": o, "final_state": final, "M": M, "delta_S": dS, "S_in": S_in}


def cp_backward(q, k, v, g, decay, dO, P, initial_state=None, seq_idx=None, d_final_state=None):
    """Backward through summaries: gamma, reverse-causal composition, local finish."""
    if _per_row(seq_idx):
        B = np.shape(q)[0]
        return _stack([cp_backward(_row(q, b), _row(k, b), _row(v, b), _row(g, b), decay, _row(dO, b), P,
                                   _row(initial_state, b), np.asarray(seq_idx)[b], _row(d_final_state, b))
                       for b in range(B)], _SHARD_MAJOR)
    fw = cp_forward(q, k, v, g, decay, P, initial_state, seq_idx)
    q, k, v, dO = _np(q), _np(k), _np(v), _np(dO)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    starts = rec.starts_from_seq_idx(seq_idx, T)
    M, gam = backward_summaries(q, dO, g, decay, P, dv, seq_idx)
    _, frs = slices(P, seq_idx)
    dS_out, d_init = compose_suffix(M, gam, d_final_state, frs)
    dq = np.zeros_like(q)
    dk_ = np.zeros_like(k)
    dv_ = np.zeros_like(v)
    dg = None if g is None else np.zeros_like(_np(g))
    for r, bd in enumerate(shard_bounds(T, P)):
        a, b, c, e, _ = rec.backward(_shard(q, bd), _shard(k, bd), _shard(v, bd), _shard(g, bd), decay,
                                     _shard(dO, bd), initial_state=fw["S_in"][r], d_final_state=dS_out[r],
                                     resets=_local_resets(starts, bd))
        dq[:, bd[0]:bd[1]] = a
        dk_[:, bd[0]:bd[1]] = b
        dv_[:, bd[0]:bd[1]] = c
        if dg is not None:
            dg[:, bd[0]:bd[1]] = e
    if seq_idx is not None:
        d_init = None
    return {"dq": dq, "dk": dk_, "dv": dv_, "dg": dg, "d_initial_state": d_init,
            "gamma": gam, "dS_out": dS_out, "M": M, "fwd": fw}
