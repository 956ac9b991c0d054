"""Per-token gated linear-attention recurrence in fp64 (oracle; test use only).

Definition (one independent stream per (b, h) row):

    S_{-1} = S_init (zero unless given)
    if token t starts a packed sequence:  S_{t-1} := 0
    S_t = diag(a_t) S_{t-1} + k_t v_t^T,   a_t = exp(g_t)     (S_t is d_k x d_v)
    o_t = S_t^T q_t                                            (inclusive of t)

``g`` is absent (a_t = 1), one scalar per (b, t, h), or one value per key
dimension (b, t, h, d_k). This is the local computation of one contiguous shard
that the Megatron-Core page ``core.ssm.context_parallel.chunkwise`` delegates to
``LinearAttentionCPBackend``; composing shards is in ``oracle.cp``.

The adjoint is the same recurrence run backwards. With dS_t the gradient of the
loss with respect to S_t from tokens >= t:

    dS_t   = q_t dO_t^T + diag(a_{t+1}) dS_{t+1}   (second term dropped when
             t+1 starts a sequence; at t = T-1 it is dS_final, zero unless given)
    dq_t   = S_t dO_t
    dk_t   = dS_t v_t
    dv_t   = dS_t^T k_t
    dg_t   = a_t * rowsum(dS_t * S_{t-1})          (diagonal decay; summed over
             the key dimension for a scalar decay; 0 at a sequence start)
    dS_init = diag(a_0) dS_0

With a per-token input weight w (scalar decay; the recurrence becomes
S_t = diag(a_t) S_{t-1} + w_t k_t v_t^T) the same chain rule gives
dk_t = w_t dS_t v_t, dv_t = w_t dS_t^T k_t and dw_t = k_t^T dS_t v_t.

These are the chain rule applied to the definition above, written out plainly.
Everything is vectorised over rows only; the token loop is a Python loop.
"""
from __future__ import annotations

import numpy as np

CKPT = 64  # tokens between stored states when the adjoint recomputes S_t


def _np(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def to_rows(x):
    """[B, T, H, ...] -> [B*H, T, ...]."""
    B, T, H = x.shape[:3]
    return np.ascontiguousarray(np.moveaxis(x, 2, 1).reshape(B * H, T, *x.shape[3:]))


def from_rows(x, B, H):
    """[B*H, T, ...] -> [B, T, H, ...]."""
    T = x.shape[1]
    return np.ascontiguousarray(np.moveaxis(x.reshape(B, H, T, *x.shape[2:]), 1, 2))


def decay_rows(g, decay, R, T, dk):
    """Per-row, per-token, per-key-dim multiplicative decay a = exp(g): [R, T, dk]."""
    if decay == "none":
        return np.ones((R, T, dk))
    gr = to_rows(_np(g))
    if decay == "scalar":
        return np.repeat(np.exp(gr)[:, :, None], dk, axis=2)
    if decay == "diag":
        return np.exp(gr)
    raise ValueError(decay)


def starts_from_seq_idx(seq_idx, T):
    """Boolean [T] (or [B, T] for one packing per batch row): True where a packed
    sequence starts (token 0 always does)."""
    if seq_idx is None:
        return np.zeros(T, dtype=bool)
    s = np.asarray(seq_idx).astype(np.int64)
    st = np.zeros(s.shape, dtype=bool)
    st[..., 0] = True
    st[..., 1:] = s[..., 1:] != s[..., :-1]
    return st


def resets_per_row(resets, B, H):
    """[T] (shared by every batch row) or [B, T] -> [B*H, T], rows ordered as to_rows."""
    r = np.asarray(resets, dtype=bool)
    if r.ndim == 1:
        return np.broadcast_to(r, (B * H, r.shape[0]))
    return np.repeat(r, H, axis=0)


def run_forward_rows(q, k, v, a, resets, S0, wr=None):
    """Rows form. q, k: [R,T,dk]; v: [R,T,dv]; a: [R,T,dk]; resets: [R,T] bool; S0: [R,dk,dv];
    wr: per-token input weights [R,T] or None.

    Returns o [R,T,dv] and the final state [R,dk,dv]."""
    R, T, dk = q.shape
    S = S0.copy()
    o = np.empty((R, T, v.shape[2]))
    wr = np.ones((R, T)) if wr is None else wr
    for t in range(T):
        S = np.where(resets[:, t, None, None], 0.0, S)
        S = a[:, t, :, None] * S + wr[:, t, None, None] * k[:, t, :, None] * v[:, t, None, :]
        o[:, t] = np.einsum("rkv,rk->rv", S, q[:, t])
    return o, S


def run_backward_rows(q, k, v, a, resets, S0, dO, dSf, decay, wr=None):
    """Rows form of the adjoint. Returns dq, dk, dv, dg_rows [R,T,dk] (per key
    dim; summed by the caller for a scalar decay), dS_init [R,dk,dv] and dw [R,T]
    (the input-weight gradient; zeros without weights)."""
    R, T, dk = q.shape
    dv_ = v.shape[2]
    wr = np.ones((R, T)) if wr is None else wr
    dw = np.zeros((R, T))
    # forward sweep storing the state before every CKPT-th token
    nblk = (T + CKPT - 1) // CKPT
    ck = np.empty((nblk, R, dk, dv_))
    S = S0.copy()
    for t in range(T):
        if t % CKPT == 0:
            ck[t // CKPT] = S
        S = np.where(resets[:, t, None, None], 0.0, S)
        S = a[:, t, :, None] * S + wr[:, t, None, None] * k[:, t, :, None] * v[:, t, None, :]

    dq = np.empty((R, T, dk))
    dk_ = np.empty((R, T, dk))
    dvv = np.empty((R, T, dv_))
    dg = np.zeros((R, T, dk))
    G = dSf.copy()  # gradient w.r.t. S_t arriving from tokens > t
    for b in range(nblk - 1, -1, -1):
        t0, t1 = b * CKPT, min(T, (b + 1) * CKPT)
        prev = []   # S_{t-1} as seen by token t (zero after a reset)
        cur = []    # S_t
        S = ck[b].copy()
        for t in range(t0, t1):
            Sp = np.where(resets[:, t, None, None], 0.0, S)
            S = a[:, t, :, None] * Sp + wr[:, t, None, None] * k[:, t, :, None] * v[:, t, None, :]
            prev.append(Sp)
            cur.append(S)
        for t in range(t1 - 1, t0 - 1, -1):
            i = t - t0
            dS = G + q[:, t, :, None] * dO[:, t, None, :]
            dq[:, t] = np.einsum("rkv,rv->rk", cur[i], dO[:, t])
            dk_[:, t] = wr[:, t, None] * np.einsum("rkv,rv->rk", dS, v[:, t])
            dvv[:, t] = wr[:, t, None] * np.einsum("rkv,rk->rv", dS, k[:, t])
            dw[:, t] = np.einsum("rkv,rk,rv->r", dS, k[:, t], v[:, t])
            keep = ~resets[:, t]          # rows where token t continues its sequence
            if decay != "none":
                dg[:, t] = np.where(keep[:, None], a[:, t] * np.einsum("rkv,rkv->rk", dS, prev[i]), 0.0)
            G = np.where(keep[:, None, None], a[:, t, :, None] * dS, 0.0)
    return dq, dk_, dvv, dg, G, dw


def _prep(q, k, v, g, decay, initial_state, seq_idx, resets):
    q, k, v = _np(q), _np(k), _np(v)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    R = B * H
    if resets is None:
        resets = starts_from_seq_idx(seq_idx, T)
    resets = resets_per_row(resets, B, H)
    if initial_state is None:
        S0 = np.zeros((R, dk, dv))
    else:
        S0 = _np(initial_state).reshape(R, dk, dv).copy()
    a = decay_rows(g, decay, R, T, dk)
    return q, k, v, B, T, H, dk, dv, R, resets, S0, a


def forward(q, k, v, g=None, decay="none", initial_state=None, seq_idx=None, resets=None, w=None):
    """o [B,T,H,dv] and final state [B,H,dk,dv], fp64.

    ``seq_idx`` (int [T], or [B, T] for one packing per batch row) marks packed
    sequences: the state resets at each start, token 0 included. ``resets`` may
    be given instead (bool [T] or [B, T]) to reset only at chosen tokens, e.g. a
    shard whose first token continues a sequence.
    ``w`` [B,T,H]: per-token input weights (S_t = a_t S_{t-1} + w_t k_t v_t^T)."""
    q, k, v, B, T, H, dk, dv, R, resets, S0, a = _prep(q, k, v, g, decay, initial_state, seq_idx, resets)
    wr = None if w is None else to_rows(_np(w))
    o, S = run_forward_rows(to_rows(q), to_rows(k), to_rows(v), a, resets, S0, wr)
    return from_rows(o, B, H), S.reshape(B, H, dk, dv)


def backward(q, k, v, g=None, decay="none", dO=None, initial_state=None, seq_idx=None,
             d_final_state=None, resets=None, w=None):
    """dq, dk, dv (like q, k, v), dg (like g, or None), dS_init [B,H,dk,dv], all fp64;
    with input weights ``w`` [B,T,H], also dw [B,T,H] as a sixth element."""
    q, k, v, B, T, H, dk, dv, R, resets, S0, a = _prep(q, k, v, g, decay, initial_state, seq_idx, resets)
    dO = to_rows(_np(dO))
    dSf = np.zeros((R, dk, dv)) if d_final_state is None else _np(d_final_state).reshape(R, dk, dv).copy()
    wr = None if w is None else to_rows(_np(w))
    dq, dk_, dv_, dg, dS0, dw = run_backward_rows(to_rows(q), to_rows(k), to_rows(v), a, resets, S0, dO, dSf,
                                                  decay, wr)
    dgo = None
    if decay == "diag":
        dgo = from_rows(dg, B, H)
    elif decay == "scalar":
        dgo = from_rows(dg.sum(axis=2), B, H)
    res = (from_rows(dq, B, H), from_rows(dk_, B, H), from_rows(dv_, B, H), dgo, dS0.reshape(B, H, dk, dv))
    if w is not None:
        res = res + (from_rows(dw, B, H),)
    return res
