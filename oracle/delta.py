"""Gated delta rule (a dense state transition) in fp64 (oracle; test use only).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The Megatron-Core page ``core.ssm.context_parallel.chunkwise`` states the shard
summaries for a general transition: ``S_out = M S_in + delta_S`` (classes
``CPForward*Summary``) and ``dS_in = M^T dS_out + gamma`` (classes
``CPBackward*Summary``), M being whatever linear map the shard applies to its
incoming state. The axolotl-ringmaster README (Status table) validates
gated-DeltaNet linear attention on that state passing. The diagonal decays of
``oracle.recurrence`` make M diagonal; the gated delta rule makes it a full
d_k x d_k matrix, and M^T a true transpose. Reading taken: the gated delta rule
in its usual form, with the state laid out [d_k, d_v] as elsewhere here and no
scaling of q (a caller folds any scale into q):

    S_{-1} = S_init (zero unless given);  S_{t-1} := 0 at a packed-sequence start
    A_t = a_t (I - beta_t k_t k_t^T),  a_t = exp(g_t)             (d_k x d_k)
    S_t = A_t S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t

g is one log-decay per (b, t, h) and beta one write strength per (b, t, h).
A shard's map is M = A_last ... A_first (zero when the shard holds a sequence
start, its first token included) and delta_S its final state from zero.

Adjoint (dS_t = dL/dS_t from tokens >= t; S'_{t-1} the state token t reads,
zero at a start):

    dS_t   = q_t dO_t^T + A_{t+1}^T dS_{t+1}   (second term dropped when t+1 starts)
    dq_t   = S_t dO_t
    dv_t   = beta_t dS_t^T k_t
    dk_t   = beta_t dS_t v_t - a_t beta_t (dS_t S'_{t-1}^T k_t + S'_{t-1} dS_t^T k_t)
    dbeta_t = k_t^T dS_t v_t - a_t (k_t^T dS_t)(S'_{t-1}^T k_t)
    dg_t   = a_t (<dS_t, S'_{t-1}> - beta_t (k_t^T dS_t)(S'_{t-1}^T k_t))
    dS_init = A_0^T dS_0

A_t is symmetric, so A_t^T dS = a_t (dS - beta_t k_t (k_t^T dS)). These are the
chain rule on the definition, written out plainly; tokens are a Python loop and
rows (b, h) are vectorised.
"""
from __future__ import annotations

import numpy as np

from . import recurrence as rec
from .cp import shard_bounds
from .metadata import rank_slices

CKPT = 64   # tokens between stored states when the adjoint recomputes S_t


def _np(x):
    return rec._np(x)


def _rows(q, k, v, g, beta):
    q, k, v = _np(q), _np(k), _np(v)
    B, T, H, dk = q.shape
    R = B * H
    a = np.exp(rec.to_rows(_np(g)))              # [R, T]
    bt = rec.to_rows(_np(beta))                  # [R, T]
    return q, k, v, B, T, H, dk, v.shape[3], R, a, bt


def _step(S, a, bt, k, v):
    """A_t S + beta_t k_t v_t^T for every row: S [R, dk, dv], k [R, dk], v [R, dv]."""
    kS = np.einsum("rk,rkv->rv", k, S)
    return a[:, None, None] * (S - bt[:, None, None] * k[:, :, None] * kS[:, None, :]) + \
        bt[:, None, None] * k[:, :, None] * v[:, None, :]


def forward(q, k, v, g, beta, initial_state=None, seq_idx=None, resets=None):
    """o [B,T,H,dv] and the final state [B,H,dk,dv], fp64. ``seq_idx`` [T] or [B, T]
    marks packed sequences; ``resets`` (bool [T] or [B, T]) may be given instead."""
    q, k, v, B, T, H, dk, dv, R, a, bt = _rows(q, k, v, g, beta)
    qr, kr, vr = rec.to_rows(q), rec.to_rows(k), rec.to_rows(v)
    rs = rec.resets_per_row(rec.starts_from_seq_idx(seq_idx, T) if resets is None else resets, B, H)
    S = np.zeros((R, dk, dv)) if initial_state is None else _np(initial_state).reshape(R, dk, dv).copy()
    o = np.empty((R, T, dv))
    for t in range(T):
        S = np.where(rs[:, t, None, None], 0.0, S)
        S = _step(S, a[:, t], bt[:, t], kr[:, t], vr[:, t])
        o[:, t] = np.einsum("rkv,rk->rv", S, qr[:, t])
    return rec.from_rows(o, B, H), S.reshape(B, H, dk, dv)


def backward(q, k, v, g, beta, dO, initial_state=None, seq_idx=None, d_final_state=None, resets=None):
    """(dq, dk, dv, dg, dbeta, dS_init), fp64; dS_init [B,H,dk,dv] (the gradient of
    the incoming state, whether or not one was given)."""
    q, k, v, B, T, H, dk, dv, R, a, bt = _rows(q, k, v, g, beta)
    qr, kr, vr = rec.to_rows(q), rec.to_rows(k), rec.to_rows(v)
    dOr = rec.to_rows(_np(dO))
    rs = rec.resets_per_row(rec.starts_from_seq_idx(seq_idx, T) if resets is None else resets, B, H)
    S0 = np.zeros((R, dk, dv)) if initial_state is None else _np(initial_state).reshape(R, dk, dv).copy()
    nblk = (T + CKPT - 1) // CKPT
    ck = np.empty((nblk, R, dk, dv))
    S = S0.copy()
    for t in range(T):
        if t % CKPT == 0:
            ck[t // CKPT] = S
        S = _step(np.where(rs[:, t, None, None], 0.0, S), a[:, t], bt[:, t], kr[:, t], vr[:, t])

    dq = np.empty((R, T, dk))
    dkk = np.empty((R, T, dk))
    dvv = np.empty((R, T, dv))
    dg = np.empty((R, T))
    db = np.empty((R, T))
    G = np.zeros((R, dk, dv)) if d_final_state is None else _np(d_final_state).reshape(R, dk, dv).copy()
    for blk in range(nblk - 1, -1, -1):
        t0, t1 = blk * CKPT, min(T, (blk + 1) * CKPT)
        prev, cur = [], []
        S = ck[blk].copy()
        for t in range(t0, t1):
            Sp = np.where(rs[:, t, None, None], 0.0, S)
            S = _step(Sp, a[:, t], bt[:, t], kr[:, t], vr[:, t])
            prev.append(Sp)
            cur.append(S)
        for t in range(t1 - 1, t0 - 1, -1):
            i = t - t0
            Sp, St = prev[i], cur[i]
            kt, vt, at, btt = kr[:, t], vr[:, t], a[:, t], bt[:, t]
            dS = G + qr[:, t, :, None] * dOr[:, t, None, :]
            dq[:, t] = np.einsum("rkv,rv->rk", St, dOr[:, t])
            kS = np.einsum("rk,rkv->rv", kt, Sp)         # S'^T k
            kdS = np.einsum("rk,rkv->rv", kt, dS)        # dS^T k
            dvv[:, t] = btt[:, None] * kdS
            dkk[:, t] = btt[:, None] * np.einsum("rkv,rv->rk", dS, vt) - (at * btt)[:, None] * (
                np.einsum("rkv,rv->rk", dS, kS) + np.einsum("rkv,rv->rk", Sp, kdS))
            kdSkS = np.einsum("rv,rv->r", kdS, kS)
            db[:, t] = np.einsum("rv,rv->r", kdS, vt) - at * kdSkS
            dg[:, t] = at * (np.einsum("rkv,rkv->r", dS, Sp) - btt * kdSkS)
            G = at[:, None, None] * (dS - btt[:, None, None] * kt[:, :, None] * kdS[:, None, :])
            G = np.where(rs[:, t, None, None], 0.0, G)
    fr = rec.from_rows
    return (fr(dq, B, H), fr(dkk, B, H), fr(dvv, B, H), fr(dg, B, H), fr(db, B, H),
            G.reshape(B, H, dk, dv))


# ---- shard summaries and their composition ------------------------------------------------

def transitions(k, g, beta, P, starts):
    """M_r = A_last ... A_first of every shard: [P, B, H, dk, dk] (0 with a start,
    the identity for an empty shard), by explicit d_k x d_k products."""
    k = _np(k)
    B, T, H, dk = k.shape
    a = np.exp(_np(g))
    bt = _np(beta)
    M = np.zeros((P, B, H, dk, dk))
    st = np.broadcast_to(np.asarray(starts, dtype=bool), (B, T))
    eye = np.eye(dk)
    for r, (s, e) in enumerate(shard_bounds(T, P)):
        for b in range(B):
            if st[b, s:e].any():
                continue
            for h in range(H):
                m = eye.copy()
                for t in range(s, e):
                    kt = k[b, t, h]
                    m = a[b, t, h] * (eye - bt[b, t, h] * np.outer(kt, kt)) @ m
                M[r, b, h] = m
    return M


def _shard(x, bd):
    return None if x is None else _np(x)[:, bd[0]:bd[1]]


def forward_summaries(k, v, g, beta, P, seq_idx=None):
    """(M [P,B,H,dk,dk], delta_S [P,B,H,dk,dv]): each shard run alone from zero."""
    k, v = _np(k), _np(v)
    B, T, H, dk = k.shape
    starts = rec.starts_from_seq_idx(seq_idx, T)
    dS = np.zeros((P, B, H, dk, v.shape[3]))
    for r, bd in enumerate(shard_bounds(T, P)):
        zq = np.zeros((B, bd[1] - bd[0], H, dk))
        _, fin = forward(zq, _shard(k, bd), _shard(v, bd), _shard(g, bd), _shard(beta, bd),
                         resets=starts[..., bd[0]:bd[1]])
        dS[r] = fin
    return transitions(k, g, beta, P, starts), dS


def backward_summaries(q, k, g, beta, dO, P, dv, seq_idx=None):
    """(M, gamma [P,B,H,dk,dv]): each shard's incoming-state gradient with a zero
    outgoing gradient (it does not depend on v: the map is affine in the state)."""
    q, dO = _np(q), _np(dO)
    B, T, H, dk = q.shape
    starts = rec.starts_from_seq_idx(seq_idx, T)
    gam = np.zeros((P, B, H, dk, dv))
    for r, bd in enumerate(shard_bounds(T, P)):
        L = bd[1] - bd[0]
        zv = np.zeros((B, L, H, dv))
        *_, dS0 = backward(_shard(q, bd), _shard(k, bd), zv, _shard(g, bd), _shard(beta, bd), _shard(dO, bd),
                           resets=starts[..., bd[0]:bd[1]])
        gam[r] = dS0
    return transitions(k, g, beta, P, starts), gam


def compose_prefix(M, dS, initial_state=None, prs=None):
    """Incoming state of every shard [P,B,H,dk,dv] (fold of S <- M_j S + delta_S_j
    over [prs_r, r)) and the stream's final state. ``prs`` is [P] (every row)."""
    P = M.shape[0]
    if prs is None:
        prs = np.zeros(P, dtype=np.int32)
    S_in = np.zeros_like(dS)
    for r in range(P):
        S = _np(initial_state).copy() if (initial_state is not None and prs[r] == 0) else np.zeros_like(dS[0])
        for j in range(int(prs[r]), r):
            S = M[j] @ S + dS[j]
        S_in[r] = S
    return S_in, M[P - 1] @ S_in[P - 1] + dS[P - 1]


def compose_suffix(M, gam, d_final_state=None, frs=None):
    """Gradient arriving at every shard's end (fold of dS <- M_j^T dS + gamma_j over
    (r, frs_r), backwards) and dS_init = M_0^T dS_out_0 + gamma_0."""
    P = M.shape[0]
    if frs is None:
        frs = np.full(P, P, dtype=np.int32)
    Mt = np.swapaxes(M, -1, -2)
    dS_out = np.zeros_like(gam)
    for r in range(P):
        dS = _np(d_final_state).copy() if (d_final_state is not None and frs[r] == P) else np.zeros_like(gam[0])
        for j in range(int(frs[r]) - 1, r, -1):
            dS = Mt[j] @ dS + gam[j]
        dS_out[r] = dS
    return dS_out, Mt[0] @ dS_out[0] + gam[0]


def _per_row(seq_idx):
    return seq_idx is not None and np.ndim(seq_idx) == 2


def _row(x, b):
    return None if x is None else _np(x)[b:b + 1]


def cp_forward(q, k, v, g, beta, P, initial_state=None, seq_idx=None):
    """The method end to end through summaries: o, final state, M, delta_S, S_in."""
    q, k, v = _np(q), _np(k), _np(v)
    B, T, H, dk = q.shape
    if _per_row(seq_idx):
        parts = [cp_forward(_row(q, b), _row(k, b), _row(v, b), _row(g, b), _row(beta, b), P,
                            _row(initial_state, b), np.asarray(seq_idx)[b]) for b in range(B)]
        return {n: np.concatenate([p[n] for p in parts], axis=1 if n in ("M", "delta_S", "S_in") else 0)
                for n in parts[0]}
    starts = rec.starts_from_seq_idx(seq_idx, T)
    M, dS = forward_summaries(k, v, g, beta, P, seq_idx)
    prs = np.zeros(P, dtype=np.int32) if seq_idx is None else rank_slices(seq_idx, P)[0]
    S_in, final = compose_prefix(M, dS, initial_state, prs)
    o = np.zeros((B, T, H, v.shape[3]))
    for r, bd in enumerate(shard_bounds(T, P)):
        o_r, _ = forward(_shard(q, bd), _shard(k, bd), _shard(v, bd), _shard(g, bd), _shard(beta, bd),
                         initial_state=S_in[r], resets=starts[bd[0]:bd[1]])
        o[:, bd[0]:bd[1]] = o_r
    return {"o": o, "final_state": final, "M": M, "delta_S": dS, "S_in": S_in}


def cp_backward(q, k, v, g, beta, dO, P, initial_state=None, seq_idx=None, d_final_state=None):
    """Backward through summaries: gamma, reverse composition, local finish. Returns
    dq, dk, dv, dg, dbeta, d_initial_state (None with packed sequences) and the
    intermediates (gamma, dS_out, M) and the forward's (under "fwd")."""
    q, k, v, dO = _np(q), _np(k), _np(v), _np(dO)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if _per_row(seq_idx):
        parts = [cp_backward(_row(q, b), _row(k, b), _row(v, b), _row(g, b), _row(beta, b), _row(dO, b), P,
                             _row(initial_state, b), np.asarray(seq_idx)[b], _row(d_final_state, b))
                 for b in range(B)]
        out = {}
        for n in parts[0]:
            if n == "fwd":
                out[n] = {m: np.concatenate([p[n][m] for p in parts], axis=1 if m in ("M", "delta_S", "S_in") else 0)
                          for m in parts[0][n]}
            elif parts[0][n] is None:
                out[n] = None
            else:
                out[n] = np.concatenate([p[n] for p in parts], axis=1 if n in ("gamma", "dS_out", "M") else 0)
        return out
    fw = cp_forward(q, k, v, g, beta, P, initial_state, seq_idx)
    starts = rec.starts_from_seq_idx(seq_idx, T)
    M, gam = backward_summaries(q, k, g, beta, dO, P, dv, seq_idx)
    frs = np.full(P, P, dtype=np.int32) if seq_idx is None else rank_slices(seq_idx, P)[1]
    dS_out, d_init = compose_suffix(M, gam, d_final_state, frs)
    outs = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros((B, T, H)), np.zeros((B, T, H))]
    for r, bd in enumerate(shard_bounds(T, P)):
        res = backward(_shard(q, bd), _shard(k, bd), _shard(v, bd), _shard(g, bd), _shard(beta, bd),
                       _shard(dO, bd), initial_state=fw["S_in"][r], d_final_state=dS_out[r],
                       resets=starts[bd[0]:bd[1]])
        for o_, x in zip(outs, res[:5]):
            o_[:, bd[0]:bd[1]] = x
    return {"dq": outs[0], "dk": outs[1], "dv": outs[2], "dg": outs[3], "dbeta": outs[4],
            "d_initial_state": None if seq_idx is not None else d_init,
            "gamma": gam, "dS_out": dS_out, "M": M, "fwd": fw}
