"""Mamba2 selective state space (SSD) in fp64, written in its own terms (oracle; test use only).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The axolotl-ringmaster README (Status table: "Mamba2 SSM CP ... + linear-attention
state-passing"; Layout: state_passing.py, an exact CP linear scan shared by
Mamba2 and linear attention) puts Mamba2 on the same context-parallel state
passing as linear attention, and the Megatron-Core chunkwise CP interfaces live
in its SSM module. This module states Mamba2's recurrence directly — it does not
go through the linear-attention oracle — so that a test can pin the mapping
between the two.

Per (b, h) with group gr = h // (H // G) sharing B and C, state h_t of shape
[N, P] (state size N, head dim P; N and P may differ):

    h_{-1} = h_init (zero unless given);  h_{t-1} := 0 at a packed-sequence start
    a_t = exp(dt_t * A_h)
    h_t = a_t h_{t-1} + dt_t * B_t x_t^T
    y_t = h_t^T C_t

Adjoint (dh_t = dL/dh_t from tokens >= t; zero after the last token unless a
final-state gradient is given):

    dh_t   = C_t dy_t^T + a_{t+1} dh_{t+1}      (second term dropped when t+1 starts)
    dC_t  += h_t dy_t
    dB_t  += dt_t * dh_t x_t
    dx_t   = dt_t * dh_t^T B_t
    da_t   = sum(dh_t * h_{t-1})                 (0 at a start)
    d_dt_t = sum_{n,p} dh_t[n,p] B_t[n] x_t[p] + da_t * a_t * A_h
    dA_h  += da_t * a_t * dt_t
    dh_init = a_0 dh_0

dB and dC sum over the heads of a group. Tokens are a Python loop; rows (b, h)
are vectorised.
"""
from __future__ import annotations

import numpy as np


def _np(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _starts(seq_idx, Bt, T):
    """[Bt, T] bool: True where a packed sequence starts after token 0. ``seq_idx``
    is [T] (one packing for every batch row) or [Bt, T] (one per row)."""
    st = np.zeros((Bt, T), dtype=bool)
    if seq_idx is not None:
        s = np.broadcast_to(np.asarray(seq_idx), (Bt, T))
        st[:, 1:] = s[:, 1:] != s[:, :-1]
    return st   # token 0 starts from h_init (zero in packed use)


def ssd_forward(x, dt, A, B, C, h_init=None, seq_idx=None):
    """y [Bt, T, H, P] and final state [Bt, H, N, P] (fp64)."""
    x, dt, A, B, C, h0 = (_np(t) for t in (x, dt, A, B, C, h_init))
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    grp = np.arange(H) // (H // G)
    st = _starts(seq_idx, Bt, T)
    h = np.zeros((Bt, H, N, P)) if h0 is None else h0.copy()
    y = np.zeros((Bt, T, H, P))
    for t in range(T):
        h = np.where(st[:, t, None, None, None], 0.0, h)
        a = np.exp(dt[:, t, :] * A[None, :])                       # [Bt, H]
        Bt_ = B[:, t, grp, :]                                      # [Bt, H, N]
        Ct_ = C[:, t, grp, :]
        h = a[:, :, None, None] * h + dt[:, t, :, None, None] * Bt_[:, :, :, None] * x[:, t, :, None, :]
        y[:, t] = np.einsum("bhnp,bhn->bhp", h, Ct_)
    return y, h


def ssd_backward(x, dt, A, B, C, dy, h_init=None, seq_idx=None, dh_final=None):
    """(dx, d_dt, dA, dB, dC, dh_init) in fp64; dh_init is None without h_init."""
    x, dt, A, B, C, dy, h0, dhf = (_np(t) for t in (x, dt, A, B, C, dy, h_init, dh_final))
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    grp = np.arange(H) // (H // G)
    st = _starts(seq_idx, Bt, T)
    a = np.exp(dt * A[None, None, :])                              # [Bt, T, H]
    # states h_{t-1} for every t (T is small in tests)
    hs = np.zeros((T + 1, Bt, H, N, P))
    hs[0] = 0.0 if h0 is None else h0
    for t in range(T):
        prev = np.where(st[:, t, None, None, None], 0.0, hs[t])
        hs[t + 1] = a[:, t, :, None, None] * prev + dt[:, t, :, None, None] * \
            B[:, t, grp, :][:, :, :, None] * x[:, t, :, None, :]
    dx = np.zeros_like(x)
    ddt = np.zeros_like(dt)
    dA = np.zeros(H)
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    dh = np.zeros((Bt, H, N, P)) if dhf is None else dhf.copy()
    for t in range(T - 1, -1, -1):
        Bt_ = B[:, t, grp, :]
        Ct_ = C[:, t, grp, :]
        dh = np.einsum("bhn,bhp->bhnp", Ct_, dy[:, t]) + dh
        np.add.at(dC, (slice(None), t, grp), np.einsum("bhnp,bhp->bhn", hs[t + 1], dy[:, t]))
        np.add.at(dB, (slice(None), t, grp), dt[:, t, :, None] * np.einsum("bhnp,bhp->bhn", dh, x[:, t]))
        dx[:, t] = dt[:, t, :, None] * np.einsum("bhnp,bhn->bhp", dh, Bt_)
        prev = np.where(st[:, t, None, None, None], 0.0, hs[t])
        da = np.einsum("bhnp,bhnp->bh", dh, prev)
        ddt[:, t] = np.einsum("bhnp,bhn,bhp->bh", dh, Bt_, x[:, t]) + da * a[:, t] * A[None, :]
        dA += np.sum(da * a[:, t] * dt[:, t], axis=0)
        dh = np.where(st[:, t, None, None, None], 0.0, a[:, t, :, None, None] * dh)
    dh0 = None if h0 is None else dh
    return dx, ddt, dA, dB, dC, dh0


def ssd_matrix_form(x, dt, A, B, C):
    """y from the quadratic form y_t = sum_{s<=t} (C_t . B_s) exp(A sum_{s<r<=t} dt_r) dt_s x_s
    (no initial state, no packing): O(T^2) brute force for tiny T."""
    x, dt, A, B, C = (_np(t) for t in (x, dt, A, B, C))
    Bt, T, H, P = x.shape
    G = B.shape[2]
    grp = np.arange(H) // (H // G)
    y = np.zeros((Bt, T, H, P))
    for b in range(Bt):
        for h in range(H):
            cs = np.concatenate([[0.0], np.cumsum(dt[b, :, h])])
            for t in range(T):
                for s in range(t + 1):
                    w = C[b, t, grp[h]] @ B[b, s, grp[h]] * np.exp(A[h] * (cs[t + 1] - cs[s + 1])) * dt[b, s, h]
                    y[b, t, h] += w * x[b, s, h]
    return y
