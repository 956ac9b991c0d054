"""The chunk algebra of gated linear attention, in plain fp64 (oracle; test use only).

This is NOT the definition (that is ``oracle.recurrence``); it writes out the
chunkwise form that a "chunkwise" CP backend (Megatron-Core page
``core.ssm.context_parallel.chunkwise``, module docstring and
``LinearAttentionCPBackend``) evaluates, so that tests can check that algebra
against the per-token recurrence at several chunk lengths.

Inside one chunk with tokens i = 0..n-1, incoming state S0 and log-decays g:

* Gam_i = sum_{s<=i} g_s (per key dim; inclusive, from the chunk start);
* seg_i = number of packed-sequence starts at chunk positions <= i
  (tokens with seg 0 still see S0);
* D_ij[d] = [i >= j][seg_i == seg_j] exp(Gam_i[d] - Gam_j[d]);
* o_i = sum_j sum_d q_i[d] k_j[d] D_ij[d] v_j + [seg_i == 0] S0^T (q_i * exp(Gam_i));
* S_end = [seg_last == 0] diag(exp(Gam_last)) S0
          + sum_{j: seg_j == seg_last} diag(exp(Gam_last - Gam_j)) k_j v_j^T.

Backward with dSC = gradient w.r.t. S_end from later tokens, X_i = S0 dO_i and
Y_j = dSC v_j:

* dq_i = [seg_i == 0] exp(Gam_i) * X_i + sum_j D_ij * k_j (dO_i . v_j);
* dk_j = sum_i D_ij * q_i (dO_i . v_j) + [seg_j == seg_last] exp(Gam_last - Gam_j) * Y_j;
* dv_j = sum_i (sum_d D_ij q_i k_j) dO_i + [seg_j == seg_last] dSC^T (k_j * exp(Gam_last - Gam_j));
* dS0 = [seg_last == 0] diag(exp(Gam_last)) dSC + sum_{i: seg_i == 0} diag(exp(Gam_i)) q_i dO_i^T;
* dg_t = a_t * rowsum(dS_t * S_{t-1}) split into four terms that never cancel
  each other:
    T1 = [seg_t == 0] sum_{i >= t, seg_i == 0} exp(Gam_i) q_i * X_i
    T2 = sum_{i >= t > j, same sequence} exp(Gam_i - Gam_j) q_i * k_j (dO_i . v_j)
    T3 = [seg_t == 0][seg_last == 0] exp(Gam_last) * rowsum(dSC * S0)
    T4 = [seg_t == seg_last] sum_{j < t, seg_j == seg_t} exp(Gam_last - Gam_j) k_j * Y_j
  and dg_t = 0 where t starts a sequence.
"""
from __future__ import annotations

import numpy as np

from . import recurrence as rec


def _chunk_terms(g_rows, resets, t0, t1):
    gc = g_rows[:, t0:t1]                               # [R,n,dk] log-decay
    Gam = np.cumsum(gc, axis=1)
    seg = np.cumsum(resets[t0:t1].astype(np.int64))
    n = t1 - t0
    same = (seg[:, None] == seg[None, :]) & (np.arange(n)[:, None] >= np.arange(n)[None, :])
    D = np.exp(Gam[:, :, None, :] - Gam[:, None, :, :]) * same[None, :, :, None]  # [R,i,j,dk]
    return Gam, seg, D


def _log_decay_rows(g, decay, R, T, dk):
    if decay == "none":
        return np.zeros((R, T, dk))
    gr = rec.to_rows(rec._np(g))
    if decay == "scalar":
        return np.repeat(gr[:, :, None], dk, axis=2)
    return gr


def forward(q, k, v, g=None, decay="none", initial_state=None, seq_idx=None, chunk=64):
    q, k, v = rec._np(q), rec._np(k), rec._np(v)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    R = B * H
    qr, kr, vr = rec.to_rows(q), rec.to_rows(k), rec.to_rows(v)
    lg = _log_decay_rows(g, decay, R, T, dk)
    if seq_idx is not None and np.ndim(seq_idx) != 1:
        raise ValueError("the chunked form takes one packing shared by the batch ([T] seq_idx)")
    resets = rec.starts_from_seq_idx(seq_idx, T)
    S = np.zeros((R, dk, dv)) if initial_state is None else rec._np(initial_state).reshape(R, dk, dv).copy()
    o = np.zeros((R, T, dv))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        Gam, seg, D = _chunk_terms(lg, resets, t0, t1)
        qc, kc, vc = qr[:, t0:t1], kr[:, t0:t1], vr[:, t0:t1]
        A = np.einsum("rid,rjd,rijd->rij", qc, kc, D)
        o[:, t0:t1] = np.einsum("rij,rjv->riv", A, vc)
        live = (seg == 0).astype(np.float64)
        o[:, t0:t1] += live[None, :, None] * np.einsum("rid,rdv->riv", qc * np.exp(Gam), S)
        last = seg[-1]
        w = np.exp(Gam[:, -1:, :] - Gam) * (seg == last)[None, :, None]
        S = (S * np.exp(Gam[:, -1, :])[:, :, None] if last == 0 else 0.0) + np.einsum("rjd,rjv->rdv", kc * w, vc)
    return rec.from_rows(o, B, H), S.reshape(B, H, dk, dv)


def backward(q, k, v, g=None, decay="none", dO=None, initial_state=None, seq_idx=None,
             d_final_state=None, chunk=64):
    q, k, v = rec._np(q), rec._np(k), rec._np(v)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    R = B * H
    qr, kr, vr, dOr = rec.to_rows(q), rec.to_rows(k), rec.to_rows(v), rec.to_rows(rec._np(dO))
    lg = _log_decay_rows(g, decay, R, T, dk)
    if seq_idx is not None and np.ndim(seq_idx) != 1:
        raise ValueError("the chunked form takes one packing shared by the batch ([T] seq_idx)")
    resets = rec.starts_from_seq_idx(seq_idx, T)
    # forward pass: state entering every chunk
    S = np.zeros((R, dk, dv)) if initial_state is None else rec._np(initial_state).reshape(R, dk, dv).copy()
    starts = list(range(0, T, chunk))
    S0s = []
    for t0 in starts:
        t1 = min(T, t0 + chunk)
        S0s.append(S.copy())
        Gam, seg, _ = _chunk_terms(lg, resets, t0, t1)
        last = seg[-1]
        w = np.exp(Gam[:, -1:, :] - Gam) * (seg == last)[None, :, None]
        S = (S * np.exp(Gam[:, -1, :])[:, :, None] if last == 0 else 0.0) + \
            np.einsum("rjd,rjv->rdv", kr[:, t0:t1] * w, vr[:, t0:t1])
    dSC = np.zeros((R, dk, dv)) if d_final_state is None else rec._np(d_final_state).reshape(R, dk, dv).copy()
    dq = np.zeros((R, T, dk))
    dkk = np.zeros((R, T, dk))
    dvv = np.zeros((R, T, dv))
    dg = np.zeros((R, T, dk))
    for ci in range(len(starts) - 1, -1, -1):
        t0 = starts[ci]
        t1 = min(T, t0 + chunk)
        n = t1 - t0
        S0 = S0s[ci]
        Gam, seg, D = _chunk_terms(lg, resets, t0, t1)
        qc, kc, vc, dOc = qr[:, t0:t1], kr[:, t0:t1], vr[:, t0:t1], dOr[:, t0:t1]
        last = seg[-1]
        live = (seg == 0)
        tail = (seg == last)
        dA = np.einsum("riv,rjv->rij", dOc, vc)                     # dO_i . v_j
        X = np.einsum("rdv,riv->rid", S0, dOc)                      # S0 dO_i
        Y = np.einsum("rdv,rjv->rjd", dSC, vc)                      # dSC v_j
        eG = np.exp(Gam)
        eL = np.exp(Gam[:, -1:, :] - Gam)                           # exp(Gam_last - Gam_j)
        dq[:, t0:t1] = live[None, :, None] * eG * X + np.einsum("rij,rijd,rjd->rid", dA, D, kc)
        dkk[:, t0:t1] = np.einsum("rij,rijd,rid->rjd", dA, D, qc) + tail[None, :, None] * eL * Y
        A = np.einsum("rid,rjd,rijd->rij", qc, kc, D)
        dvv[:, t0:t1] = np.einsum("rij,riv->rjv", A, dOc) + \
            tail[None, :, None] * np.einsum("rjd,rdv->rjv", kc * eL, dSC)
        # dg in four non-cancelling terms
        T1 = np.zeros((R, n, dk))
        T2 = np.zeros((R, n, dk))
        T4 = np.zeros((R, n, dk))
        u1 = live[None, :, None] * eG * qc * X
        u4 = tail[None, :, None] * eL * kc * Y
        W = np.einsum("rijd,rid,rjd,rij->rijd", D, qc, kc, dA)
        W = W * (np.arange(n)[:, None] > np.arange(n)[None, :])[None, :, :, None]
        for t in range(n):
            T1[:, t] = u1[:, t:].sum(axis=1) if live[t] else 0.0
            T2[:, t] = W[:, t:, :t].sum(axis=(1, 2))
            if tail[t]:
                T4[:, t] = (u4[:, :t] * (seg[:t] == seg[t])[None, :, None]).sum(axis=1)
        T3 = (np.exp(Gam[:, -1, :]) * np.einsum("rdv,rdv->rd", dSC, S0))[:, None, :] * \
            (live & (last == 0))[None, :, None]
        dgc = T1 + T2 + T3 + T4
        dgc[:, resets[t0:t1]] = 0.0
        dg[:, t0:t1] = dgc
        dSC = (dSC * np.exp(Gam[:, -1, :])[:, :, None] if last == 0 else 0.0) + \
            np.einsum("rid,riv->rdv", qc * eG * live[None, :, None], dOc)
    out_dg = None
    if decay == "diag":
        out_dg = rec.from_rows(dg, B, H)
    elif decay == "scalar":
        out_dg = rec.from_rows(dg.sum(axis=2), B, H)
    return (rec.from_rows(dq, B, H), rec.from_rows(dkk, B, H), rec.from_rows(dvv, B, H), out_dg,
            dSC.reshape(B, H, dk, dv))
