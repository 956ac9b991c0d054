"""Pins for the gated delta rule oracle (oracle/delta.py): against things other
than the oracle itself.

* the product form S_t = (A_t ... A_0) S_init + sum_j (A_t ... A_{j+1}) beta_j k_j v_j^T
  with explicit d_k x d_k matrices (brute force, tiny T);
* special cases: beta = 0 (pure decay), and unit keys with beta = 1 and no decay,
  where reading the key just written returns its value exactly;
* central finite differences of a scalar loss, for every input (packed
  sequences, one packing or one per row, included);
* sharded (summaries with a dense M, composition) == unsharded, with uneven and
  empty shards, packed and per-row packed; the summaries against their
  definition (the shard's map applied to a random incoming state, and its
  adjoint);
* the chunkwise (WY) algebra the kernels use, written out here, against the
  per-token recurrence: forward and every gradient, with sequence starts inside
  chunks.
"""
import numpy as np
import pytest

from oracle import delta, metadata, recurrence as rec


def _rand(rng, B=2, T=9, H=2, dk=3, dv=2, init=False, unit_keys=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5 if init else None
    return q, k, v, g, beta, S0


def _seq(lengths):
    cu = np.concatenate([[0], np.cumsum(lengths)])
    return metadata.seq_idx_from_cu_seqlens(cu, int(cu[-1]))


def test_product_form_brute_force():
    rng = np.random.default_rng(1)
    q, k, v, g, beta, S0 = _rand(rng, T=6, init=True, unit_keys=False)
    o, fin = delta.forward(q, k, v, g, beta, initial_state=S0)
    B, T, H, dk = q.shape
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            A = [np.exp(g[b, t, h]) * (eye - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h])) for t in range(T)]
            for t in range(T):
                S = np.zeros((dk, v.shape[3]))
                P = eye.copy()
                for j in range(t, -1, -1):        # P = A_t ... A_{j+1}
                    S += P @ (beta[b, j, h] * np.outer(k[b, j, h], v[b, j, h]))
                    P = P @ A[j]
                S += P @ S0[b, h]
                np.testing.assert_allclose(o[b, t, h], S.T @ q[b, t, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(fin[b, h], S, rtol=1e-12, atol=1e-12)


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(2)
    q, k, v, g, beta, S0 = _rand(rng, init=True)
    o, fin = delta.forward(q, k, v, g, np.zeros_like(beta), initial_state=S0)
    Gam = np.cumsum(g, axis=1)
    want = np.exp(Gam)[..., None] * np.einsum("bhkv,bthk->bthv", S0, q)
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin, np.exp(Gam[:, -1])[..., None, None] * S0, rtol=1e-12, atol=1e-12)


def test_unit_keys_read_back_their_values():
    """beta = 1, no decay, |k| = 1: the write replaces what the state held along k,
    so querying with k_t returns v_t exactly."""
    rng = np.random.default_rng(3)
    _, k, v, _, _, S0 = _rand(rng, T=12, init=True)
    o, _ = delta.forward(k, k, v, np.zeros(k.shape[:3]), np.ones(k.shape[:3]), initial_state=S0)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("packed", [0, 1, 2])
def test_backward_finite_differences(packed):
    rng = np.random.default_rng(10 + packed)
    B = 1 if packed == 1 else 2
    q, k, v, g, beta, S0 = _rand(rng, B=B, T=8, init=packed == 0, unit_keys=False)
    seq = None
    if packed == 1:
        seq = _seq([3, 1, 4])
    elif packed == 2:
        seq = np.stack([_seq([3, 1, 4]), _seq([8])])
    Wo = rng.standard_normal((B, 8, 2, 2))
    Wf = rng.standard_normal((B, 2, 3, 2))

    def loss(q_, k_, v_, g_, b_, S_):
        o, fin = delta.forward(q_, k_, v_, g_, b_, initial_state=S_, seq_idx=seq)
        return float(np.sum(o * Wo) + np.sum(fin * Wf))

    got = delta.backward(q, k, v, g, beta, Wo, initial_state=S0, seq_idx=seq, d_final_state=Wf)
    args = [q, k, v, g, beta, S0]
    eps = 1e-6
    for i, ga in enumerate(got):
        if args[i] is None:
            continue
        num = np.zeros_like(args[i])
        it = np.nditer(args[i], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            hi = [a.copy() if a is not None else None for a in args]
            lo = [a.copy() if a is not None else None for a in args]
            hi[i][idx] += eps
            lo[i][idx] -= eps
            num[idx] = (loss(*hi) - loss(*lo)) / (2 * eps)
        np.testing.assert_allclose(ga, num, rtol=1e-6, atol=1e-7, err_msg=f"input {i}")


def test_summaries_follow_their_definition():
    """M delta_S: the shard run from a random S_in ends at M S_in + delta_S; its adjoint
    with an outgoing gradient G gives M^T G + gamma."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, _ = _rand(rng, B=1, T=10, dk=4, dv=3)
    P = 3
    M, dS = delta.forward_summaries(k, v, g, beta, P)
    dO = rng.standard_normal(v.shape)
    _, gam = delta.backward_summaries(q, k, g, beta, dO, P, 3)
    from oracle.cp import shard_bounds
    for r, (s, e) in enumerate(shard_bounds(10, P)):
        Sin = rng.standard_normal((1, 2, 4, 3))
        _, fin = delta.forward(q[:, s:e], k[:, s:e], v[:, s:e], g[:, s:e], beta[:, s:e], initial_state=Sin)
        np.testing.assert_allclose(fin, M[r] @ Sin + dS[r], rtol=1e-12, atol=1e-12)
        G = rng.standard_normal((1, 2, 4, 3))
        *_, dSin = delta.backward(q[:, s:e], k[:, s:e], v[:, s:e], g[:, s:e], beta[:, s:e], dO[:, s:e],
                                  initial_state=Sin, d_final_state=G)
        np.testing.assert_allclose(dSin, np.swapaxes(M[r], -1, -2) @ G + gam[r], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P,lengths", [(1, None), (3, None), (4, None), (16, None), (3, [5, 1, 9, 2, 3]),
                                       (4, [20]), (5, [2, 2, 2, 14])])
def test_sharded_equals_unsharded(P, lengths):
    rng = np.random.default_rng(20 + P)
    T = 20
    q, k, v, g, beta, S0 = _rand(rng, B=1 if lengths else 2, T=T, init=lengths is None)
    seq = None if lengths is None else _seq(lengths)
    dO = rng.standard_normal(v.shape)
    o, fin = delta.forward(q, k, v, g, beta, initial_state=S0, seq_idx=seq)
    want = delta.backward(q, k, v, g, beta, dO, initial_state=S0, seq_idx=seq)
    f = delta.cp_forward(q, k, v, g, beta, P, initial_state=S0, seq_idx=seq)
    np.testing.assert_allclose(f["o"], o, atol=1e-12)
    np.testing.assert_allclose(f["final_state"], fin, atol=1e-12)
    r = delta.cp_backward(q, k, v, g, beta, dO, P, initial_state=S0, seq_idx=seq)
    for name, w in zip(["dq", "dk", "dv", "dg", "dbeta"], want):
        np.testing.assert_allclose(r[name], w, atol=1e-11, err_msg=name)
    if seq is None and S0 is not None:
        np.testing.assert_allclose(r["d_initial_state"], want[5], atol=1e-11)


def test_sharded_per_row_packing():
    rng = np.random.default_rng(30)
    seq = np.stack([_seq([5, 1, 9, 2, 3]), _seq([20]), _seq([1, 19])])
    q, k, v, g, beta, _ = _rand(rng, B=3, T=20)
    dO = rng.standard_normal(v.shape)
    o, _ = delta.forward(q, k, v, g, beta, seq_idx=seq)
    want = delta.backward(q, k, v, g, beta, dO, seq_idx=seq)
    f = delta.cp_forward(q, k, v, g, beta, 6, seq_idx=seq)
    np.testing.assert_allclose(f["o"], o, atol=1e-12)
    r = delta.cp_backward(q, k, v, g, beta, dO, 6, seq_idx=seq)
    for name, w in zip(["dq", "dk", "dv", "dg", "dbeta"], want):
        np.testing.assert_allclose(r[name], w, atol=1e-11, err_msg=name)
    # rows with different packings: separate runs agree
    for b in range(3):
        ob, _ = delta.forward(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], beta[b:b + 1], seq_idx=seq[b])
        np.testing.assert_allclose(o[b:b + 1], ob, atol=1e-13)


# ---- the chunkwise (WY) algebra ------------------------------------------------------------

def _chunk_terms(g, starts, s0, s1):
    """Gamma (segment-local inclusive cumsum), live f (no start at or before i),
    sequence counts and the same-segment causal decay D (C x C)."""
    gg = g[s0:s1]
    st = starts[s0:s1]
    C = s1 - s0
    Gam = np.zeros(C)
    acc = 0.0
    for i in range(C):
        acc = gg[i] if st[i] else acc + gg[i]
        Gam[i] = acc
    cnt = np.cumsum(st)
    live = (cnt == 0).astype(float)
    same = (cnt[:, None] == cnt[None, :]) & (np.arange(C)[:, None] >= np.arange(C)[None, :])
    D = np.where(same, np.exp(np.where(same, Gam[:, None] - Gam[None, :], 0.0)), 0.0)
    tail = (cnt == cnt[-1]).astype(float)
    return Gam, live, D, tail, same


def _wy_forward_row(q, k, v, g, beta, starts, C, S):
    """One row (q, k [T, dk], v [T, dv], g, beta [T]) in chunks of C: the per-chunk
    solve X = (I + A)^{-1} [beta V | beta e^Gam live K], U = U~ - W S,
    O = live e^Gam Q S + (tril(Q K^T) . D) U, S <- live_last e^Gam_last S + K~^T U."""
    T = q.shape[0]
    o = np.zeros((T, v.shape[1]))
    states = []
    for s0 in range(0, T, C):
        s1 = min(T, s0 + C)
        Gam, live, D, tail, same = _chunk_terms(g, starts, s0, s1)
        K, V, Q, b = k[s0:s1], v[s0:s1], q[s0:s1], beta[s0:s1]
        A = np.tril(b[:, None] * (K @ K.T) * D, -1)
        X = np.linalg.solve(np.eye(s1 - s0) + A, np.concatenate(
            [b[:, None] * V, (b * np.exp(Gam) * live)[:, None] * K], axis=1))
        Ut, W = X[:, :V.shape[1]], X[:, V.shape[1]:]
        states.append(S.copy())
        U = Ut - W @ S
        o[s0:s1] = (live * np.exp(Gam))[:, None] * (Q @ S) + ((Q @ K.T) * D) @ U
        Kt = (tail * np.exp(Gam[-1] - Gam))[:, None] * K
        S = live[-1] * np.exp(Gam[-1]) * S + Kt.T @ U
    return o, S, states


def _wy_backward_row(q, k, v, g, beta, starts, C, states, dO, dS):
    """The adjoint of _wy_forward_row chunk by chunk (reverse), dS = gradient at the end."""
    T, dk = q.shape
    dv_ = v.shape[1]
    dq, dk_, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dgam = np.zeros(T)
    db = np.zeros(T)
    chunks = list(range(0, T, C))
    for ci in range(len(chunks) - 1, -1, -1):
        s0 = chunks[ci]
        s1 = min(T, s0 + C)
        S0 = states[ci]
        Gam, live, D, tail, same = _chunk_terms(g, starts, s0, s1)
        K, V, Q, b, dOc = k[s0:s1], v[s0:s1], q[s0:s1], beta[s0:s1], dO[s0:s1]
        L = s1 - s0
        A = np.tril(b[:, None] * (K @ K.T) * D, -1)
        Bv = b[:, None] * V
        Bk = (b * np.exp(Gam) * live)[:, None] * K
        IA = np.eye(L) + A
        X = np.linalg.solve(IA, np.concatenate([Bv, Bk], axis=1))
        Ut, W = X[:, :dv_], X[:, dv_:]
        U = Ut - W @ S0
        Pm = (Q @ K.T) * D
        el = np.exp(Gam[-1] - Gam) * tail
        Kt = el[:, None] * K
        Qf = (live * np.exp(Gam))[:, None] * Q
        # outputs and the state update, backwards
        dU = Pm.T @ dOc + Kt @ dS
        dS0 = Qf.T @ dOc + live[-1] * np.exp(Gam[-1]) * dS - W.T @ dU
        dX = np.concatenate([dU, -dU @ S0.T], axis=1)
        dB = np.linalg.solve(IA.T, dX)
        dBv, dBk = dB[:, :dv_], dB[:, dv_:]
        dA = np.tril(-(dB @ X.T), -1) * (D > 0)
        dPr = (dOc @ U.T) * D                       # gradient of the raw scores Q K^T
        dOS = dOc @ S0.T
        dq[s0:s1] = dPr @ K + (live * np.exp(Gam))[:, None] * dOS
        dAr = dA * D * b[:, None]                   # gradient of the raw K K^T entries
        dK = dPr.T @ Q + el[:, None] * (U @ dS.T) + dAr @ K + dAr.T @ K + \
            (b * np.exp(Gam) * live)[:, None] * dBk
        dk_[s0:s1] = dK
        dvv[s0:s1] = b[:, None] * dBv
        db[s0:s1] = np.sum(dA * D * (K @ K.T), axis=1) + np.sum(dBv * V, axis=1) + \
            np.exp(Gam) * live * np.sum(dBk * K, axis=1)
        # d Gamma: decays inside P and A (row minus column sums), e^Gam in Qf and Bk,
        # e^(Gam_last - Gam) in K~ and e^Gam_last in the carried state
        PA = dPr * (Q @ K.T)                        # dP . P (dPr already carries D)
        AA = dA * A
        dG = PA.sum(1) - PA.sum(0) + AA.sum(1) - AA.sum(0)
        dG += (live * np.exp(Gam)) * np.sum(Q * dOS, axis=1)
        dG += np.sum(dBk * Bk, axis=1)
        tk = np.sum((U @ dS.T) * Kt, axis=1)
        dG -= tk
        dG[-1] += tk.sum() + live[-1] * np.exp(Gam[-1]) * np.sum(dS * S0)
        dgam[s0:s1] = dG
        dS = dS0
    # g_t enters Gamma_i for i >= t in t's segment of its chunk
    dg = np.zeros(T)
    for s0 in chunks:
        s1 = min(T, s0 + C)
        acc = 0.0
        for i in range(s1 - 1, s0 - 1, -1):
            acc += dgam[i]
            dg[i] = acc
            if starts[i]:
                acc = 0.0
    return dq, dk_, dvv, dg, db, dS


@pytest.mark.parametrize("C,lengths", [(4, None), (5, [3, 9, 1, 7]), (8, [1, 1, 18]), (20, [6, 14])])
def test_wy_chunk_form_matches_recurrence(C, lengths):
    rng = np.random.default_rng(40 + C)
    T = 20
    q, k, v, g, beta, S0 = _rand(rng, B=1, H=1, T=T, dk=4, dv=3, init=lengths is None)
    seq = None if lengths is None else _seq(lengths)
    dO = rng.standard_normal(v.shape)
    dSf = rng.standard_normal((1, 1, 4, 3))
    o, fin = delta.forward(q, k, v, g, beta, initial_state=S0, seq_idx=seq)
    want = delta.backward(q, k, v, g, beta, dO, initial_state=S0, seq_idx=seq, d_final_state=dSf)
    starts = rec.starts_from_seq_idx(seq, T) if seq is not None else np.zeros(T, dtype=bool)
    S = np.zeros((4, 3)) if S0 is None else S0[0, 0]
    row = [x[0, :, 0] for x in (q, k, v, g, beta)]
    o_c, fin_c, states = _wy_forward_row(*row, starts, C, S)
    np.testing.assert_allclose(o_c, o[0, :, 0], atol=1e-12)
    np.testing.assert_allclose(fin_c, fin[0, 0], atol=1e-12)
    dq, dk, dv, dg, db, dS0 = _wy_backward_row(*row, starts, C, states, dO[0, :, 0], dSf[0, 0])
    for name, got, w in [("dq", dq, want[0]), ("dk", dk, want[1]), ("dv", dv, want[2]), ("dg", dg, want[3]),
                         ("dbeta", db, want[4])]:
        np.testing.assert_allclose(got, w[0, :, 0], atol=1e-11, err_msg=name)
    if seq is None:
        np.testing.assert_allclose(dS0, want[5][0, 0], atol=1e-11)
