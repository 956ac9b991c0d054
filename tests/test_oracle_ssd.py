"""Pins for the Mamba2 (SSD) oracle: against things other than itself.

* the O(T^2) quadratic form of the selective state space (brute force, tiny T);
* central finite differences of a scalar loss, for every input (initial state
  and packed sequences, one packing for the batch or one per row, included);
* the linear-attention oracle, an independent implementation, under the map
  q = C[group], k = B[group], v = x, input weight w = dt, g = A dt — forward and,
  through the chain rule, backward;
* and the linear-attention oracle's input-weight gradients against central
  finite differences.
"""
import numpy as np
import pytest

from oracle import metadata, recurrence as rec, ssd


def _inputs(rng, Bt=2, T=9, H=4, G=2, N=3, init=False, P=None):
    P = N if P is None else P           # head dim of x and y; N is the state size
    x = rng.standard_normal((Bt, T, H, P))
    dt = np.log1p(np.exp(rng.standard_normal((Bt, T, H)) - 1.0))
    A = -np.exp(rng.uniform(0.0, 1.5, H))
    B = rng.standard_normal((Bt, T, G, N))
    C = rng.standard_normal((Bt, T, G, N))
    h0 = rng.standard_normal((Bt, H, N, P)) * 0.5 if init else None
    return x, dt, A, B, C, h0


@pytest.mark.parametrize("N,P", [(3, 3), (3, 2), (2, 5)])
def test_forward_matches_quadratic_form(N, P):
    rng = np.random.default_rng(7)
    x, dt, A, B, C, _ = _inputs(rng, N=N, P=P)
    y, _ = ssd.ssd_forward(x, dt, A, B, C)
    y2 = ssd.ssd_matrix_form(x, dt, A, B, C)
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)


def _seq(packed, Bt, cu, T):
    """packed: 0 none, 1 one packing for the batch (Bt = 1), 2 one per row."""
    if packed == 1:
        return metadata.seq_idx_from_cu_seqlens(np.array(cu), T)
    if packed == 2:
        rows = [cu, [0, T]] + [[0, 1, T]] * (Bt - 2)
        return np.stack([metadata.seq_idx_from_cu_seqlens(np.array(c), T) for c in rows[:Bt]])
    return None


@pytest.mark.parametrize("init,packed,P", [(False, 0, 3), (True, 0, 3), (False, 1, 3), (False, 2, 3),
                                           (True, 0, 2), (False, 1, 4)])
def test_backward_matches_finite_differences(init, packed, P):
    # P != 3: a head dim different from the state size N = 3
    rng = np.random.default_rng(11 + 2 * init + packed)
    Bt = 1 if packed == 1 else 2
    x, dt, A, B, C, h0 = _inputs(rng, Bt=Bt, T=8, init=init, P=P)
    seq = _seq(packed, Bt, [0, 3, 8], 8)
    W = rng.standard_normal(x.shape)
    Wf = rng.standard_normal((Bt, x.shape[2], 3, P))

    def loss(x_, dt_, A_, B_, C_, h0_):
        y, hT = ssd.ssd_forward(x_, dt_, A_, B_, C_, h_init=h0_, seq_idx=seq)
        return float(np.sum(y * W) + np.sum(hT * Wf))

    grads = ssd.ssd_backward(x, dt, A, B, C, W, h_init=h0, seq_idx=seq, dh_final=Wf)
    args = [x, dt, A, B, C, h0]
    eps = 1e-6
    for i, gexp in enumerate(grads):
        if args[i] is None:
            assert gexp is None
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
        np.testing.assert_allclose(gexp, num, rtol=1e-6, atol=1e-7, err_msg=f"input {i}")


@pytest.mark.parametrize("init,packed,P", [(False, 0, 4), (True, 0, 4), (False, 1, 4), (False, 2, 4),
                                           (True, 0, 6), (False, 2, 2)])
def test_matches_linear_attention_oracle(init, packed, P):
    rng = np.random.default_rng(23 + 2 * init + packed)
    Bt = 1 if packed == 1 else 3
    x, dt, A, B, C, h0 = _inputs(rng, Bt=Bt, T=21, H=4, G=2, N=4, init=init, P=P)
    seq = _seq(packed, Bt, [0, 5, 6, 21], 21)
    H, G = x.shape[2], B.shape[2]
    grp = np.arange(H) // (H // G)
    q, k = C[:, :, grp], B[:, :, grp]
    g = A[None, None, :] * dt
    y, hT = ssd.ssd_forward(x, dt, A, B, C, h_init=h0, seq_idx=seq)
    o, ST = rec.forward(q, k, x, g, "scalar", initial_state=h0, seq_idx=seq, w=dt)
    np.testing.assert_allclose(y, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hT, ST, rtol=1e-12, atol=1e-12)

    dy = rng.standard_normal(y.shape)
    dx, ddt, dA, dB, dC, dh0 = ssd.ssd_backward(x, dt, A, B, C, dy, h_init=h0, seq_idx=seq)
    dq, dk, dv, dg, dS0, dw = rec.backward(q, k, x, g, "scalar", dO=dy, initial_state=h0, seq_idx=seq, w=dt)
    np.testing.assert_allclose(dx, dv, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ddt, dw + A[None, None, :] * dg, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dA, np.sum(dt * dg, axis=(0, 1)), rtol=1e-10, atol=1e-12)
    dB2 = np.zeros_like(B)
    dC2 = np.zeros_like(C)
    for h in range(H):
        dB2[:, :, grp[h]] += dk[:, :, h]
        dC2[:, :, grp[h]] += dq[:, :, h]
    np.testing.assert_allclose(dB, dB2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dC, dC2, rtol=1e-10, atol=1e-12)
    if init:
        np.testing.assert_allclose(dh0, dS0, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("packed", [False, True])
def test_weighted_linear_attention_matches_finite_differences(packed):
    rng = np.random.default_rng(31 + packed)
    Bt, T, H, d = (1, 10, 2, 3) if packed else (2, 9, 2, 3)
    q, k, v = (rng.standard_normal((Bt, T, H, d)) for _ in range(3))
    g = -np.log1p(np.exp(rng.standard_normal((Bt, T, H))))
    w = np.exp(rng.standard_normal((Bt, T, H)) * 0.5)
    S0 = None if packed else rng.standard_normal((Bt, H, d, d)) * 0.3
    seq = metadata.seq_idx_from_cu_seqlens(np.array([0, 4, 10]), 10) if packed else None
    W = rng.standard_normal((Bt, T, H, d))

    def loss(q_, k_, v_, g_, w_):
        o, _ = rec.forward(q_, k_, v_, g_, "scalar", initial_state=S0, seq_idx=seq, w=w_)
        return float(np.sum(o * W))

    got = rec.backward(q, k, v, g, "scalar", dO=W, initial_state=S0, seq_idx=seq, w=w)
    grads = {"q": got[0], "k": got[1], "v": got[2], "g": got[3], "w": got[5]}
    args = {"q": q, "k": k, "v": v, "g": g, "w": w}
    eps = 1e-6
    for name, gexp in grads.items():
        num = np.zeros_like(args[name])
        it = np.nditer(args[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            hi = {n: a.copy() for n, a in args.items()}
            lo = {n: a.copy() for n, a in args.items()}
            hi[name][idx] += eps
            lo[name][idx] -= eps
            num[idx] = (loss(**{n + "_": a for n, a in hi.items()}) - loss(**{n + "_": a for n, a in lo.items()})) / (2 * eps)
        np.testing.assert_allclose(gexp, num, rtol=1e-6, atol=1e-7, err_msg=name)
