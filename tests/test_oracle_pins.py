"""Pins for the fp64 oracle: checks against things other than the oracle itself.

* O(T^2) closed forms (identity decay: tril(Q K^T) V; decayed: explicit double sum);
* central finite differences of a scalar loss (backward);
* packed stream == each sequence run alone (one packing for the batch, or one per row);
* sharded (summaries + composition) == unsharded, packed and unpacked;
* chunk algebra == per-token recurrence at chunk lengths 1, 7, 64;
* the adjoint identity sum_t (q*dq - k*dk) == 0 over a sequence with zero
  boundary state, and dg == 0 at sequence starts.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunked, cp, metadata, recurrence as rec

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(rng, B, T, H, dk, dv, decay, init=False, scale=1.0, gscale=1.0):
    q = rng.standard_normal((B, T, H, dk)) * scale
    k = rng.standard_normal((B, T, H, dk)) * scale
    v = rng.standard_normal((B, T, H, dv)) * scale
    if decay == "scalar":
        g = -np.log1p(np.exp(rng.standard_normal((B, T, H)))) * gscale
    elif decay == "diag":
        g = -np.log1p(np.exp(-rng.standard_normal((B, T, H, dk)))) / 4 * gscale
    else:
        g = None
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3 if init else None
    return q, k, v, g, S0


def _packed_seq_idx(lengths):
    cu = np.concatenate([[0], np.cumsum(lengths)])
    return metadata.seq_idx_from_cu_seqlens(cu, int(cu[-1])), cu


# --- forward closed forms ---------------------------------------------------

@pytest.mark.parametrize("init", [False, True])
def test_identity_forward_is_masked_matmul(init):
    rng = np.random.default_rng(0)
    q, k, v, _, S0 = _rand(rng, 2, 40, 3, 5, 4, "none", init)
    o, fin = oracle.forward(q, k, v, None, "none", initial_state=S0)
    for b in range(2):
        for h in range(3):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            ref = np.tril(Q @ K.T) @ V
            if init:
                ref = ref + Q @ S0[b, h]
            np.testing.assert_allclose(o[b, :, h], ref, rtol=1e-12, atol=1e-12)
            ref_fin = K.T @ V + (S0[b, h] if init else 0)
            np.testing.assert_allclose(fin[b, h], ref_fin, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("decay", ["scalar", "diag"])
def test_decayed_forward_closed_form(decay):
    rng = np.random.default_rng(1)
    B, T, H, dk, dv = 1, 13, 2, 3, 2
    q, k, v, g, S0 = _rand(rng, B, T, H, dk, dv, decay, init=True)
    o, _ = oracle.forward(q, k, v, g, decay, initial_state=S0)
    for h in range(H):
        gg = g[0, :, h] if decay == "diag" else np.repeat(g[0, :, h][:, None], dk, axis=1)
        G = np.cumsum(gg, axis=0)       # G_t = sum_{u<=t} g_u, per key dim
        for t in range(T):
            ref = (q[0, t, h] * np.exp(G[t])) @ S0[0, h]
            for s in range(t + 1):
                w = float(np.sum(q[0, t, h] * np.exp(G[t] - G[s]) * k[0, s, h]))
                ref = ref + w * v[0, s, h]
            np.testing.assert_allclose(o[0, t, h], ref, rtol=1e-12, atol=1e-12)


def test_packed_equals_separate():
    rng = np.random.default_rng(2)
    lengths = [5, 1, 17, 9, 2, 30]
    seq, cu = _packed_seq_idx(lengths)
    T = int(cu[-1])
    for decay in ["none", "scalar", "diag"]:
        q, k, v, g, _ = _rand(rng, 1, T, 2, 4, 3, decay)
        o, fin = oracle.forward(q, k, v, g, decay, seq_idx=seq)
        dO = rng.standard_normal(o.shape)
        dq, dk, dv, dg, _ = oracle.backward(q, k, v, g, decay, dO, seq_idx=seq)
        for s in range(len(lengths)):
            a, b = int(cu[s]), int(cu[s + 1])
            gs = None if g is None else g[:, a:b]
            o_s, fin_s = oracle.forward(q[:, a:b], k[:, a:b], v[:, a:b], gs, decay)
            np.testing.assert_allclose(o[:, a:b], o_s, rtol=0, atol=1e-13)
            r = oracle.backward(q[:, a:b], k[:, a:b], v[:, a:b], gs, decay, dO[:, a:b])
            np.testing.assert_allclose(dq[:, a:b], r[0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(dk[:, a:b], r[1], rtol=0, atol=1e-13)
            np.testing.assert_allclose(dv[:, a:b], r[2], rtol=0, atol=1e-13)
            if dg is not None:
                np.testing.assert_allclose(dg[:, a:b], r[3], rtol=0, atol=1e-13)
                assert np.all(dg[:, a] == 0.0)       # a start never sees its decay
        np.testing.assert_allclose(fin, fin_s, rtol=0, atol=1e-13)


ROW_LENGTHS = [[5, 1, 17, 9, 2, 30], [64], [30, 34], [1, 1, 62]]   # one packing per batch row, T = 64


def _row_packing(lengths_per_row):
    seqs, cus = zip(*(_packed_seq_idx(L) for L in lengths_per_row))
    return np.stack(seqs), cus


def test_per_row_packing_equals_separate():
    """seq_idx [B, T]: every row keeps its own boundaries; each sequence of each
    row equals that sequence run alone, forward and backward."""
    rng = np.random.default_rng(12)
    seq, cus = _row_packing(ROW_LENGTHS)
    B, T = seq.shape
    for decay in ["none", "scalar", "diag"]:
        q, k, v, g, _ = _rand(rng, B, T, 2, 4, 3, decay)
        o, fin = oracle.forward(q, k, v, g, decay, seq_idx=seq)
        dO = rng.standard_normal(o.shape)
        dq, dk, dv, dg, _ = oracle.backward(q, k, v, g, decay, dO, seq_idx=seq)
        for b, cu in enumerate(cus):
            for s in range(len(cu) - 1):
                a, e = int(cu[s]), int(cu[s + 1])
                sl = (slice(b, b + 1), slice(a, e))
                gs = None if g is None else g[sl]
                o_s, fin_s = oracle.forward(q[sl], k[sl], v[sl], gs, decay)
                np.testing.assert_allclose(o[sl], o_s, rtol=0, atol=1e-13)
                r = oracle.backward(q[sl], k[sl], v[sl], gs, decay, dO[sl])
                for got, want in [(dq, r[0]), (dk, r[1]), (dv, r[2])]:
                    np.testing.assert_allclose(got[sl], want, rtol=0, atol=1e-13)
                if dg is not None:
                    np.testing.assert_allclose(dg[sl], r[3], rtol=0, atol=1e-13)
                    assert np.all(dg[b, a] == 0.0)
            np.testing.assert_allclose(fin[b:b + 1], fin_s, rtol=0, atol=1e-13)


# --- backward: finite differences ---------------------------------------------

def _loss(q, k, v, g, decay, S0, Wo, Wf, seq=None):
    o, fin = oracle.forward(q, k, v, g, decay, initial_state=S0, seq_idx=seq)
    return float(np.sum(o * Wo) + np.sum(fin * Wf))


@pytest.mark.parametrize("decay,packed", [("none", False), ("scalar", False), ("diag", False),
                                          ("scalar", True), ("diag", True)])
def test_backward_finite_differences(decay, packed):
    rng = np.random.default_rng(3)
    B, H, dk, dv = 1, 2, 3, 2
    if packed:
        seq, cu = _packed_seq_idx([4, 1, 7, 6])
        T = int(cu[-1])
    else:
        seq, T = None, 14
    q, k, v, g, S0 = _rand(rng, B, T, H, dk, dv, decay, init=not packed)
    Wo = rng.standard_normal((B, T, H, dv))
    Wf = rng.standard_normal((B, H, dk, dv))
    dq, dk_, dv_, dg, dS0 = oracle.backward(q, k, v, g, decay, Wo, initial_state=S0, seq_idx=seq,
                                            d_final_state=Wf)
    eps = 1e-6
    named = {"q": (q, dq), "k": (k, dk_), "v": (v, dv_)}
    if g is not None:
        named["g"] = (g, dg)
    if S0 is not None:
        named["S0"] = (S0, dS0)
    for name, (x, grad) in named.items():
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, g, decay, S0, Wo, Wf, seq)
            x[idx] = old - eps
            lm = _loss(q, k, v, g, decay, S0, Wo, Wf, seq)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_adjoint_identity_and_starts():
    # sum over a sequence of q*dq - k*dk vanishes with zero boundary state and
    # zero final gradient (dg telescopes); dg is exactly 0 at every start.
    rng = np.random.default_rng(4)
    seq, cu = _packed_seq_idx([9, 3, 12])
    T = int(cu[-1])
    q, k, v, g, _ = _rand(rng, 1, T, 2, 4, 3, "diag")
    dO = rng.standard_normal((1, T, 2, 3))
    dq, dk, dv, dg, _ = oracle.backward(q, k, v, g, "diag", dO, seq_idx=seq)
    for s in range(3):
        a, b = int(cu[s]), int(cu[s + 1])
        tot = np.sum(q[:, a:b] * dq[:, a:b] - k[:, a:b] * dk[:, a:b], axis=1)
        np.testing.assert_allclose(tot, 0.0, atol=1e-12)
        assert np.all(dg[:, a] == 0.0)
        # dg_t == sum_{s >= t in the sequence} (q*dq - k*dk)
        rev = np.cumsum((q * dq - k * dk)[:, a:b][:, ::-1], axis=1)[:, ::-1]
        np.testing.assert_allclose(dg[:, a + 1:b], rev[:, 1:], atol=1e-12)


# --- sharded == unsharded ---------------------------------------------------

@pytest.mark.parametrize("decay", ["none", "scalar", "diag"])
@pytest.mark.parametrize("P", [1, 2, 4, 8, 3, 5, 7, 40])
def test_sharded_equals_unsharded(decay, P):
    # P = 3, 5, 7: torch.chunk's uneven split of 32 tokens (the last shard shorter,
    # or empty: 7 parts of ceil(32/7) = 5 leave the seventh with 2); P = 40: shards
    # of one token and eight empty ones
    rng = np.random.default_rng(10 + P)
    B, T, H, dk, dv = 2, 32, 2, 3, 4
    q, k, v, g, S0 = _rand(rng, B, T, H, dk, dv, decay, init=True, gscale=0.1)
    dO = rng.standard_normal((B, T, H, dv))
    dSf = rng.standard_normal((B, H, dk, dv))
    o, fin = oracle.forward(q, k, v, g, decay, initial_state=S0)
    dq, dk_, dv_, dg, dS0 = oracle.backward(q, k, v, g, decay, dO, initial_state=S0, d_final_state=dSf)
    f = cp.cp_forward(q, k, v, g, decay, P, initial_state=S0)
    np.testing.assert_allclose(f["o"], o, atol=1e-12)
    np.testing.assert_allclose(f["final_state"], fin, atol=1e-12)
    r = cp.cp_backward(q, k, v, g, decay, dO, P, initial_state=S0, d_final_state=dSf)
    for a, b in [(r["dq"], dq), (r["dk"], dk_), (r["dv"], dv_), (r["d_initial_state"], dS0)]:
        np.testing.assert_allclose(a, b, atol=1e-12)
    if g is not None:
        np.testing.assert_allclose(r["dg"], dg, atol=1e-12)


@pytest.mark.parametrize("lengths", [[7, 9, 3, 13, 8], [40], [8, 8, 8, 8, 8], [1, 2, 3, 30, 4], [16, 24]])
def test_sharded_packed_equals_whole_stream(lengths):
    rng = np.random.default_rng(5)
    seq, cu = _packed_seq_idx(lengths)
    T = int(cu[-1])
    for decay, P in [("none", 5 if T % 5 == 0 else 4), ("scalar", 3), ("diag", 7)]:
        q, k, v, g, _ = _rand(rng, 1, T, 2, 3, 2, decay, gscale=0.1)
        dO = rng.standard_normal((1, T, 2, 2))
        o, fin = oracle.forward(q, k, v, g, decay, seq_idx=seq)
        dq, dk_, dv_, dg, _ = oracle.backward(q, k, v, g, decay, dO, seq_idx=seq)
        f = cp.cp_forward(q, k, v, g, decay, P, seq_idx=seq)
        np.testing.assert_allclose(f["o"], o, atol=1e-12)
        np.testing.assert_allclose(f["final_state"], fin, atol=1e-12)
        r = cp.cp_backward(q, k, v, g, decay, dO, P, seq_idx=seq)
        for a, b in [(r["dq"], dq), (r["dk"], dk_), (r["dv"], dv_)]:
            np.testing.assert_allclose(a, b, atol=1e-12)
        if g is not None:
            np.testing.assert_allclose(r["dg"], dg, atol=1e-12)
        # composing every shard from rank 0 with the true transitions (M = 0 across a
        # start) gives the same incoming states as the sliced prefixes, except at ranks
        # that begin with a start: their incoming state is never read (the slice gives 0)
        S_in_all, _ = cp.compose_prefix(f["M"], f["delta_S"], None, None)
        starts = rec.starts_from_seq_idx(seq, T)
        for r, (a, e) in enumerate(cp.shard_bounds(T, P)):
            if a == e:
                continue                                    # empty shard: nothing reads its state
            if starts[a]:
                assert np.all(f["S_in"][r] == 0.0)
            else:
                np.testing.assert_allclose(S_in_all[r], f["S_in"][r], atol=1e-12)


@pytest.mark.parametrize("P", [3, 4, 7])
def test_sharded_per_row_packing_equals_whole_stream(P):
    """One packing per batch row: each row gets its own rank slices, and the
    sharded method equals the per-token recurrence on every row."""
    rng = np.random.default_rng(50 + P)
    seq, _ = _row_packing(ROW_LENGTHS)
    B, T = seq.shape
    for decay in ["scalar", "diag"]:
        q, k, v, g, _ = _rand(rng, B, T, 2, 3, 2, decay, gscale=0.1)
        dO = rng.standard_normal((B, T, 2, 2))
        o, fin = oracle.forward(q, k, v, g, decay, seq_idx=seq)
        dq, dk_, dv_, dg, _ = oracle.backward(q, k, v, g, decay, dO, seq_idx=seq)
        f = cp.cp_forward(q, k, v, g, decay, P, seq_idx=seq)
        np.testing.assert_allclose(f["o"], o, atol=1e-12)
        np.testing.assert_allclose(f["final_state"], fin, atol=1e-12)
        assert f["S_in"].shape == (P, B, 2, 3, 2)
        r = cp.cp_backward(q, k, v, g, decay, dO, P, seq_idx=seq)
        for a, b in [(r["dq"], dq), (r["dk"], dk_), (r["dv"], dv_), (r["dg"], dg)]:
            np.testing.assert_allclose(a, b, atol=1e-12)
        # a row's slices depend on that row only
        for b in range(B):
            prs, frs = metadata.rank_slices(seq[b], P)
            one = cp.cp_forward(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], decay, P, seq_idx=seq[b])
            np.testing.assert_array_equal(one["S_in"][:, 0], f["S_in"][:, b])
            assert prs.shape == frs.shape == (P,)


# --- chunk algebra ------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 7, 64])
@pytest.mark.parametrize("decay", ["none", "scalar", "diag"])
def test_chunked_equals_sequential(chunk, decay):
    rng = np.random.default_rng(6)
    B, T, H, dk, dv = 1, 70, 2, 4, 3
    q, k, v, g, S0 = _rand(rng, B, T, H, dk, dv, decay, init=True)
    dO = rng.standard_normal((B, T, H, dv))
    dSf = rng.standard_normal((B, H, dk, dv))
    o, fin = oracle.forward(q, k, v, g, decay, initial_state=S0)
    oc, finc = chunked.forward(q, k, v, g, decay, initial_state=S0, chunk=chunk)
    np.testing.assert_allclose(oc, o, atol=1e-11)
    np.testing.assert_allclose(finc, fin, atol=1e-11)
    ref = oracle.backward(q, k, v, g, decay, dO, initial_state=S0, d_final_state=dSf)
    got = chunked.backward(q, k, v, g, decay, dO, initial_state=S0, d_final_state=dSf, chunk=chunk)
    for i, name in enumerate(["dq", "dk", "dv", "dg", "dS0"]):
        if ref[i] is None:
            assert got[i] is None
            continue
        np.testing.assert_allclose(got[i], ref[i], atol=1e-10, err_msg=name)


@pytest.mark.parametrize("decay", ["scalar", "diag"])
def test_chunked_packed_many_starts_per_chunk(decay):
    rng = np.random.default_rng(7)
    seq, cu = _packed_seq_idx([3, 1, 1, 6, 20, 2, 9, 30])
    T = int(cu[-1])
    q, k, v, g, _ = _rand(rng, 1, T, 2, 3, 2, decay)
    dO = rng.standard_normal((1, T, 2, 2))
    o, _ = oracle.forward(q, k, v, g, decay, seq_idx=seq)
    oc, _ = chunked.forward(q, k, v, g, decay, seq_idx=seq, chunk=16)
    np.testing.assert_allclose(oc, o, atol=1e-12)
    ref = oracle.backward(q, k, v, g, decay, dO, seq_idx=seq)
    got = chunked.backward(q, k, v, g, decay, dO, seq_idx=seq, chunk=16)
    for i in range(4):
        np.testing.assert_allclose(got[i], ref[i], atol=1e-11)


# --- metadata -----------------------------------------------------------------

def test_metadata_worked_example():
    with open(os.path.join(HERE, "golden", "packed_metadata_example.json")) as f:
        ex = json.load(f)
    cu = np.array(ex["cu_seqlens"])
    seq = metadata.seq_idx_from_cu_seqlens(cu, int(cu[-1]))
    for r in range(ex["cp_size"]):
        m = metadata.build_packed_sequence_cp_metadata(seq, r, ex["cp_size"])
        assert m["preceding_rank_start"] == ex["preceding_rank_start"][r]
        assert m["following_rank_stop"] == ex["following_rank_stop"][r]
        assert m["local_cu_seqlens"].tolist() == ex["local_cu_seqlens"][r]
        assert m["local_seq_idx"].tolist() == ex["local_seq_idx"][r]


def test_metadata_edge_cases():
    # one sequence spanning every rank
    seq = np.zeros(32, dtype=np.int32)
    prs, frs = metadata.rank_slices(seq, 4)
    assert prs.tolist() == [0, 0, 0, 0] and frs.tolist() == [4, 4, 4, 4]
    # every rank starts exactly at a sequence start
    seq = np.repeat(np.arange(4), 8).astype(np.int32)
    prs, frs = metadata.rank_slices(seq, 4)
    assert prs.tolist() == [0, 1, 2, 3] and frs.tolist() == [1, 2, 3, 4]
    # uneven division (torch.chunk): 3 tokens on 2 ranks are [0, 2) and [2, 3)
    m = metadata.build_packed_sequence_cp_metadata(np.array([0, 0, 0]), 1, 2)
    assert m["local_seq_idx"].tolist() == [0] and m["local_cu_seqlens"].tolist() == [0, 1]
    assert m["preceding_rank_start"] == 0 and m["following_rank_stop"] == 2
    # 5 tokens on 8 ranks: ranks 5..7 are empty and compose nothing
    seq = np.array([0, 0, 1, 1, 1], dtype=np.int32)
    prs, frs = metadata.rank_slices(seq, 8)
    assert prs.tolist() == [0, 0, 2, 2, 2, 5, 6, 7] and frs.tolist() == [2, 2, 5, 5, 5, 6, 7, 8]
    # malformed inputs fail
    for bad in [np.array([1, 1, 1, 1]), np.array([0, 2, 2, 2]), np.array([0, 1, 0, 1])]:
        with pytest.raises(metadata.MetadataError):
            metadata.build_packed_sequence_cp_metadata(bad, 0, 2)
    with pytest.raises(metadata.MetadataError):
        metadata.seq_idx_from_cu_seqlens([0, 3, 3, 5], 5)


def test_shard_bounds_follow_torch_chunk():
    import torch
    for T in [1, 5, 9, 10, 32, 100, 4097]:
        for P in [1, 2, 3, 4, 7, 8, 40]:
            want = [len(c) for c in torch.arange(T).chunk(P)]
            got = [e - a for a, e in cp.shard_bounds(T, P)]
            assert got[:len(want)] == want and all(n == 0 for n in got[len(want):]), (T, P)
