"""Shared helpers for the GPU parity tests: run the HIP path and the fp64 oracle
on the same seeded workload and compare element by element.

Tolerance (elementwise |x - ref| <= atol + rtol * |ref|): fp32 inputs rtol 1e-4,
atol 1e-5; bf16 inputs rtol 2e-2, atol 2e-3. Integer metadata is compared with ==.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from oracle import cp as ocp
from oracle import metadata as omd


def tolerances(dtype):
    return (1e-4, 1e-5) if dtype == torch.float32 else (2e-2, 2e-3)


# worst |got - ref| / (atol + rtol |ref|) of each compared output, keyed by the
# running test and the output name (reported at the end of the session when
# CPLA_MARGINS_OUT names a file; see conftest.py)
MARGINS = {}


def assert_close(name, got, ref, rtol, atol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    if err.size:
        test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        MARGINS[(test, name)] = max(MARGINS.get((test, name), 0.0),
                                    float(np.max(err / (atol + rtol * np.abs(ref)))))
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        idx = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} elements outside tolerance; worst at {idx}: "
            f"got {got[idx]!r} ref {ref[idx]!r} (max abs err {err.max():.3e}, max |ref| {np.abs(ref).max():.3e})")


def _np(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def _select(key, t, heads):
    """Keep the sampled heads of a device tensor before it is copied to the host."""
    if t is None or heads is None:
        return t
    idx = torch.as_tensor(heads, device=t.device)
    if key in ("final_state", "d_initial_state"):           # [B,H,...]
        return t.index_select(1, idx)
    if key in ("fwd_summary", "bwd_summary", "shard_in_state", "shard_out_grad"):   # [P,B,H,...]
        return t.index_select(2, idx)
    return t.index_select(2, idx)                            # [B,T,H,...]


def gpu_run(wl, backward=True, device="cuda:0", d_final_state=None, heads=None):
    import context_state_passing_amd as cpla
    dev = torch.device(device)
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    g = None if wl.g is None else wl.g.to(dev)
    S0 = None if wl.initial_state is None else wl.initial_state.to(dev)
    o, ctx = cpla.forward(q, k, v, g, num_shards=wl.num_shards, initial_state=S0, cu_seqlens=wl.cu_seqlens,
                          save_for_backward=backward)
    out = {"o": o, "final_state": ctx.final_state, "fwd_summary": ctx.fwd_summary,
           "shard_in_state": ctx.shard_in_state}
    if backward:
        dSf = None if d_final_state is None else d_final_state.to(dev)
        (dq, dk, dv, dg, dS0), inter = cpla.backward(wl.dO.to(dev), ctx, d_final_state=dSf,
                                                     want_intermediates=True)
        out.update(dq=dq, dk=dk, dv=dv, dg=dg, d_initial_state=dS0, **inter)
    torch.cuda.synchronize(dev)
    return {key: _np(_select(key, val, heads)) for key, val in out.items()}


def _rows(x, heads):
    if x is None or heads is None:
        return x
    return x[:, :, heads]


def oracle_run(wl, backward=True, heads=None, d_final_state=None):
    """CP method in fp64 on the selected heads (all if None)."""
    q, k, v = _rows(wl.q, heads), _rows(wl.k, heads), _rows(wl.v, heads)
    g = _rows(wl.g, heads)
    S0 = wl.initial_state if (wl.initial_state is None or heads is None) else wl.initial_state[:, heads]
    dSf = d_final_state if (d_final_state is None or heads is None) else d_final_state[:, heads]
    seq = None
    if wl.cu_seqlens is not None:
        seq = omd.seq_idx_rows(wl.cu_seqlens, wl.T)
    if backward:
        dO = _rows(wl.dO, heads)
        r = ocp.cp_backward(q, k, v, g, wl.decay, dO, wl.num_shards, initial_state=S0, seq_idx=seq,
                            d_final_state=dSf)
        fw = r["fwd"]
        return {"o": fw["o"], "final_state": fw["final_state"], "M": fw["M"], "delta_S": fw["delta_S"],
                "shard_in_state": fw["S_in"], "dq": r["dq"], "dk": r["dk"], "dv": r["dv"], "dg": r["dg"],
                "d_initial_state": r["d_initial_state"], "gamma": r["gamma"], "shard_out_grad": r["dS_out"]}
    fw = ocp.cp_forward(q, k, v, g, wl.decay, wl.num_shards, initial_state=S0, seq_idx=seq)
    return {"o": fw["o"], "final_state": fw["final_state"], "M": fw["M"], "delta_S": fw["delta_S"],
            "shard_in_state": fw["S_in"]}


def split_summary(rec, decay, dk, dv):
    """[P,B,H,W] -> (M [P,B,H,m], state [P,B,H,dk,dv])."""
    m_slot = dk if decay == "diag" else 4
    m_w = dk if decay == "diag" else 1
    P, B, H, _ = rec.shape
    return rec[..., :m_w], rec[..., m_slot:].reshape(P, B, H, dk, dv)


def compare(wl, got, ref, heads=None, backward=True):
    rtol, atol = tolerances(wl.dtype)
    hs = slice(None) if heads is None else heads

    def pick_bthd(x):   # [B,T,H,...]
        return x[:, :, hs]

    def pick_bh(x):     # [B,H,...]
        return x[:, hs]

    def pick_pbh(x):    # [P,B,H,...]
        return x[:, :, hs]

    assert_close("o", pick_bthd(got["o"]), ref["o"], rtol, atol)
    assert_close("final_state", pick_bh(got["final_state"]), ref["final_state"], rtol, atol)
    M, dS = split_summary(got["fwd_summary"], wl.decay, wl.d, wl.dv)
    assert_close("fwd_summary.M", pick_pbh(M), ref["M"], rtol, atol)
    assert_close("fwd_summary.delta_S", pick_pbh(dS), ref["delta_S"], rtol, atol)
    assert_close("shard_in_state", pick_pbh(got["shard_in_state"]), ref["shard_in_state"], rtol, atol)
    if not backward:
        return
    for name in ["dq", "dk", "dv"]:
        assert_close(name, pick_bthd(got[name]), ref[name], rtol, atol)
    if ref["dg"] is not None:
        assert_close("dg", pick_bthd(got["dg"]), ref["dg"], rtol, atol)
    if ref["d_initial_state"] is not None:
        assert_close("d_initial_state", pick_bh(got["d_initial_state"]), ref["d_initial_state"], rtol, atol)
    Mb, gam = split_summary(got["bwd_summary"], wl.decay, wl.d, wl.dv)
    assert_close("bwd_summary.M", pick_pbh(Mb), ref["M"], rtol, atol)
    assert_close("bwd_summary.gamma", pick_pbh(gam), ref["gamma"], rtol, atol)
    assert_close("shard_out_grad", pick_pbh(got["shard_out_grad"]), ref["shard_out_grad"], rtol, atol)
