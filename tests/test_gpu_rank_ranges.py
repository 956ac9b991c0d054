"""Calls restricted to a range of shards (cpla_problem.rank_begin / rank_end) give
the same bits as one call over every shard: the interface through which each GPU
of a context-parallel group would run its own shards, with only the summaries
exchanged between the prepare and apply calls (here every shard's record sits
in one buffer). Each shard's calls are issued one rank at a time, prepare for all
ranks before any apply, as the protocol orders them."""
import ctypes
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def _la_step(wl, ranges):
    import context_state_passing_amd as cpla
    from context_state_passing_amd import _lib
    from context_state_passing_amd.api import _decay_of, _ptr, make_problem, packed_meta
    dev = torch.device("cuda:0")
    q, k, v, dO = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.dO))
    g = None if wl.g is None else wl.g.to(dev)
    B, T, H, d = q.shape
    P = wl.num_shards
    decay = _decay_of(g, q)
    L = _lib.lib()
    p_all = make_problem(q, v, P, decay)
    W = L.cpla_summary_width(ctypes.byref(p_all))
    f32 = dict(device=dev, dtype=torch.float32)
    fsum, bsum = torch.zeros((P, B, H, W), **f32), torch.zeros((P, B, H, W), **f32)
    s_in, s_out = torch.zeros((P, B, H, d, d), **f32), torch.zeros((P, B, H, d, d), **f32)
    fin = torch.zeros((B, H, d, d), **f32)
    cs = torch.zeros((L.cpla_chunk_states_bytes(ctypes.byref(p_all)) // 4,), **f32)
    o, dq, dk, dv = (torch.zeros_like(x) for x in (v, q, k, v))
    dg = None if g is None else torch.zeros_like(g)
    meta = None if wl.cu_seqlens is None else packed_meta(wl.cu_seqlens, T, P, dev, B)
    pk = None if meta is None else ctypes.byref(meta.c())
    dS0 = torch.zeros((B, H, d, d), **f32) if meta is None else None
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    probs = [make_problem(q, v, P, decay, rank_range=r) for r in ranges]
    chk = _lib.check
    for p in probs:
        chk(L.cp_forward_prepare(ctypes.byref(p), pk, _ptr(k), _ptr(v), _ptr(g), _ptr(fsum), st))
    for p in probs:
        chk(L.cp_forward_apply(ctypes.byref(p), pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(fsum), None, _ptr(o),
                               _ptr(s_in), _ptr(fin), _ptr(cs), st))
    for p in probs:
        chk(L.cp_backward_prepare(ctypes.byref(p), pk, _ptr(q), _ptr(g), _ptr(dO), _ptr(bsum), st))
    for p in probs:
        chk(L.cp_backward_apply(ctypes.byref(p), pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dO), _ptr(cs),
                                _ptr(bsum), None, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(s_out), _ptr(dS0), st))
    torch.cuda.synchronize()
    out = {"fsum": fsum, "bsum": bsum, "s_in": s_in, "s_out": s_out, "o": o, "dq": dq, "dk": dk, "dv": dv}
    if dg is not None:
        out["dg"] = dg
    if dS0 is not None:
        out["dS0"] = dS0
    return {n: t.cpu() for n, t in out.items()}


def _delta_step(wl, ranges):
    from context_state_passing_amd import _lib
    from context_state_passing_amd.api import _ptr, make_problem, packed_meta
    dev = torch.device("cuda:0")
    q, k, v, g, beta, dO = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta, wl.dO))
    B, T, H, d = q.shape
    P = wl.num_shards
    L = _lib.lib()
    p_all = make_problem(q, v, P, _lib.DECAY_DELTA)
    W = L.cpla_summary_width(ctypes.byref(p_all))
    f32 = dict(device=dev, dtype=torch.float32)
    ws = torch.zeros((L.cpla_delta_workspace_bytes(ctypes.byref(p_all)) // 4,), **f32)
    fsum, bsum = torch.zeros((P, B, H, W), **f32), torch.zeros((P, B, H, W), **f32)
    s_in, s_out = torch.zeros((P, B, H, d, d), **f32), torch.zeros((P, B, H, d, d), **f32)
    fin = torch.zeros((B, H, d, d), **f32)
    o, dq, dk, dv = (torch.zeros_like(x) for x in (v, q, k, v))
    dg, db = torch.zeros_like(g), torch.zeros_like(beta)
    meta = None if wl.cu_seqlens is None else packed_meta(wl.cu_seqlens, T, P, dev, B)
    pk = None if meta is None else ctypes.byref(meta.c())
    dS0 = torch.zeros((B, H, d, d), **f32) if meta is None else None
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    probs = [make_problem(q, v, P, _lib.DECAY_DELTA, rank_range=r) for r in ranges]
    chk = _lib.check
    for p in probs:
        chk(L.cp_forward_prepare_delta(ctypes.byref(p), pk, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(fsum),
                                       _ptr(ws), st))
    for p in probs:
        chk(L.cp_forward_apply_delta(ctypes.byref(p), pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(fsum), None, _ptr(o), _ptr(s_in), _ptr(fin), _ptr(ws), st))
    for p in probs:
        chk(L.cp_backward_prepare_delta(ctypes.byref(p), pk, _ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(dO),
                                        _ptr(fsum), _ptr(bsum), _ptr(ws), st))
    for p in probs:
        chk(L.cp_backward_apply_delta(ctypes.byref(p), pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(dO),
                                      _ptr(bsum), None, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db),
                                      _ptr(s_out), _ptr(dS0), _ptr(ws), st))
    torch.cuda.synchronize()
    out = {"fsum": fsum, "bsum": bsum, "s_in": s_in, "s_out": s_out, "o": o, "dq": dq, "dk": dk, "dv": dv,
           "dg": dg, "dbeta": db}
    if dS0 is not None:
        out["dS0"] = dS0
    return {n: t.cpu() for n, t in out.items()}


CASES = {
    "diag": ("la", dict(name="diag_fwdbwd", B=1, H=2, T=700, num_shards=5)),
    "packed_scalar": ("la", dict(name="packed_fwdbwd", B=2, T=1024, H=2, num_shards=4, len_range=(40, 400))),
    "delta": ("delta", dict(B=1, T=640, H=2, d=64, num_shards=5)),
    "delta_packed": ("delta", dict(B=1, T=768, H=2, d=32, num_shards=4, packed=True, len_range=(30, 300))),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_rank_ranges_match_one_call(case, gpu_available):
    print(f"[gpu-case] rank ranges {case}", file=sys.stderr, flush=True)
    kind, ov = CASES[case]
    if kind == "la":
        ov = dict(ov)
        wl = workloads.make(ov.pop("name"), **ov)
        run = _la_step
    else:
        wl = workloads.make_delta(**ov)
        run = _delta_step
    P = wl.num_shards
    whole = run(wl, [(0, P)])
    single = run(wl, [(r, r + 1) for r in range(P)])
    pairs = run(wl, [(r, min(r + 2, P)) for r in range(0, P, 2)])
    for name in whole:
        assert torch.equal(whole[name], single[name]), f"{name}: one rank per call differs"
        assert torch.equal(whole[name], pairs[name]), f"{name}: two ranks per call differ"
