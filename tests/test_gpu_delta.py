"""GPU parity for the gated delta rule (dense transition) through the C ABI: the
four _delta calls against the fp64 oracle (oracle/delta.py, the per-token
recurrence composed through dense shard summaries) on the same seeded inputs,
element by element: o, final state, the forward summaries (M and delta_S), the
composed incoming states, every gradient (dq, dk, dv, dg, dbeta, dS_init), the
backward summaries (gamma) and the composed outgoing gradients.

Cases span several chunks per shard and several shards, d = 16, 32, 64 in fp32
and bf16 and d = 128 in bf16, an initial state, uneven shards with partial last chunks and empty
shards, and packed sequences (one stream, and one packing per batch row) with
boundaries inside chunks; the two benchmark workloads (d = 64 and 128) at full
size, on sampled (b, h) rows. Tolerances are the linear-attention ones (fp32 rtol
1e-4 / atol 1e-5, bf16 rtol 2e-2 / atol 2e-3).
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import workloads
from _parity import assert_close, tolerances
from oracle import delta as odelta, metadata as omd

pytestmark = pytest.mark.gpu

CASES = {
    "fp32_d16": dict(B=2, T=512, H=2, d=16, num_shards=4, dtype=torch.float32),
    "fp32_d32_init": dict(B=1, T=384, H=2, d=32, num_shards=3, dtype=torch.float32, with_initial_state=True),
    "fp32_d64": dict(B=1, T=512, H=2, d=64, num_shards=4, dtype=torch.float32, with_initial_state=True),
    "bf16_d64": dict(B=2, T=1024, H=2, d=64, num_shards=4),
    "fp32_d64_uneven": dict(B=1, T=500, H=2, d=64, num_shards=3, dtype=torch.float32),
    "fp32_d32_empty_shards": dict(B=1, T=200, H=1, d=32, num_shards=64, dtype=torch.float32),
    "fp32_d16_many_shards": dict(B=1, T=2000, H=1, d=16, num_shards=300, dtype=torch.float32),
    "fp32_d64_packed": dict(B=1, T=768, H=2, d=64, num_shards=4, packed=True, len_range=(30, 300),
                            dtype=torch.float32),
    "bf16_d64_rows_packed": dict(B=2, T=640, H=2, d=64, num_shards=5, packed=True, len_range=(1, 200)),
    # d = 128 (bf16): walks over state-column slabs, gradients over value slices
    "bf16_d128": dict(B=1, T=1024, H=2, d=128, num_shards=4),
    "bf16_d128_init_uneven": dict(B=1, T=500, H=2, d=128, num_shards=3, with_initial_state=True),
    "bf16_d128_rows_packed": dict(B=2, T=640, H=1, d=128, num_shards=5, packed=True, len_range=(1, 200)),
    "bf16_d128_empty_shards": dict(B=1, T=150, H=1, d=128, num_shards=40),
}


def _np(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def _run_gpu(wl):
    import context_state_passing_amd as cpla
    dev = torch.device("cuda:0")
    q, k, v, g, beta, dO = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta, wl.dO))
    S0 = None if wl.initial_state is None else wl.initial_state.to(dev)
    o, ctx = cpla.delta_forward(q, k, v, g, beta, num_shards=wl.num_shards, initial_state=S0,
                                cu_seqlens=wl.cu_seqlens)
    (dq, dk, dv, dg, db, dS0), inter = cpla.delta_backward(dO, ctx, want_intermediates=True)
    torch.cuda.synchronize()
    D = wl.d
    out = {"o": o, "final_state": ctx.final_state, "M": ctx.fwd_summary[..., :D * D].reshape(-1, wl.B, wl.H, D, D),
           "delta_S": ctx.fwd_summary[..., D * D:].reshape(-1, wl.B, wl.H, D, D), "S_in": ctx.shard_in_state,
           "gamma": inter["bwd_summary"][..., D * D:].reshape(-1, wl.B, wl.H, D, D),
           "dS_out": inter["shard_out_grad"], "dq": dq, "dk": dk, "dv": dv, "dg": dg, "dbeta": db}
    if S0 is not None:
        out["d_initial_state"] = dS0
    return {n: _np(t) for n, t in out.items()}


def _run_oracle(wl):
    seq = None if wl.cu_seqlens is None else omd.seq_idx_rows(wl.cu_seqlens, wl.T)
    args = [_np(t) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta)]
    r = odelta.cp_backward(*args, _np(wl.dO), wl.num_shards, initial_state=_np(wl.initial_state), seq_idx=seq)
    fw = r["fwd"]
    out = {"o": fw["o"], "final_state": fw["final_state"], "M": fw["M"], "delta_S": fw["delta_S"],
           "S_in": fw["S_in"], "gamma": r["gamma"], "dS_out": r["dS_out"], "dq": r["dq"], "dk": r["dk"],
           "dv": r["dv"], "dg": r["dg"], "dbeta": r["dbeta"]}
    if wl.initial_state is not None:
        out["d_initial_state"] = r["d_initial_state"]
    return out


@pytest.mark.parametrize("case", sorted(CASES))
def test_delta_parity(case, gpu_available):
    print(f"[gpu-case] delta {case}", file=sys.stderr, flush=True)
    wl = workloads.make_delta(**CASES[case])
    got = _run_gpu(wl)
    ref = _run_oracle(wl)
    rtol, atol = tolerances(wl.dtype)
    for name in ref:
        assert_close(name, got[name], ref[name], rtol, atol)


def test_delta_deterministic(gpu_available):
    print("[gpu-case] delta determinism", file=sys.stderr, flush=True)
    wl = workloads.make_delta(**CASES["bf16_d64"])
    a = _run_gpu(wl)
    b = _run_gpu(wl)
    for name in a:
        assert np.array_equal(a[name], b[name]), name


def _delta_sweep(seed, n):
    """Seeded random gated-delta problems: head sizes 16/32/64, both dtypes,
    uneven and empty shards, packing, an initial state."""
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        over = dict(B=rng.choice([1, 2]), T=rng.choice([rng.randint(1, 130), rng.randint(64, 600)]),
                    H=rng.choice([1, 2, 3]), d=rng.choice([16, 32, 64]), num_shards=rng.randint(1, 9),
                    dtype=rng.choice([torch.float32, torch.bfloat16]))
        if rng.random() < 0.35:
            over.update(packed=True, len_range=(1, rng.randint(1, 300)))
        elif rng.random() < 0.4:
            over.update(with_initial_state=True)
        out.append(over)
    return out


@pytest.mark.parametrize("case", range(30))
def test_random_delta_problems(case, gpu_available):
    over = _delta_sweep(2026, 30)[case]
    print(f"[gpu-case] delta random {case}: {over}", file=sys.stderr, flush=True)
    wl = workloads.make_delta(**over)
    got, ref = _run_gpu(wl), _run_oracle(wl)
    rtol, atol = tolerances(wl.dtype)
    for name in ref:
        assert_close(name, got[name], ref[name], rtol, atol)


def _delta_sweep_wide(seed, n):
    """Seeded random d = 128 (bf16) problems: ragged lengths, uneven and empty
    shards, packing, an initial state."""
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        over = dict(B=rng.choice([1, 2]), T=rng.choice([rng.randint(1, 130), rng.randint(64, 400)]),
                    H=rng.choice([1, 2]), d=128, num_shards=rng.randint(1, 7), dtype=torch.bfloat16)
        if rng.random() < 0.35:
            over.update(packed=True, len_range=(1, rng.randint(1, 250)))
        elif rng.random() < 0.4:
            over.update(with_initial_state=True)
        out.append(over)
    return out


@pytest.mark.parametrize("case", range(8))
def test_random_delta_problems_d128(case, gpu_available):
    over = _delta_sweep_wide(2027, 8)[case]
    print(f"[gpu-case] delta random d128 {case}: {over}", file=sys.stderr, flush=True)
    wl = workloads.make_delta(**over)
    got, ref = _run_gpu(wl), _run_oracle(wl)
    rtol, atol = tolerances(wl.dtype)
    for name in ref:
        assert_close(name, got[name], ref[name], rtol, atol)


# The benchmark workloads at full size, in the launch configuration the bench
# times (B2 H16 T8192, 8 shards, bf16): every output of the GPU run for a few
# sampled (b, h) rows against the oracle run on those rows alone (rows are
# independent problems).
BENCH_ROWS = {"d64": ("delta_fwdbwd", 64, [(0, 3), (1, 12)]), "d128": ("delta_d128_fwdbwd", 128, [(1, 5)])}


def _row(name, x, b, h):
    if name in ("M", "delta_S", "S_in", "gamma", "dS_out"):
        return x[:, b:b + 1, h:h + 1]
    if name in ("final_state", "d_initial_state"):
        return x[b:b + 1, h:h + 1]
    return x[b:b + 1, :, h:h + 1]


@pytest.mark.parametrize("case", sorted(BENCH_ROWS))
def test_delta_bench_shape_sampled_rows(case, gpu_available):
    name, d, rows = BENCH_ROWS[case]
    print(f"[gpu-case] delta bench shape {name} rows {rows}", file=sys.stderr, flush=True)
    wl = workloads.make_delta(name)
    assert (wl.B, wl.T, wl.H, wl.d, wl.num_shards) == (2, 8192, 16, d, 8)
    got = _run_gpu(wl)
    rtol, atol = tolerances(wl.dtype)
    for b, h in rows:
        one = dataclasses.replace(wl, B=1, H=1, **{n: getattr(wl, n)[b:b + 1, :, h:h + 1].contiguous()
                                                  for n in ("q", "k", "v", "g", "beta", "dO")})
        ref = _run_oracle(one)
        for n in ref:
            assert_close(f"{n}[b={b},h={h}]", _row(n, got[n], b, h), ref[n], rtol, atol)
