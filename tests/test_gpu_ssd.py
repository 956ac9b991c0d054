"""GPU parity for the Mamba2 (SSD) parametrisation: cpla_ssd_inputs, the four CP
calls (scalar decay) and cpla_ssd_input_grads, through the C ABI, against the
fp64 SSD oracle (oracle/ssd.py: the recurrence in Mamba2's own terms) on the
same seeded inputs, element by element, for y and every input gradient.

Cases span several chunks per shard and several shards, groups shared by 1, 2
and 4 heads, state sizes 16, 64 and 128, an initial state, and packed
sequences with boundaries inside chunks. Tolerances are those of the
linear-attention parity tests (fp32 rtol 1e-4 / atol 1e-5, bf16 rtol 2e-2 /
atol 2e-3) for every output, d_dt included: d_dt = dw + A dg is a difference of
two terms that cancel to results thousands of times smaller than themselves on
some tokens, which the fp32 inputs meet because their walks form every sum, and
the scalar decay's running log-decay, in fp64.
"""
import sys

import pytest
import torch

import workloads
from _parity import assert_close, tolerances
from oracle import metadata as omd, recurrence as orec, ssd as ossd

pytestmark = pytest.mark.gpu

CASES = {
    # name: make_ssd overrides
    "bf16_n64_g2": dict(B=2, T=512, H=8, G=2, N=64, num_shards=4),
    "bf16_n128_init": dict(B=1, T=512, H=4, G=1, N=128, num_shards=2, with_initial_state=True),
    "bf16_n64_packed": dict(B=1, T=1024, H=4, G=2, N=64, num_shards=4, packed=True, len_range=(40, 300)),
    "fp32_n16_g4": dict(B=2, T=256, H=4, G=4, N=16, num_shards=4, dtype=torch.float32),
    "fp32_n64_init": dict(B=1, T=384, H=2, G=1, N=64, num_shards=3, dtype=torch.float32,
                          with_initial_state=True),
    "bf16_n64_uneven": dict(B=1, T=1000, H=4, G=2, N=64, num_shards=3),
    "bf16_n64_rows_packed": dict(B=2, T=512, H=4, G=2, N=64, num_shards=4, packed=True, len_range=(40, 300)),
    # state size N != head dim P (Mamba2's usual N = 128, P = 64, and the reverse)
    "bf16_n128_p64_init": dict(B=1, T=700, H=4, G=2, N=128, P=64, num_shards=3, with_initial_state=True),
    "bf16_n128_p64_packed": dict(B=1, T=1024, H=4, G=1, N=128, P=64, num_shards=4, packed=True,
                                 len_range=(40, 300)),
    "bf16_n64_p128_g2": dict(B=2, T=512, H=4, G=2, N=64, P=128, num_shards=4),
}


def _np(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def _run_gpu(wl):
    import context_state_passing_amd as cpla
    dev = torch.device("cuda:0")
    x, dt, A, Bm, Cm, dy = (t.to(dev) for t in (wl.x, wl.dt, wl.A, wl.Bm, wl.Cm, wl.dy))
    h0 = None if wl.initial_state is None else wl.initial_state.to(dev)
    y, ctx = cpla.ssd_forward(x, dt, A, Bm, Cm, num_shards=wl.num_shards, initial_state=h0,
                              cu_seqlens=wl.cu_seqlens)
    dx, ddt, dA, dB, dC, dh0 = cpla.ssd_backward(dy, ctx)
    torch.cuda.synchronize()
    out = {"y": y, "dx": dx, "d_dt": ddt, "dA": dA, "dB": dB, "dC": dC}
    if h0 is not None:
        out["d_initial_state"] = dh0
    return {k: v.detach().cpu() for k, v in out.items()}


def _run_oracle(wl):
    seq = None
    if wl.cu_seqlens is not None:
        seq = omd.seq_idx_rows(wl.cu_seqlens, wl.T)
    args = [_np(t) for t in (wl.x, wl.dt, wl.A, wl.Bm, wl.Cm)]
    h0 = _np(wl.initial_state)
    y, _ = ossd.ssd_forward(*args, h_init=h0, seq_idx=seq)
    dx, ddt, dA, dB, dC, dh0 = ossd.ssd_backward(*args, _np(wl.dy), h_init=h0, seq_idx=seq)
    out = {"y": y, "dx": dx, "d_dt": ddt, "dA": dA, "dB": dB, "dC": dC}
    if h0 is not None:
        out["d_initial_state"] = dh0
    return out


@pytest.mark.parametrize("case", sorted(CASES))
def test_ssd_parity(case, gpu_available):
    print(f"[gpu-case] ssd {case}", file=sys.stderr, flush=True)
    wl = workloads.make_ssd(**CASES[case])
    got = _run_gpu(wl)
    ref = _run_oracle(wl)
    rtol, atol = tolerances(wl.dtype)
    for name in ref:
        assert_close(name, _np(got[name]), ref[name], rtol, atol)


def test_ssd_deterministic(gpu_available):
    print("[gpu-case] ssd determinism", file=sys.stderr, flush=True)
    wl = workloads.make_ssd(**CASES["bf16_n64_g2"])
    a = _run_gpu(wl)
    b = _run_gpu(wl)
    for name in a:
        assert torch.equal(a[name], b[name]), name


# ---- the weighted scalar-decay calls on their own ----------------------------------------
WEIGHTED = {
    # name: (workload, overrides)
    "w_bf16_d128": ("packed_fwdbwd", dict(T=1024, H=2, num_shards=4, len_range=(40, 400))),
    "w_bf16_d64_init": ("long_fwdbwd", dict(T=512, H=2, d=64, num_shards=4)),
    "w_fp32_d64": ("scalar_fwd", dict(B=1, H=2, T=512, num_shards=4, backward=True, dtype=torch.float32)),
}


@pytest.mark.parametrize("case", sorted(WEIGHTED))
def test_weighted_parity(case, gpu_available):
    import context_state_passing_amd as cpla
    print(f"[gpu-case] weighted {case}", file=sys.stderr, flush=True)
    name, ov = WEIGHTED[case]
    wl = workloads.make(name, **ov)
    gen = torch.Generator().manual_seed(77)
    w = torch.exp(0.5 * torch.randn(wl.B, wl.T, wl.H, generator=gen)).contiguous()
    dev = torch.device("cuda:0")
    S0 = None if wl.initial_state is None else wl.initial_state.to(dev)
    o, ctx = cpla.forward(wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), wl.g.to(dev), num_shards=wl.num_shards,
                          initial_state=S0, cu_seqlens=wl.cu_seqlens, w=w.to(dev))
    dq, dk, dv, dg, dS0, dw = cpla.backward(wl.dO.to(dev), ctx)
    torch.cuda.synchronize()
    seq = None if wl.cu_seqlens is None else omd.seq_idx_rows(wl.cu_seqlens, wl.T)
    args = [_np(t) for t in (wl.q, wl.k, wl.v, wl.g)]
    ref_o, ref_S = orec.forward(*args, "scalar", initial_state=_np(wl.initial_state), seq_idx=seq, w=_np(w))
    ref = orec.backward(*args, "scalar", dO=_np(wl.dO), initial_state=_np(wl.initial_state), seq_idx=seq,
                        w=_np(w))
    rtol, atol = tolerances(wl.dtype)
    got = {"o": o, "final_state": ctx.final_state, "dq": dq, "dk": dk, "dv": dv, "dg": dg, "dw": dw}
    want = {"o": ref_o, "final_state": ref_S, "dq": ref[0], "dk": ref[1], "dv": ref[2], "dg": ref[3], "dw": ref[5]}
    if S0 is not None:
        got["d_initial_state"] = dS0
        want["d_initial_state"] = ref[4]
    for n in want:
        assert_close(n, _np(got[n]), want[n], rtol, atol)


def _ssd_sweep(seed, n):
    """Seeded random Mamba2 problems: state size / head dim pairs (N = P and
    N != P), groups, uneven and empty shards, packing, an initial state."""
    import random
    rng = random.Random(seed)
    pairs = [((16, 16), torch.float32), ((64, 64), torch.float32), ((16, 16), torch.bfloat16),
             ((64, 64), torch.bfloat16), ((128, 128), torch.bfloat16), ((128, 64), torch.bfloat16),
             ((64, 128), torch.bfloat16)]
    out = []
    for _ in range(n):
        (N, P), dt = rng.choice(pairs)
        H = rng.choice([1, 2, 4, 8])
        over = dict(B=rng.choice([1, 2]), T=rng.choice([rng.randint(1, 130), rng.randint(64, 800)]), H=H,
                    G=rng.choice([g for g in (1, 2, 4, 8) if H % g == 0]), N=N, P=P,
                    num_shards=rng.randint(1, 9), dtype=dt)
        if rng.random() < 0.35:
            over.update(packed=True, len_range=(1, rng.randint(1, 300)))
        elif rng.random() < 0.4:
            over.update(with_initial_state=True)
        out.append(over)
    return out


@pytest.mark.parametrize("case", range(30))
def test_random_ssd_problems(case, gpu_available):
    over = _ssd_sweep(2026, 30)[case]
    print(f"[gpu-case] ssd random {case}: {over}", file=sys.stderr, flush=True)
    wl = workloads.make_ssd(**over)
    got, ref = _run_gpu(wl), _run_oracle(wl)
    rtol, atol = tolerances(wl.dtype)
    for name in ref:
        assert_close(name, _np(got[name]), ref[name], rtol, atol)
