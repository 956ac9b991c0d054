"""q and k shared by groups of heads (cpla_problem.qk_heads = G: head h reads q, k
head h / (H / G), as Mamba2's B and C; scalar decay) against per-head copies of
the same tensors through the same calls.

Both runs hand the walks identical values in identical order, so o, dq, dk, dv,
dg, dw and the state gradients must be bitwise equal; the per-head path itself
is held to the oracle by the parity tests. The cases cover both dtypes, head
dims 16, 64 and 128, d_k != d_v, packed sequences, input weights with fp32
gradients, an initial state, uneven shards with a partial last chunk, and both
the divided small-grid walks and the one-workgroup-per-shard walks.
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, make overrides, groups, weighted)
    "bf16_d128_full_grid": ("packed_fwdbwd", dict(B=4, T=2048, H=16, num_shards=8, packed=False), 4, False),
    "bf16_d128_packed_uneven": ("packed_fwdbwd", dict(B=1, T=1000, H=4, num_shards=3, len_range=(40, 300)), 2,
                                False),
    "bf16_d64_weighted": ("scalar_fwd", dict(B=2, T=512, H=8, num_shards=4, backward=True), 2, True),
    "bf16_64x128_init": ("long_fwdbwd", dict(B=1, T=640, H=4, d=64, dv=128, num_shards=2), 2, False),
    "fp32_d16_weighted": ("scalar_fwd", dict(B=2, T=256, H=4, d=16, num_shards=4, backward=True,
                                             dtype=torch.float32), 4, True),
    "fp32_d64_init": ("long_fwdbwd", dict(B=1, T=384, H=2, d=64, num_shards=3, dtype=torch.float32), 1, False),
}


def _grouped(t, G):
    """Heads 0, H/G, 2H/G, ... of t [B,T,H,d]: one head per group, contiguous."""
    H = t.shape[2]
    return t[:, :, :: H // G].contiguous()


def _run(q, k, v, g, w, dO, S0, wl):
    import context_state_passing_amd as cpla
    o, ctx = cpla.forward(q, k, v, g, num_shards=wl.num_shards, initial_state=S0, cu_seqlens=wl.cu_seqlens, w=w)
    grads = cpla.backward(dO, ctx, grad_dtype=torch.float32 if w is not None else None)
    torch.cuda.synchronize()
    return [o] + [x for x in grads if x is not None]


@pytest.mark.parametrize("case", sorted(CASES))
def test_grouped_heads_equal_per_head_copies(case):
    name, kw, G, weighted = CASES[case]
    wl = workloads.make(name, **kw)
    dev = torch.device("cuda:0")
    H = wl.H
    qg, kg = (_grouped(t, G).to(dev) for t in (wl.q, wl.k))
    qe, ke = (t.repeat_interleave(H // G, dim=2).contiguous() for t in (qg, kg))
    v, dO = wl.v.to(dev), wl.dO.to(dev)
    g = None if wl.g is None else wl.g.to(dev)
    S0 = None if wl.initial_state is None else wl.initial_state.to(dev)
    w = None
    if weighted:
        gen = torch.Generator().manual_seed(77)
        w = (0.5 + torch.rand(wl.B, wl.T, H, generator=gen)).to(dev)
    print(f"grouped heads: case {case} B={wl.B} T={wl.T} H={H} G={G}", flush=True)
    a = _run(qg, kg, v, g, w, dO, S0, wl)
    b = _run(qe, ke, v, g, w, dO, S0, wl)
    assert len(a) == len(b)
    assert a[1].shape == (wl.B, wl.T, H, qg.shape[-1])        # dq per head
    for i, (x, y) in enumerate(zip(a, b)):
        assert x.shape == y.shape, (case, i)
        assert torch.isfinite(x).all(), (case, i)
        assert torch.equal(x, y), (case, i, (x.float() - y.float()).abs().max().item())
