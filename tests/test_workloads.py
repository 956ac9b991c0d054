"""The seeded generators produce the workloads' shapes, dtypes and distributions."""
import math

import torch

import workloads


def test_shapes_and_dtypes_small():
    for name, spec in workloads.SPECS.items():
        wl = workloads.make(name, T=512, H=2, B=1, num_shards=4, backward=True)
        assert wl.q.shape == (1, 512, 2, spec.d) and wl.q.dtype == spec.dtype
        assert wl.v.shape == (1, 512, 2, spec.d)
        if spec.decay == "scalar":
            assert wl.g.shape == (1, 512, 2) and wl.g.dtype == torch.float32 and (wl.g < 0).all()
        elif spec.decay == "diag":
            assert wl.g.shape == (1, 512, 2, spec.d) and (wl.g <= 0).all() and (wl.g > -2).all()
        else:
            assert wl.g is None
        assert (wl.initial_state is not None) == spec.initial_state


def test_packed_lengths():
    wl = workloads.make("packed_fwdbwd", H=1, T=32768)
    cu = wl.cu_seqlens.tolist()
    assert cu[0] == 0 and cu[-1] == 32768
    lens = [b - a for a, b in zip(cu[:-1], cu[1:])]
    assert all(128 <= n <= 4096 for n in lens[:-1]) and 1 <= lens[-1] <= 4096


def test_per_row_packing():
    wl = workloads.make("packed_fwdbwd", B=3, H=1, T=1000, len_range=(10, 300))
    assert isinstance(wl.cu_seqlens, list) and len(wl.cu_seqlens) == 3
    for cu in wl.cu_seqlens:
        c = cu.tolist()
        assert c[0] == 0 and c[-1] == 1000 and all(b > a for a, b in zip(c[:-1], c[1:]))
    assert wl.cu_seqlens[0].tolist() != wl.cu_seqlens[1].tolist()
    d = workloads.make("diag_fwdbwd", B=2, T=512, H=1, packed=True, len_range=(30, 300))
    assert len(d.cu_seqlens) == 2
    s = workloads.make_ssd(B=2, T=512, packed=True, len_range=(40, 300))
    assert len(s.cu_seqlens) == 2


def test_seeded_and_scaled():
    a = workloads.make("scalar_fwd", T=256, H=1, B=1)
    b = workloads.make("scalar_fwd", T=256, H=1, B=1)
    assert torch.equal(a.q, b.q) and torch.equal(a.g, b.g)
    x = workloads.make("diag_fwdbwd", T=1024, H=4, B=1).q.float()
    assert abs(x.std().item() - 1 / math.sqrt(128)) < 0.01
    k = workloads.make("long_fwdbwd", T=256, H=2).k.float()
    assert torch.allclose(k.norm(dim=-1), torch.ones(1, 256, 2), atol=0.02)
