"""cp_forward_apply_noalloc against cp_forward_apply, through the C ABI.

The no-allocation entry point keeps the composed per-shard incoming states in a
per-GPU scratch array inside the library instead of a caller buffer, and runs
the same kernels: its outputs (o, final_state, chunk_states) must be the bits of
cp_forward_apply's on the same inputs. Two calls in a row, the second on a
smaller problem, so that the scratch holds the first call's contents when the
second starts; a problem too large for the scratch is refused before any launch.
"""
import ctypes
import sys

import pytest
import torch

import workloads
from context_state_passing_amd import _lib
from context_state_passing_amd.api import _ptr, make_problem, packed_meta

pytestmark = pytest.mark.gpu

DECAY = {"none": _lib.DECAY_NONE, "scalar": _lib.DECAY_SCALAR, "diag": _lib.DECAY_DIAG}


def _both(wl, dev):
    """o, final_state, chunk_states from cp_forward_apply and from the no-alloc call."""
    L = _lib.lib()
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    g = None if wl.g is None else wl.g.to(dev)
    S0 = None if wl.initial_state is None else wl.initial_state.to(dev)
    p = make_problem(q, v, wl.num_shards, DECAY[wl.decay])
    pp = ctypes.byref(p)
    B, T, H, dk, dv, P = wl.B, wl.T, wl.H, wl.d, wl.dv, wl.num_shards
    f32 = dict(device=dev, dtype=torch.float32)
    fsum = torch.empty((P, B, H, L.cpla_summary_width(pp)), **f32)
    pk, meta = None, None
    if wl.cu_seqlens is not None:
        meta = packed_meta(wl.cu_seqlens, T, P, dev, B)
        pk = ctypes.byref(meta.c())
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _lib.check(L.cp_forward_prepare(pp, pk, _ptr(k), _ptr(v), _ptr(g), _ptr(fsum), st))
    outs = []
    for noalloc in (False, True):
        o = torch.full_like(v, float("nan"))
        fin = torch.full((B, H, dk, dv), float("nan"), **f32)
        cs = torch.full((L.cpla_chunk_states_bytes(pp) // 4,), float("nan"), **f32)
        if noalloc:
            _lib.check(L.cp_forward_apply_noalloc(pp, pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(fsum),
                                                  _ptr(S0), _ptr(o), _ptr(fin), _ptr(cs), st))
        else:
            s_in = torch.empty((P, B, H, dk, dv), **f32)
            _lib.check(L.cp_forward_apply(pp, pk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(fsum), _ptr(S0),
                                          _ptr(o), _ptr(s_in), _ptr(fin), _ptr(cs), st))
        outs.append((o, fin, cs))
    torch.cuda.synchronize(dev)
    return outs


@pytest.mark.parametrize("first,second", [
    # the full diagonal-decay workload (its composed states fill the 32 MiB scratch
    # exactly), then a smaller packed problem
    (("diag_fwdbwd", {}), ("packed_fwdbwd", dict(T=2048, H=2, num_shards=4, len_range=(30, 400)))),
    # scalar decay with an initial state, then a smaller uneven identity problem
    (("long_fwdbwd", dict(T=4096, H=4, num_shards=8)), ("identity_fwd", dict(T=300, num_shards=3))),
])
def test_noalloc_matches_forward_apply(first, second, gpu_available):
    dev = torch.device("cuda:0")
    for name, over in (first, second):
        print(f"[gpu-case] noalloc {name} {over}", file=sys.stderr, flush=True)
        wl = workloads.make(name, **over)
        (o, fin, cs), (o2, fin2, cs2) = _both(wl, dev)
        assert torch.equal(o, o2), "o"
        assert torch.equal(fin, fin2), "final_state"
        assert torch.equal(cs, cs2), "chunk_states"


def test_noalloc_rejects_oversize(gpu_available):
    L = _lib.lib()
    assert L.cpla_noalloc_scratch_bytes() == 32 << 20
    # 9 shards of the 32 MiB workload: 36 MiB of composed states
    p = _lib.Problem(B=4, T=8192, H=16, dk=128, dv=128, num_shards=9, chunk=64, rank_begin=0, rank_end=9,
                     dtype=_lib.BF16, decay=_lib.DECAY_DIAG)
    fake = 0x10000
    st = L.cp_forward_apply_noalloc(ctypes.byref(p), None, fake, fake, fake, fake, fake, None, fake, None, None, None)
    assert st == 5
    assert b"scratch holds" in L.cpla_last_error()
