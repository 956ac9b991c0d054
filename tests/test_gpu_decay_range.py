"""The diagonal-decay range check (cpla_check_decay_range) on the GPU.

The diagonal-decay kernels factor the decay inside a 64-token chunk as
exp(Gam_i) exp(-Gam_j); a chunk whose running log-decay falls below
CPLA_DIAG_GAMMA_MIN (-80) per key dim is outside the supported range, and the
check reports every such (chunk, key dim) pair. The counts below are computed
from the inputs on the host (running sums per chunk of each shard).
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from context_state_passing_amd import _lib, api
from context_state_passing_amd._lib import CplaError, Problem

pytestmark = pytest.mark.gpu


def _expected(g, P):
    """(chunk, key dim) pairs of the shards' 64-token chunks whose running sum of g
    falls below -80, by brute force over the torch.chunk division."""
    B, T, H, d = g.shape
    L = -(-T // P)
    bad = 0
    for r in range(P):
        t0, t1 = min(r * L, T), min((r + 1) * L, T)
        for c0 in range(t0, t1, 64):
            run = np.cumsum(g[:, c0:min(c0 + 64, t1)].astype(np.float64), axis=1)
            bad += int((run.min(axis=1) < -80.0).sum())
    return bad


def _count(g, P):
    B, T, H, d = g.shape
    p = Problem(B, T, H, d, d, P, 64, 0, P, _lib.BF16, _lib.DECAY_DIAG)
    cnt = torch.full((4,), -1, dtype=torch.int32, device=g.device)
    st = _lib.lib().cpla_check_decay_range(ctypes.byref(p), ctypes.c_void_p(g.data_ptr()),
                                           ctypes.c_void_p(cnt.data_ptr()),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, int(cnt[0].item())


@pytest.mark.parametrize("T,P,d", [(1024, 4, 128), (500, 3, 64), (1000, 16, 16)])
def test_decay_range_counts(T, P, d, gpu_available):
    print(f"[gpu-case] decay range T={T} P={P} d={d}", file=sys.stderr, flush=True)
    gen = torch.Generator().manual_seed(T + P)
    # mild decay everywhere (about -0.05 per token, as in the diagonal workload) ...
    g = torch.nn.functional.logsigmoid(torch.randn(2, T, 3, d, generator=gen)) / 16
    st, n = _count(g.cuda(), P)
    assert (st, n) == (0, 0)
    # ... then a few key dims of a few stretches at -2 per token (-128 over a chunk)
    g[0, 100:300, 1, : d // 4] = -2.0
    g[1, T - 70:, 2, 3] = -1.4
    exp = _expected(g.numpy(), P)
    assert exp > 0
    st, n = _count(g.cuda(), P)
    assert st == 1 and n == exp
    with pytest.raises(CplaError) as e:
        api.check_decay_range(g.cuda(), P)
    assert e.value.status == 1 and "out of range" in e.value.message


def test_decay_range_whole_stream_strong(gpu_available):
    # about -2 nats per token everywhere: every (chunk, key dim) pair of full chunks fails
    g = torch.full((1, 512, 2, 128), -2.0)
    st, n = _count(g.cuda(), 2)
    assert st == 1 and n == _expected(g.numpy(), 2) == 1 * 8 * 2 * 128
