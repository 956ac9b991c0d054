"""The benchmark's attainable-peak probes (libcpla_peaks.so) on the GPU.

bench.py prices its kernels against a streaming copy and MFMA issue loops of
its own; these tests check that the copy copies (every variant, grid sizes that
leave a ragged tail) and that the MFMA loops run and accumulate what they issue
(the sums grow linearly with the iteration count and repeat bitwise).
"""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    P = ctypes.CDLL(os.path.join(ROOT, "context_state_passing_amd", "libcpla_peaks.so"))
    P.cpla_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    P.cpla_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return P


@pytest.mark.parametrize("variant", [0, 1, 2])
@pytest.mark.parametrize("n16,blocks", [(1, 1), (1000, 3), (65536 + 37, 7), (1 << 18, 1024)])
def test_copy_copies(variant, n16, blocks):
    P = _lib()
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(n16 + blocks)
    src = torch.randint(-2**31, 2**31 - 1, (4 * n16,), generator=g, dtype=torch.int32).to(dev)
    dst = torch.zeros_like(src)
    guard = torch.full((64,), 7, dtype=torch.int32, device=dev)   # the copy must not run past its end
    out = torch.cat([dst, guard])
    s = torch.cuda.current_stream()
    assert P.cpla_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(out.data_ptr()), 16 * n16, blocks,
                            variant, ctypes.c_void_p(s.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert torch.equal(out[:4 * n16], src)
    assert torch.equal(out[4 * n16:], guard)


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_mfma_loops_accumulate(kind):
    P = _lib()
    dev = torch.device("cuda:0")
    blocks = 8
    s = torch.cuda.current_stream()
    sums = []
    for iters in (16, 32, 32):
        out = torch.zeros(blocks * 256, device=dev)
        assert P.cpla_peak_mfma(kind, ctypes.c_void_p(out.data_ptr()), blocks, iters,
                                ctypes.c_void_p(s.cuda_stream)) == 0
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        sums.append(out.double())
    assert (sums[0].abs() > 0).all()
    assert torch.equal(sums[1], sums[2])
    assert torch.allclose(sums[1], 2 * sums[0], rtol=1e-2, atol=0)
