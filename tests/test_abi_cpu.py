"""CPU tests of the C ABI: symbol exports, host-side validation (every case fails
before any launch, so no GPU is touched), the packed-metadata builder against
the oracle's brute-force twin (bit-exact), and product/oracle independence."""
import ctypes
import os
import re

import numpy as np
import pytest

from context_state_passing_amd import _lib
from context_state_passing_amd._lib import Packed, Problem
import context_state_passing_amd as cpla
from oracle import metadata as omd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = _lib.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "cpla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\*]+\s+\**\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("typedef",)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 11
    assert sorted(names) == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_peaks_library_exports():
    # the benchmark's attainable-peak probes (copy kernel, MFMA issue loops)
    P = ctypes.CDLL(os.path.join(ROOT, "context_state_passing_amd", "libcpla_peaks.so"))
    for n in ("cpla_peak_copy", "cpla_peak_mfma", "cpla_peak_mfma_flops"):
        assert hasattr(P, n), n
    P.cpla_peak_mfma_flops.restype = ctypes.c_int64
    assert [P.cpla_peak_mfma_flops(k) for k in (0, 1, 2, 3, 4)] == [8 * 16384, 8 * 2048, 8 * 2048, 4 * 32768, 0]
    # bad arguments are refused before any launch
    P.cpla_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    assert P.cpla_peak_copy(FAKE, FAKE, 15, 1, 0, None) == -1
    assert P.cpla_peak_copy(MISALIGNED, FAKE, 16, 1, 0, None) == -1
    assert P.cpla_peak_copy(FAKE, FAKE, 16, 1, 3, None) == -1


def test_noalloc_refuses_oversize_before_launch():
    assert L.cpla_noalloc_scratch_bytes() == 32 << 20
    p = prob(B=4, T=8192, H=16, num_shards=9, rank_end=9, decay=_lib.DECAY_DIAG)
    st = L.cp_forward_apply_noalloc(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
                                    None)
    assert st == 5 and b"scratch holds" in L.cpla_last_error()
    # an invalid problem is refused as by cp_forward_apply
    assert L.cp_forward_apply_noalloc(ctypes.byref(prob(B=0)), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                      None, None, None) == 2


def test_decay_range_check_host_paths():
    # nothing to check without a factorised decay: OK without launching
    assert L.cpla_check_decay_range(ctypes.byref(prob()), FAKE, FAKE, None) == 0
    assert L.cpla_check_decay_range(ctypes.byref(prob(decay=_lib.DECAY_NONE)), None, None, None) == 0
    # a diagonal decay needs g and a device count (checked before any launch)
    p = prob(decay=_lib.DECAY_DIAG)
    assert L.cpla_check_decay_range(ctypes.byref(p), None, FAKE, None) == 1
    assert L.cpla_check_decay_range(ctypes.byref(p), FAKE, None, None) == 1
    assert L.cpla_check_decay_range(ctypes.byref(p), MISALIGNED, FAKE, None) == 4
    assert L.cpla_check_decay_range(ctypes.byref(prob(B=0, decay=_lib.DECAY_DIAG)), FAKE, FAKE, None) == 2


def test_apply_parts_knob():
    assert L.cpla_set_apply_parts(3) == -1
    assert L.cpla_set_apply_parts(2) == 0
    assert L.cpla_set_apply_parts(0) == 2


def test_abi_version():
    assert L.cpla_abi_version() == 6


def prob(**kw):
    base = dict(B=1, T=1024, H=2, dk=128, dv=128, num_shards=4, chunk=64, rank_begin=0, rank_end=4,
                dtype=_lib.BF16, decay=_lib.DECAY_SCALAR)
    base.update(kw)
    return Problem(**base)


FAKE = 0x10000            # aligned, never dereferenced: validation fails before any launch
MISALIGNED = 0x10004


def fwd_prepare(p, k=FAKE, v=FAKE, g=FAKE, out=FAKE, packed=None):
    return L.cp_forward_prepare(ctypes.byref(p) if p is not None else None, packed, k, v, g, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(dtype=7), 3), (dict(decay=5), 1), (dict(chunk=32), 5), (dict(T=0), 2),
    (dict(T=64 * 1025, num_shards=1025), 5),
    (dict(rank_begin=2, rank_end=2), 1), (dict(rank_end=5), 1), (dict(dv=32), 5), (dict(dk=32, dv=32), 5),
    (dict(dk=64, dv=16), 5), (dict(dk=64, dv=128, dtype=_lib.F32), 5), (dict(dk=16, dv=128), 5),
    (dict(dtype=_lib.F32), 5), (dict(num_shards=0), 2),
    (dict(qk_heads=3), 2), (dict(qk_heads=-1), 2),     # q, k heads must divide H
    (dict(qk_heads=1, decay=_lib.DECAY_DIAG), 5), (dict(qk_heads=1, decay=_lib.DECAY_NONE), 5),   # scalar only
])
def test_problem_validation(kw, status):
    assert fwd_prepare(prob(**kw)) == status
    assert L.cpla_last_error()


def test_pointer_validation():
    p = prob()
    assert fwd_prepare(None) == 1
    assert fwd_prepare(p, k=None) == 1
    assert fwd_prepare(p, v=MISALIGNED) == 4
    assert fwd_prepare(p, g=None) == 1                              # scalar decay needs g
    assert fwd_prepare(prob(decay=_lib.DECAY_NONE), g=FAKE) == 1     # no decay: g must be NULL
    assert fwd_prepare(p, out=None) == 1
    assert b"NULL" in L.cpla_last_error() or L.cpla_last_error()


def test_packed_validation():
    pk = Packed(FAKE, FAKE, FAKE)
    assert fwd_prepare(prob(), packed=ctypes.byref(Packed(None, FAKE, FAKE))) == 1
    # B > 1 is accepted (one packing per row): the checks reach the same errors
    assert fwd_prepare(prob(B=2), packed=ctypes.byref(Packed(None, FAKE, FAKE))) == 1
    p = prob(B=3)
    # initial_state with packed sequences
    st = L.cp_forward_apply(ctypes.byref(p), ctypes.byref(pk), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, None)
    assert st == 1
    # d_final_state with packed sequences
    st = L.cp_backward_apply(ctypes.byref(p), ctypes.byref(pk), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == 1


def test_backward_requires_chunk_states_and_dg():
    p = prob()
    st = L.cp_backward_apply(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                             FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == 1 and b"chunk_states" in L.cpla_last_error()
    st = L.cp_backward_apply(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                             FAKE, FAKE, FAKE, None, FAKE, None, None)
    assert st == 1 and b"dg" in L.cpla_last_error()


def test_sizes():
    p = prob(decay=_lib.DECAY_DIAG)
    assert L.cpla_summary_width(ctypes.byref(p)) == 128 + 128 * 128
    p = prob(decay=_lib.DECAY_SCALAR)
    assert L.cpla_summary_width(ctypes.byref(p)) == 4 + 128 * 128
    assert L.cpla_chunk_states_bytes(ctypes.byref(p)) == 1 * 2 * (1024 // 64) * 128 * 128 * 4
    # uneven division: 1000 tokens on 3 shards are 334 + 334 + 332 -> 6 + 6 + 6 chunks;
    # 200 tokens on 64 shards are 50 shards of 4 (one chunk each) and 14 empty ones
    for T, P, chunks in [(1000, 3, 18), (200, 64, 50), (1000, 1, 16), (65, 2, 2)]:
        p = prob(T=T, num_shards=P, rank_end=P)
        assert L.cpla_chunk_states_bytes(ctypes.byref(p)) == 2 * chunks * 128 * 128 * 4, (T, P)


def test_uneven_division_is_accepted():
    for T, P in [(1000, 3), (200, 64), (7, 4), (1, 8)]:
        # validation passes, so the call reaches the (absent) pointers' checks
        assert fwd_prepare(prob(T=T, num_shards=P, rank_end=P), k=None) == 1
        assert b"k is NULL" in L.cpla_last_error()


# ---- packed metadata: C++ builder == oracle twin, bit-exact --------------------------------

def random_stream(rng, T, lo, hi):
    lens = []
    while sum(lens) < T:
        lens.append(int(rng.integers(lo, hi + 1)))
    lens[-1] -= sum(lens) - T
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return cu


@pytest.mark.parametrize("seed", range(6))
def test_metadata_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    T, P = 4096, 16
    cu = random_stream(rng, T, [1, 128, 64][seed % 3], [300, 4096, 64][seed % 3])
    s_c = cpla.seq_idx_from_cu_seqlens(cu, T)
    s_o = omd.seq_idx_from_cu_seqlens(cu, T)
    assert np.array_equal(s_c, s_o)
    prs, frs = cpla.packed_rank_slices(s_c, P)
    prs_o, frs_o = omd.rank_slices(s_o, P)
    assert np.array_equal(prs, prs_o) and np.array_equal(frs, frs_o)
    for r in range(P):
        a = cpla.build_packed_sequence_cp_metadata(s_c, r, P)
        b = omd.build_packed_sequence_cp_metadata(s_o, r, P)
        assert np.array_equal(a["local_seq_idx"], b["local_seq_idx"])
        assert np.array_equal(a["local_cu_seqlens"], b["local_cu_seqlens"])
        assert a["preceding_rank_start"] == b["preceding_rank_start"]
        assert a["following_rank_stop"] == b["following_rank_stop"]


@pytest.mark.parametrize("T,P", [(4000, 16), (4000, 7), (10, 4), (9, 4), (5, 8), (130, 64)])
def test_metadata_uneven_matches_oracle(T, P):
    rng = np.random.default_rng(T + P)
    cu = random_stream(rng, T, 1, max(2, T // 5))
    s = cpla.seq_idx_from_cu_seqlens(cu, T)
    prs, frs = cpla.packed_rank_slices(s, P)
    prs_o, frs_o = omd.rank_slices(s, P)
    assert np.array_equal(prs, prs_o) and np.array_equal(frs, frs_o)
    for r in range(P):
        a = cpla.build_packed_sequence_cp_metadata(s, r, P)
        b = omd.build_packed_sequence_cp_metadata(s, r, P)
        for key in a:
            assert np.array_equal(a[key], b[key]), (key, r)


def test_metadata_edge_cases_match_oracle():
    cases = [np.zeros(64, np.int32),                                 # one sequence everywhere
             np.repeat(np.arange(4), 16).astype(np.int32),           # starts exactly at rank starts
             np.arange(64).astype(np.int32),                         # every token its own sequence
             np.concatenate([np.zeros(63), [1]]).astype(np.int32)]   # last sequence of length 1
    for s in cases:
        for r in range(4):
            a = cpla.build_packed_sequence_cp_metadata(s, r, 4)
            b = omd.build_packed_sequence_cp_metadata(s, r, 4)
            for key in a:
                assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("bad", [[1, 1, 1, 1], [0, 2, 2, 2], [0, 1, 0, 1]])
def test_metadata_rejects_malformed(bad):
    with pytest.raises(cpla.CplaError) as e:
        cpla.build_packed_sequence_cp_metadata(np.array(bad, np.int32), 0, 2)
    assert e.value.status == 6


def test_cu_seqlens_rejects_malformed():
    with pytest.raises(cpla.CplaError):
        cpla.seq_idx_from_cu_seqlens([0, 3, 3, 8], 8)
    with pytest.raises(cpla.CplaError):
        cpla.seq_idx_from_cu_seqlens([1, 8], 8)


# ---- independence ------------------------------------------------------------------------

def test_product_does_not_use_oracle():
    pkg = os.path.join(ROOT, "context_state_passing_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, flags=re.M), f
                assert "oracle/" not in text, f


def test_per_row_packed_metadata_matches_oracle():
    """packed_meta with one cu_seqlens per batch row: [B, T] ids and [B, P] slices,
    each row equal to the oracle's metadata for that row alone."""
    from context_state_passing_amd.api import packed_meta
    T, P = 300, 7
    cus = [[0, 5, 120, 300], [0, 300], [0, 1, 2, 3, 299, 300]]
    m = packed_meta(cus, T, P, "cpu", B=3)
    assert tuple(m.seq_idx.shape) == (3, T) and tuple(m.preceding_rank_start.shape) == (3, P)
    for b, cu in enumerate(cus):
        s = omd.seq_idx_from_cu_seqlens(np.array(cu), T)
        prs, frs = omd.rank_slices(s, P)
        assert np.array_equal(m.seq_idx[b].numpy(), s)
        assert np.array_equal(m.preceding_rank_start[b].numpy(), prs)
        assert np.array_equal(m.following_rank_stop[b].numpy(), frs)
    assert np.array_equal(omd.seq_idx_rows(cus, T), m.seq_idx.numpy())
    one = packed_meta(np.array(cus[0]), T, P, "cpu")
    assert tuple(one.seq_idx.shape) == (1, T)
    with pytest.raises(cpla.CplaError):
        packed_meta(cus, T, P, "cpu", B=2)


def test_delta_validation():
    """The _delta calls check their problem before any launch; the other calls
    refuse the delta decay; the workspace size follows its layout."""
    p = prob(dk=64, dv=64, dtype=_lib.F32, decay=_lib.DECAY_DELTA, T=1000, num_shards=3, rank_end=3)
    nct = 3 * 6         # shards of 334, 334 and 332 tokens: 6 chunks each
    tok = 1 * 1000 * 2 * 64
    assert L.cpla_delta_workspace_bytes(ctypes.byref(p)) == 4 * (4 * tok + 2 * 1 * 2 * nct * 64 * 64)
    assert L.cpla_summary_width(ctypes.byref(p)) == 2 * 64 * 64
    for bad in [dict(dk=128, dv=128), dict(dk=64, dv=32), dict(decay=_lib.DECAY_DIAG), dict(chunk=32),
                dict(num_shards=1025, rank_end=1025), dict(qk_heads=1)]:
        base = dict(dk=64, dv=64, dtype=_lib.F32, decay=_lib.DECAY_DELTA)
        base.update(bad)
        q = prob(**base)
        assert L.cpla_delta_workspace_bytes(ctypes.byref(q)) == -1, bad
        st = L.cp_forward_prepare_delta(ctypes.byref(q), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
        assert st in (1, 5), (bad, st)
    # d = 128 is taken in bf16 (fp32 is refused above); other head sizes are not
    wide = prob(dk=128, dv=128, dtype=_lib.BF16, decay=_lib.DECAY_DELTA, T=1000, num_shards=3, rank_end=3)
    assert L.cpla_delta_workspace_bytes(ctypes.byref(wide)) == 4 * (4 * 2 * tok + 2 * 1 * 2 * nct * 128 * 128)
    odd = prob(dk=96, dv=96, dtype=_lib.BF16, decay=_lib.DECAY_DELTA)
    assert L.cpla_delta_workspace_bytes(ctypes.byref(odd)) == -1
    # a NULL workspace or beta is refused before any launch
    assert L.cp_forward_prepare_delta(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert L.cp_forward_prepare_delta(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    # the linear-attention calls refuse the delta decay
    assert fwd_prepare(p) == 1


def ssd_prob(**kw):
    base = dict(B=1, T=256, H=4, G=2, N=128, P=64, dtype=_lib.BF16)
    base.update(kw)
    return _lib.SsdProblem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(G=3), 2), (dict(dtype=9), 3), (dict(N=12), 5), (dict(N=512), 5),
    (dict(P=0), 5), (dict(P=66), 5), (dict(P=260), 5),
])
def test_ssd_problem_validation(kw, status):
    # state size N and head dim P are separate fields; bad shapes fail before any launch
    p = ssd_prob(**kw)
    assert L.cpla_ssd_inputs(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == status
    assert L.cpla_last_error()
    assert L.cpla_ssd_input_grads(ctypes.byref(p), *([FAKE] * 12), None) == status


def test_ssd_pointer_validation():
    p = ssd_prob()
    assert L.cpla_ssd_inputs(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.cpla_ssd_inputs(ctypes.byref(p), FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE, None) == 4
    # per-head copies q, k: both or neither; without them B and C are not read here
    assert L.cpla_ssd_inputs(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert L.cpla_ssd_inputs(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, None) == 1   # g
    assert L.cpla_ssd_inputs(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, None, FAKE, None) == 1   # dt
