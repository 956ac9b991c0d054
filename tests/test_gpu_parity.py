"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element, for outputs, gradients and the
intermediate summaries / composed states.

Small cases keep every workload's distributions and head size but shrink B, T,
H so the oracle finishes in seconds; they still span several chunks per shard,
several shards, and packed sequences with boundaries inside chunks. Full-size
cases run the exact benchmark shapes on the GPU and compare sampled heads, which
the oracle computes independently.
"""
import sys

import pytest
import torch

import workloads
from _parity import compare, gpu_run, oracle_run

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[gpu-case] {name}", file=sys.stderr, flush=True)


SMALL = {
    # name: (workload, overrides, backward)
    "identity_fwd_full": ("identity_fwd", {}, False),
    "identity_fp32_bwd": ("identity_fwd", {"backward": True}, True),
    # fp32 without decay, where sums grow with the stream (|dq| reaches ~50): the
    # fp32 bound must hold far beyond the 256-token workload
    "identity_fp32_d64_T1024_bwd": ("identity_fwd", {"B": 1, "H": 2, "T": 1024, "d": 64, "num_shards": 4,
                                                     "backward": True}, True),
    "identity_fp32_d64_T657_bwd": ("identity_fwd", {"B": 2, "H": 1, "T": 657, "d": 64, "num_shards": 5,
                                                    "backward": True}, True),
    "identity_fp32_d16_T2048_bwd": ("identity_fwd", {"B": 1, "H": 2, "T": 2048, "num_shards": 8,
                                                     "backward": True}, True),
    "scalar_fp32_d64_bwd": ("scalar_fwd", {"B": 1, "H": 2, "T": 512, "num_shards": 4, "backward": True,
                                           "dtype": torch.float32}, True),
    "diag_fp32_d64_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 256, "d": 64, "num_shards": 2,
                                         "dtype": torch.float32}, True),
    "scalar_small_fwd": ("scalar_fwd", {"B": 2, "H": 2, "T": 1024, "num_shards": 4}, False),
    "scalar_small_bwd": ("scalar_fwd", {"B": 1, "H": 2, "T": 1024, "num_shards": 4, "backward": True}, True),
    "scalar_weak_bwd": ("scalar_fwd", {"B": 1, "H": 2, "T": 1024, "num_shards": 4, "backward": True,
                                       "decay_scale": 1e-3}, True),
    "diag_small_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 512, "num_shards": 4}, True),
    "diag_weak_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 512, "num_shards": 4, "decay_scale": 1e-3}, True),
    "diag_d64_bwd": ("diag_fwdbwd", {"B": 2, "H": 1, "T": 512, "d": 64, "num_shards": 2}, True),
    "packed_small_bwd": ("packed_fwdbwd", {"T": 2048, "H": 2, "num_shards": 4, "len_range": (100, 700)}, True),
    "packed_short_seqs_bwd": ("packed_fwdbwd", {"T": 1024, "H": 2, "num_shards": 4, "len_range": (1, 70)}, True),
    "packed_weak_bwd": ("packed_fwdbwd", {"T": 2048, "H": 2, "num_shards": 8, "len_range": (100, 900),
                                          "decay_scale": 1e-3}, True),
    "long_small_bwd": ("long_fwdbwd", {"T": 1024, "H": 2, "num_shards": 4}, True),
    "long_weak_bwd": ("long_fwdbwd", {"T": 1024, "H": 2, "num_shards": 4, "decay_scale": 1e-3}, True),
    "single_shard_bwd": ("diag_fwdbwd", {"B": 1, "H": 1, "T": 256, "num_shards": 1}, True),
    "scalar_d16_bf16_bwd": ("scalar_fwd", {"B": 1, "H": 2, "T": 512, "d": 16, "num_shards": 2,
                                           "backward": True}, True),
    # edge cases: one chunk per shard; 64 shards; no decay at d=128 bf16;
    # diagonal decay at d=16 in both dtypes; many (b, h) rows
    "one_chunk_shards_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 256, "num_shards": 4}, True),
    "max_shards_bwd": ("scalar_fwd", {"B": 1, "H": 1, "T": 4096, "d": 16, "num_shards": 64,
                                      "backward": True}, True),
    "identity_d128_bf16_bwd": ("identity_fwd", {"B": 1, "H": 2, "T": 512, "d": 128, "num_shards": 2,
                                                "backward": True, "dtype": torch.bfloat16}, True),
    "diag_d16_bf16_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 512, "d": 16, "num_shards": 4}, True),
    "diag_d16_fp32_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 256, "d": 16, "num_shards": 2,
                                          "dtype": torch.float32}, True),
    "many_rows_bwd": ("scalar_fwd", {"B": 3, "H": 40, "T": 128, "d": 16, "num_shards": 2,
                                     "backward": True}, True),
    # packed edge cases: every start on a chunk (and shard) boundary; one token per
    # sequence (every chunk holds 64 starts); one sequence covering the whole stream
    "packed_aligned_bwd": ("packed_fwdbwd", {"T": 1024, "H": 2, "num_shards": 4, "len_range": (128, 128)}, True),
    "packed_len1_bwd": ("packed_fwdbwd", {"T": 256, "H": 1, "num_shards": 2, "len_range": (1, 1)}, True),
    "packed_one_seq_bwd": ("packed_fwdbwd", {"T": 1024, "H": 2, "num_shards": 4, "len_range": (4096, 4096)},
                           True),
    # uneven division (torch.chunk) and partial last chunks: shards of 167/167/166
    # tokens; weak decay so the composition across the uneven shards matters;
    # shards shorter than one chunk (63 tokens, the last 55); 64 shards of 4 tokens
    # with 14 empty; a single shard of 100 tokens (64 + 36); packed streams with
    # shards of 143 tokens; d = 64 / 16 in both dtypes
    "uneven_diag_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 500, "num_shards": 3}, True),
    "uneven_diag_weak_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 700, "num_shards": 5,
                                             "decay_scale": 1e-3}, True),
    "uneven_subchunk_shards_bwd": ("diag_fwdbwd", {"B": 1, "H": 1, "T": 1000, "num_shards": 16}, True),
    "uneven_empty_shards_bwd": ("scalar_fwd", {"B": 1, "H": 2, "T": 200, "num_shards": 64, "backward": True,
                                               "decay_scale": 1e-2}, True),
    # many shards: 256 of one chunk each; 200 uneven shards over packed sequences
    # with the diagonal decay; the largest count, 1024 shards of 2 tokens
    "many_shards_bwd": ("scalar_fwd", {"B": 1, "H": 2, "T": 16384, "d": 16, "num_shards": 256,
                                       "backward": True, "decay_scale": 1e-2}, True),
    "many_shards_packed_diag_bwd": ("diag_fwdbwd", {"B": 1, "H": 1, "T": 6000, "d": 64, "num_shards": 200,
                                                    "packed": True, "len_range": (30, 900),
                                                    "decay_scale": 1e-2}, True),
    "max_shards_1024_bwd": ("scalar_fwd", {"B": 1, "H": 1, "T": 2048, "d": 16, "num_shards": 1024,
                                           "backward": True, "decay_scale": 1e-3}, True),
    "tail_identity_fp32_bwd": ("identity_fwd", {"T": 100, "num_shards": 1, "backward": True}, True),
    "uneven_packed_bwd": ("packed_fwdbwd", {"T": 1000, "H": 2, "num_shards": 7, "len_range": (40, 300)}, True),
    "uneven_diag_d64_bwd": ("diag_fwdbwd", {"B": 2, "H": 1, "T": 450, "d": 64, "num_shards": 2}, True),
    "uneven_diag_d16_fp32_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 300, "d": 16, "num_shards": 4,
                                                 "dtype": torch.float32}, True),
    "uneven_long_init_bwd": ("long_fwdbwd", {"T": 777, "H": 2, "num_shards": 3}, True),
    # one packing per batch row: rows with different boundaries (and slices); with
    # uneven shards and sequences of 1..200 tokens; the diagonal decay packed
    "rows_packed_bwd": ("packed_fwdbwd", {"B": 3, "T": 1024, "H": 2, "num_shards": 4, "len_range": (40, 400)},
                        True),
    "rows_packed_uneven_bwd": ("packed_fwdbwd", {"B": 2, "T": 1000, "H": 2, "num_shards": 5,
                                                 "len_range": (1, 200)}, True),
    "rows_packed_diag_bwd": ("diag_fwdbwd", {"B": 2, "T": 768, "H": 2, "num_shards": 4, "packed": True,
                                             "len_range": (30, 300)}, True),
    # the diagonal decay over packed sequences: one stream, bf16 d_k 128 / fp32 d_k 64,
    # and a single sequence (its only start is token 0)
    "packed_diag_bwd": ("diag_fwdbwd", {"B": 1, "T": 1024, "H": 2, "num_shards": 4, "packed": True,
                                        "len_range": (30, 300)}, True),
    "packed_diag_d64_fp32_bwd": ("diag_fwdbwd", {"B": 1, "T": 512, "H": 2, "d": 64, "num_shards": 2,
                                                 "packed": True, "len_range": (20, 200),
                                                 "dtype": torch.float32}, True),
    "packed_diag_one_seq_bwd": ("diag_fwdbwd", {"B": 1, "T": 256, "H": 1, "d": 64, "num_shards": 1,
                                                "packed": True, "len_range": (256, 256)}, True),
    # d_k != d_v (bf16 64/128 and 128/64): every decay, uneven shards with partial
    # last chunks, packed streams, a nonzero initial state, weak decay
    "mixed_none_k64_v128_bwd": ("identity_fwd", {"B": 1, "H": 2, "T": 512, "d": 64, "dv": 128, "num_shards": 2,
                                                 "backward": True, "dtype": torch.bfloat16}, True),
    "mixed_none_k128_v64_bwd": ("identity_fwd", {"B": 1, "H": 2, "T": 500, "d": 128, "dv": 64, "num_shards": 3,
                                                 "backward": True, "dtype": torch.bfloat16}, True),
    "mixed_scalar_k64_v128_bwd": ("scalar_fwd", {"B": 2, "H": 1, "T": 700, "d": 64, "dv": 128, "num_shards": 3,
                                                 "backward": True}, True),
    "mixed_scalar_k128_v64_weak_bwd": ("scalar_fwd", {"B": 1, "H": 2, "T": 1024, "d": 128, "dv": 64,
                                                      "num_shards": 4, "backward": True, "decay_scale": 1e-3},
                                       True),
    "mixed_diag_k64_v128_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 512, "d": 64, "dv": 128, "num_shards": 4},
                                True),
    "mixed_diag_k128_v64_bwd": ("diag_fwdbwd", {"B": 1, "H": 2, "T": 600, "d": 128, "dv": 64, "num_shards": 3},
                                True),
    "mixed_diag_k128_v64_weak_bwd": ("diag_fwdbwd", {"B": 2, "H": 1, "T": 512, "d": 128, "dv": 64,
                                                     "num_shards": 4, "decay_scale": 1e-3}, True),
    "mixed_packed_k128_v64_bwd": ("packed_fwdbwd", {"T": 1024, "H": 2, "d": 128, "dv": 64, "num_shards": 4,
                                                    "len_range": (30, 300)}, True),
    "mixed_packed_diag_k64_v128_bwd": ("diag_fwdbwd", {"B": 2, "T": 512, "H": 1, "d": 64, "dv": 128,
                                                       "num_shards": 3, "packed": True, "len_range": (20, 200)},
                                       True),
    "mixed_long_init_k128_v64_bwd": ("long_fwdbwd", {"T": 777, "H": 2, "d": 128, "dv": 64, "num_shards": 3},
                                     True),
    "mixed_long_init_k64_v128_bwd": ("long_fwdbwd", {"T": 512, "H": 2, "d": 64, "dv": 128, "num_shards": 2},
                                     True),
}


@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_parity(case, gpu_available):
    name, ov, bwd = SMALL[case]
    _announce(case)
    wl = workloads.make(name, **ov)
    got = gpu_run(wl, backward=bwd)
    ref = oracle_run(wl, backward=bwd)
    compare(wl, got, ref, backward=bwd)


def test_d_final_state(gpu_available):
    _announce("diag_small_dfinal")
    wl = workloads.make("diag_fwdbwd", B=1, H=2, T=512, num_shards=4, decay_scale=1e-2)
    dSf = torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(7))
    got = gpu_run(wl, backward=True, d_final_state=dSf)
    ref = oracle_run(wl, backward=True, d_final_state=dSf)
    compare(wl, got, ref, backward=True)


def test_scalar_fwd_full_size(gpu_available):
    _announce("scalar_fwd_full")
    wl = workloads.make("scalar_fwd")
    got = gpu_run(wl, backward=False)
    ref = oracle_run(wl, backward=False)
    compare(wl, got, ref, backward=False)


def test_deterministic(gpu_available):
    _announce("determinism")
    wl = workloads.make("packed_fwdbwd", T=2048, H=2, num_shards=4, len_range=(100, 700))
    a = gpu_run(wl, backward=True)
    b = gpu_run(wl, backward=True)
    for key in a:
        if a[key] is not None:
            assert (a[key] == b[key]).all(), key


FULL = [
    # full benchmark shapes; the oracle recomputes the sampled heads of every batch row
    ("diag_fwdbwd", [0, 15]),
    ("packed_fwdbwd", [0, 15]),
    ("long_fwdbwd", [7]),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,heads", FULL)
def test_full_size_sampled_heads(name, heads, gpu_available):
    _announce(f"full {name} heads {heads}")
    wl = workloads.make(name)
    got = gpu_run(wl, backward=True, heads=heads)
    ref = oracle_run(wl, backward=True, heads=heads)
    compare(wl, got, ref, backward=True)


@pytest.mark.parametrize("name,over", [
    ("scalar_fwd", dict(B=1, H=2, T=1000, num_shards=8, backward=True)),
    ("identity_fwd", dict(B=1, H=2, T=1000, d=64, num_shards=8, backward=True, dtype=torch.bfloat16)),
    ("packed_fwdbwd", dict(B=1, H=2, T=1000, d=64, num_shards=8, len_range=(30, 300))),
    ("scalar_fwd", dict(B=1, H=2, T=900, d=64, num_shards=3, backward=True, dtype=torch.float32)),
])
def test_divided_walks_bitwise(name, over, gpu_available):
    # The apply walks of small grids divide each shard among Z workgroups (no decay
    # or a scalar decay), each replaying the state or adjoint up to its own chunks
    # from the shard's boundary value; every division must give the bits of the
    # undivided walk. Z is forced to 1, 2 and 4 through the library's testing knob.
    from context_state_passing_amd import _lib
    _announce(f"divided walks {name}")
    wl = workloads.make(name, **over)
    runs = {}
    try:
        for z in (1, 2, 4):
            _lib.lib().cpla_set_apply_parts(z)
            runs[z] = gpu_run(wl, backward=True)
    finally:
        _lib.lib().cpla_set_apply_parts(0)
    for z in (2, 4):
        for key in ("o", "dq", "dk", "dv", "dg"):
            if runs[1][key] is None:
                continue
            assert (runs[1][key] == runs[z][key]).all(), (z, key)


def _sweep_cases(seed, n):
    """Seeded random problems over every decay, head-size pair and dtype, with
    uneven and empty shards, partial chunks, packing, S_init and weak decay."""
    import random
    rng = random.Random(seed)
    dims = [((16, 16), torch.float32), ((64, 64), torch.float32), ((16, 16), torch.bfloat16),
            ((64, 64), torch.bfloat16), ((128, 128), torch.bfloat16), ((64, 128), torch.bfloat16),
            ((128, 64), torch.bfloat16)]
    out = []
    for i in range(n):
        (dk, dv), dt = rng.choice(dims)
        decay = rng.choice(["none", "scalar", "diag"])
        T = rng.choice([rng.randint(1, 130), rng.randint(64, 700)])
        over = dict(B=rng.choice([1, 1, 2]), H=rng.choice([1, 2, 3]), T=T, d=dk, dv=dv,
                    num_shards=rng.randint(1, 9), dtype=dt, backward=True,
                    decay_scale=rng.choice([1.0, 1.0, 1e-2, 1e-3]))
        if rng.random() < 0.35:
            over.update(packed=True, len_range=(1, rng.randint(1, 300)))
        elif rng.random() < 0.4:
            over.update(with_initial_state=True)
        out.append(({"none": "identity_fwd", "scalar": "scalar_fwd", "diag": "diag_fwdbwd"}[decay], over))
    return out


@pytest.mark.parametrize("case", range(60))
def test_random_problems(case, gpu_available):
    name, over = _sweep_cases(2026, 60)[case]
    _announce(f"random {case}: {name} {over}")
    wl = workloads.make(name, **over)
    got = gpu_run(wl, backward=True)
    ref = oracle_run(wl, backward=True)
    compare(wl, got, ref, backward=True)
