"""Chunkwise context-parallel causal linear attention with carried state, for MI355X.

Product path: ``libcpla.so`` (HIP kernels for gfx950 behind a C ABI, declared in
``include/cpla.h``) and a thin ctypes binding. Importing this package loads the
library and fails loudly if it has not been built.
"""
from ._lib import CplaError, lib  # noqa: F401
from .api import (  # noqa: F401
    Context, DeltaContext, PackedMeta, SsdContext, backward, build_packed_sequence_cp_metadata,
    chunkwise_linear_attention, delta_backward, delta_forward, forward, gated_delta_rule, mamba2_ssd, packed_meta,
    packed_rank_slices, seq_idx_from_cu_seqlens, ssd_backward, ssd_forward)

lib()
