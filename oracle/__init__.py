"""Plain, slow, fp64 CPU oracle for chunkwise context-parallel linear attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP path (no kernels, headers, helpers or constant tables); the only thing both
sides consume is the seeded input generator in ``workloads``.

What it computes, and the passages it follows
---------------------------------------------
Megatron-Core API page ``core.ssm.context_parallel.chunkwise``:

* classes ``CPForwardUnpackedSummary`` / ``CPForwardPackedSummary``: a shard's
  summary is the affine map ``S_out = M S_in + delta_S``;
* classes ``CPBackwardUnpackedSummary`` / ``CPBackwardPackedSummary``: the
  adjoint map ``dS_in = M^T dS_out + gamma``;
* ``LinearAttentionCPBackend.cp_forward_prepare``: the summary is taken with zero
  incoming state; ``cp_forward_apply``: compose the preceding summaries, then
  emit the local output; ``cp_backward_prepare``: gamma with zero outgoing-state
  gradient; ``cp_backward_apply``: compose the reverse-causal suffix, then finish
  the local input gradients;
* ``PackedSequenceCPMetadata`` and ``build_packed_sequence_cp_metadata``: the
  rank-local packed-sequence fields, including the inclusive start of the
  forward prefix and the exclusive end of the backward suffix.

The per-token recurrence inside a shard (the "local kernel" that page leaves to
the backend) is gated causal linear attention: ``S_t = diag(exp(g_t)) S_{t-1} +
k_t v_t^T`` and ``o_t = S_t^T q_t``, with the decay either absent, a scalar per
(b, t, h) or a vector over the key dimension, and the state reset to zero at
every packed-sequence start.

Modules
-------
``recurrence``  per-token forward and adjoint recurrences (the definition).
``cp``          shard summaries, prefix/suffix composition, and the whole CP
                method run through them.
``metadata``    sequence ids from cu_seqlens and the rank-local packed metadata.
``chunked``     the chunk algebra (intra-chunk matrices + carried state) in
                fp64, used by the tests to check it against the recurrence.

Pins (what checks this oracle against something other than itself) live in
``tests/test_oracle_*.py``: the O(T^2) closed form, brute-force finite
differences, packed == separate sequences, sharded == unsharded, and the
metadata fields recomputed from their stated definitions.
"""
from . import recurrence, cp, metadata, chunked  # noqa: F401
from .recurrence import forward, backward  # noqa: F401
