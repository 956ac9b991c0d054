"""Packed-sequence metadata, brute force from the field definitions (oracle; test use only).

Megatron-Core API page ``core.ssm.context_parallel.chunkwise``, class
``PackedSequenceCPMetadata`` and function ``build_packed_sequence_cp_metadata``
(arguments: global per-token sequence ids, the CP rank and the CP size). The
fields are:

* ``local_seq_idx``     per-token sequence ids of the rank's contiguous shard;
* ``local_cu_seqlens``  sequence boundaries inside that shard;
* ``preceding_rank_start``  inclusive start of the ranks whose forward summaries
  rank r composes (the prefix runs over ranks [start, r));
* ``following_rank_stop``   exclusive end of the ranks whose backward summaries
  rank r composes (the suffix runs over ranks (r, stop)).

Readings where the page is silent: shards are the cp_size contiguous slices of
the stream that torch.chunk makes (ceil(T / cp_size) tokens each, the last
non-empty one shorter, trailing ones empty when the stream is short — the
graceful division the mixle page relies on); an empty shard has no local
tokens and no sequences (local_cu_seqlens [0]), and composes nothing (prefix
start r, suffix stop r + 1); local ids are rebased so
the shard's first token has id 0; local_cu_seqlens lists 0, every interior
position where the id changes, and the shard length; the prefix starts at the
rank holding the first token of the sequence that is live at the shard's first
token, and the suffix stops after the rank holding the last token of the
sequence live at the shard's last token. A valid global id array starts at 0
and steps by 0 or 1 (the form cu_seqlens produces).
"""
from __future__ import annotations

import numpy as np


class MetadataError(ValueError):
    pass


def seq_idx_from_cu_seqlens(cu_seqlens, T):
    """Sequence id of every token: token t belongs to sequence s iff cu[s] <= t < cu[s+1]."""
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    if len(cu) < 2 or cu[0] != 0 or cu[-1] != T:
        raise MetadataError("cu_seqlens must start at 0 and end at T")
    out = np.full(T, -1, dtype=np.int32)
    for s in range(len(cu) - 1):
        if cu[s + 1] <= cu[s]:
            raise MetadataError("cu_seqlens must be strictly increasing")
        for t in range(cu[s], cu[s + 1]):
            out[t] = s
    return out


def seq_idx_rows(cu_seqlens, T):
    """[T] ids from one cu_seqlens, or [B, T] from a list of B of them (one
    packing per batch row)."""
    if isinstance(cu_seqlens, (list, tuple)) and len(cu_seqlens) and np.ndim(cu_seqlens[0]) == 1:
        return np.stack([seq_idx_from_cu_seqlens(np.asarray(c), T) for c in cu_seqlens])
    return seq_idx_from_cu_seqlens(np.asarray(cu_seqlens), T)


def validate_global_seq_idx(global_seq_idx, cp_size):
    s = [int(x) for x in np.asarray(global_seq_idx).tolist()]
    T = len(s)
    if cp_size <= 0 or T == 0:
        raise MetadataError("stream length and cp_size must be positive")
    if s[0] != 0:
        raise MetadataError("global_seq_idx must start at 0")
    for t in range(1, T):
        if s[t] - s[t - 1] not in (0, 1):
            raise MetadataError("global_seq_idx must step by 0 or 1")
    return s


def build_packed_sequence_cp_metadata(global_seq_idx, cp_rank, cp_size):
    s = validate_global_seq_idx(global_seq_idx, cp_size)
    if not 0 <= cp_rank < cp_size:
        raise MetadataError("cp_rank out of range")
    T = len(s)
    size = -(-T // cp_size)                  # torch.chunk's part size
    a = min(cp_rank * size, T)
    L = min(size, T - a)
    if L == 0:
        return {"local_seq_idx": np.zeros(0, dtype=np.int32), "local_cu_seqlens": np.zeros(1, dtype=np.int32),
                "preceding_rank_start": cp_rank, "following_rank_stop": cp_rank + 1}
    e = a + L - 1
    local = [s[t] - s[a] for t in range(a, a + L)]
    cu = [0]
    for i in range(1, L):
        if s[a + i] != s[a + i - 1]:
            cu.append(i)
    cu.append(L)
    first_of = min(t for t in range(T) if s[t] == s[a])
    last_of = max(t for t in range(T) if s[t] == s[e])
    return {
        "local_seq_idx": np.array(local, dtype=np.int32),
        "local_cu_seqlens": np.array(cu, dtype=np.int32),
        "preceding_rank_start": first_of // size,
        "following_rank_stop": last_of // size + 1,
    }


def rank_slices(global_seq_idx, cp_size):
    """(preceding_rank_start[r], following_rank_stop[r]) for every rank."""
    prs, frs = [], []
    for r in range(cp_size):
        m = build_packed_sequence_cp_metadata(global_seq_idx, r, cp_size)
        prs.append(m["preceding_rank_start"])
        frs.append(m["following_rank_stop"])
    return np.array(prs, dtype=np.int32), np.array(frs, dtype=np.int32)
