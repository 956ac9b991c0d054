// Packed-sequence metadata (host, pure C++).
//
// Megatron-Core page core.ssm.context_parallel.chunkwise: function
// build_packed_sequence_cp_metadata and class PackedSequenceCPMetadata. Fields:
// rank-local per-token sequence ids, rank-local sequence boundaries, the
// inclusive start of the ranks whose forward summaries the rank composes, and
// the exclusive end of the ranks whose backward summaries it composes. Shards
// are torch.chunk's cp_size contiguous slices of the stream (shards.hpp): an
// empty trailing shard has no local tokens and no sequences (local_cu_seqlens
// {0}), and composes nothing (preceding_rank_start r, following_rank_stop r + 1).
//
// One O(T) sweep finds, for every token, the first and last index of its
// sequence; the per-rank fields follow from the rank's first and last token.
#include <stdint.h>

#include <vector>

#include "cpla.h"
#include "errors.hpp"
#include "shards.hpp"

namespace {

// Valid ids start at 0 and step by 0 or 1 (the form cu_seqlens produces).
cpla_status check_ids(const int32_t* s, int64_t T, int32_t cp_size) {
  if (!s) return cpla::fail(CPLA_E_INVALID, "global_seq_idx is NULL");
  if (cp_size <= 0 || T <= 0)
    return cpla::fail(CPLA_E_METADATA, "stream length %lld and cp_size %d must be positive", (long long)T, cp_size);
  if (s[0] != 0) return cpla::fail(CPLA_E_METADATA, "global_seq_idx[0] is %d, expected 0", s[0]);
  for (int64_t t = 1; t < T; ++t) {
    const int32_t step = s[t] - s[t - 1];
    if (step != 0 && step != 1)
      return cpla::fail(CPLA_E_METADATA, "global_seq_idx steps by %d at token %lld (must be 0 or 1)", step,
                        (long long)t);
  }
  return CPLA_OK;
}

// first[t] / last[t]: first and last token index of token t's sequence.
void seq_bounds(const int32_t* s, int64_t T, std::vector<int64_t>& first, std::vector<int64_t>& last) {
  first.resize(T);
  last.resize(T);
  int64_t f = 0;
  for (int64_t t = 0; t < T; ++t) {
    if (t > 0 && s[t] != s[t - 1]) f = t;
    first[t] = f;
  }
  int64_t e = T - 1;
  for (int64_t t = T - 1; t >= 0; --t) {
    if (t < T - 1 && s[t] != s[t + 1]) e = t;
    last[t] = e;
  }
}

}  // namespace

extern "C" cpla_status build_packed_sequence_cp_metadata(const int32_t* global_seq_idx, int64_t T,
                                                         int32_t cp_rank, int32_t cp_size,
                                                         int32_t* local_seq_idx, int32_t* local_cu_seqlens,
                                                         int32_t* num_local_seqs,
                                                         int32_t* preceding_rank_start,
                                                         int32_t* following_rank_stop) {
  cpla::clear_error();
  cpla_status st = check_ids(global_seq_idx, T, cp_size);
  if (st != CPLA_OK) return st;
  if (cp_rank < 0 || cp_rank >= cp_size)
    return cpla::fail(CPLA_E_INVALID, "cp_rank %d outside [0, %d)", cp_rank, cp_size);
  if (!local_seq_idx || !local_cu_seqlens || !num_local_seqs || !preceding_rank_start || !following_rank_stop)
    return cpla::fail(CPLA_E_INVALID, "an output pointer is NULL");
  const int64_t size = cpla::shard_size(T, cp_size), a = cpla::shard_begin(T, cp_size, cp_rank);
  const int64_t L = cpla::shard_len(T, cp_size, cp_rank), e = a + L - 1;
  if (L == 0) {
    local_cu_seqlens[0] = 0;
    *num_local_seqs = 0;
    *preceding_rank_start = cp_rank;
    *following_rank_stop = cp_rank + 1;
    return CPLA_OK;
  }
  const int32_t* s = global_seq_idx;
  int32_t n = 0;
  local_cu_seqlens[n++] = 0;
  for (int64_t i = 0; i < L; ++i) {
    local_seq_idx[i] = s[a + i] - s[a];
    if (i > 0 && s[a + i] != s[a + i - 1]) local_cu_seqlens[n++] = (int32_t)i;
  }
  local_cu_seqlens[n++] = (int32_t)L;
  *num_local_seqs = n - 1;
  // first token of the sequence live at a; last token of the sequence live at e
  int64_t f = a;
  while (f > 0 && s[f - 1] == s[a]) --f;
  int64_t z = e;
  while (z < T - 1 && s[z + 1] == s[e]) ++z;
  *preceding_rank_start = (int32_t)(f / size);
  *following_rank_stop = (int32_t)(z / size + 1);
  return CPLA_OK;
}

extern "C" cpla_status cpla_packed_rank_slices(const int32_t* global_seq_idx, int64_t T, int32_t cp_size,
                                               int32_t* preceding_rank_start, int32_t* following_rank_stop) {
  cpla::clear_error();
  cpla_status st = check_ids(global_seq_idx, T, cp_size);
  if (st != CPLA_OK) return st;
  if (!preceding_rank_start || !following_rank_stop) return cpla::fail(CPLA_E_INVALID, "an output pointer is NULL");
  std::vector<int64_t> first, last;
  seq_bounds(global_seq_idx, T, first, last);
  const int64_t size = cpla::shard_size(T, cp_size);
  for (int32_t r = 0; r < cp_size; ++r) {
    const int64_t a = cpla::shard_begin(T, cp_size, r), L = cpla::shard_len(T, cp_size, r);
    if (L == 0) {   // empty trailing shard: composes nothing
      preceding_rank_start[r] = r;
      following_rank_stop[r] = r + 1;
      continue;
    }
    const int64_t e = a + L - 1;
    preceding_rank_start[r] = (int32_t)(first[a] / size);
    following_rank_stop[r] = (int32_t)(last[e] / size + 1);
  }
  return CPLA_OK;
}

extern "C" cpla_status cpla_seq_idx_from_cu_seqlens(const int32_t* cu_seqlens, int32_t n_seqs, int64_t T,
                                                    int32_t* seq_idx) {
  cpla::clear_error();
  if (!cu_seqlens || !seq_idx) return cpla::fail(CPLA_E_INVALID, "cu_seqlens or seq_idx is NULL");
  if (n_seqs <= 0 || T <= 0) return cpla::fail(CPLA_E_METADATA, "need at least one sequence and T > 0");
  if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != T)
    return cpla::fail(CPLA_E_METADATA, "cu_seqlens must start at 0 and end at T=%lld", (long long)T);
  for (int32_t s = 0; s < n_seqs; ++s) {
    if (cu_seqlens[s + 1] <= cu_seqlens[s])
      return cpla::fail(CPLA_E_METADATA, "cu_seqlens not strictly increasing at %d", s);
    for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) seq_idx[t] = s;
  }
  return CPLA_OK;
}
