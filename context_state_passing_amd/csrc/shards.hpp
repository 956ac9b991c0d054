// Division of a T-token stream into P contiguous shards, as torch.chunk makes it:
// parts of ceil(T / P) tokens, the last non-empty one shorter when P does not
// divide T, and trailing parts empty when the stream is short. The mixle page
// (context_parallel_spine, module docstring) relies on exactly this graceful
// division where Megatron-style CP fails fast. A shard's chunks are 64 tokens,
// its last one partial when the shard length is not a multiple of 64. The
// functions are constexpr so that host code and kernels share them.
#pragma once
#include <stdint.h>

namespace cpla {

constexpr int64_t shard_size(int64_t T, int64_t P) { return (T + P - 1) / P; }
constexpr int64_t shard_begin(int64_t T, int64_t P, int64_t r) {
  return r * shard_size(T, P) < T ? r * shard_size(T, P) : T;
}
constexpr int64_t shard_len(int64_t T, int64_t P, int64_t r) {
  return (T - shard_begin(T, P, r)) < shard_size(T, P) ? (T - shard_begin(T, P, r)) : shard_size(T, P);
}
constexpr int64_t chunks_of(int64_t len) { return (len + 63) / 64; }
// index of shard r's first chunk among all chunks of a row (every earlier shard
// is full-size when shard r holds any token)
constexpr int64_t shard_chunk_base(int64_t T, int64_t P, int64_t r) { return r * chunks_of(shard_size(T, P)); }
// chunks of a whole row: the full shards, then the remainder
constexpr int64_t row_chunks(int64_t T, int64_t P) {
  return (T / shard_size(T, P)) * chunks_of(shard_size(T, P)) + chunks_of(T % shard_size(T, P));
}

}  // namespace cpla
