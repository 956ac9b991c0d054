// Range check of a diagonal log-decay: the kernels factor the decay between two
// tokens of one 64-token chunk as exp(Gam_i) * exp(-Gam_j), Gam the chunk's
// running sum of g per key dim, so every running sum must stay above
// CPLA_DIAG_GAMMA_MIN (exp(-Gam) finite in fp32 with a margin for the values it
// multiplies). One thread per (b, h, chunk, key dim) sums its chunk's g and counts
// the (chunk, key dim) pairs that fall below the bound.
#include "kernels.hpp"
#include "shards.hpp"

namespace cpla {

__global__ void decay_check_zero(int32_t* count) { *count = 0; }

__global__ __launch_bounds__(256) void decay_range(DecayCheckArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.n) return;
  const int64_t d = idx % a.dk;
  int64_t rest = idx / a.dk;
  const int64_t c = rest % a.nchunks;          // chunk among the handled shards' chunks
  rest /= a.nchunks;
  const int64_t h = rest % a.H, b = rest / a.H;
  const int64_t cps = chunks_of(shard_size(a.T, a.P));   // chunks of a full shard
  const int64_t r = a.rank_begin + c / cps, cl = c % cps;
  const int64_t len = shard_len(a.T, a.P, r) - cl * 64;
  if (len <= 0) return;                        // past the end of a shorter last shard
  const int n = len < 64 ? (int)len : 64;
  const float* src = a.g + ((b * a.T + shard_begin(a.T, a.P, r) + cl * 64) * a.H + h) * a.dk + d;
  float run = 0.f;
  bool bad = false;
  for (int s = 0; s < n; ++s) {
    run += src[(int64_t)s * a.H * a.dk];
    bad |= !(run >= a.limit);                  // also catches NaN
  }
  if (bad) atomicAdd(a.count, 1);
}

}  // namespace cpla
