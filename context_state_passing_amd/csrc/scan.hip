// Composition of shard summaries: the exclusive scan of the affine maps
// F_r(S) = M_r S + delta_S_r over the shards (Megatron-Core page
// core.ssm.context_parallel.chunkwise: classes CPForward*Summary /
// CPBackward*Summary and functions chunkwise_cp_forward / chunkwise_cp_backward).
//
// M is diagonal (one value per key row d), so every state element (d, n) of
// every (b, h) composes independently: one thread per element folds the maps
// in shard order, reading each shard's record with loads that are contiguous
// across the threads (the element index runs fastest), P of them in flight
// per batch.
// With packed sequences each batch row has its own slices prs / frs ([B, P]).
//   forward:  shard r gets the fold over [prs_r, r), started from S_init at
//             rank 0 (unpacked) and from zero at ranks with prs_r == r;
//   reverse:  shard r gets the fold over (r, frs_r) taken backwards, started
//             from dS_final at the last rank (unpacked) and from zero at ranks
//             with frs_r == r + 1.
// A shard that holds a sequence start has M == 0, so carrying the fold through
// it equals restarting the fold there. After the last shard the running value
// is the final state (forward) or dS_init (reverse).
#include "kernels.hpp"

namespace cpla {

__global__ __launch_bounds__(256) void affine_scan(ScanArgs a) {
  constexpr int BATCH = 8;
  const int64_t elem = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (elem >= a.n_elem) return;
  const int64_t per = (int64_t)a.dk * a.dv;
  const int64_t bh = elem / per, e = elem % per;
  const int m_off = a.diag ? (int)(e / a.dv) : 0;
  const int64_t rec_stride = a.BH * a.W, out_stride = a.BH * per;
  const float* rec0 = a.summary + bh * a.W;
  float* out0 = a.out + bh * per + e;

  const int32_t* slice = a.slice ? a.slice + (bh / a.H) * a.P : nullptr;   // row b's rank slices
  float run = a.init ? a.init[bh * per + e] : 0.f;
  for (int s0 = 0; s0 < a.P; s0 += BATCH) {
    float m[BATCH], x[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int s = s0 + j;
      if (s < a.P) {
        const int q = a.reverse ? a.P - 1 - s : s;
        const float* rec = rec0 + q * rec_stride;
        m[j] = rec[m_off];
        x[j] = rec[a.m_slot + e];
      }
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int s = s0 + j;
      if (s < a.P) {
        const int q = a.reverse ? a.P - 1 - s : s;
        if (s > 0 && slice && slice[q] == (a.reverse ? q + 1 : q)) run = 0.f;
        out0[q * out_stride] = run;
        run = m[j] * run + x[j];
      }
    }
  }
  if (a.fin) a.fin[bh * per + e] = run;
}

}  // namespace cpla
