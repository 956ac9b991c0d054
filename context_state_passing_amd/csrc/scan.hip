// Composition of shard summaries: a wavefront-level segmented associative scan
// of the affine maps F_r(S) = M_r S + delta_S_r (Megatron-Core page
// core.ssm.context_parallel.chunkwise: classes CPForward*Summary /
// CPBackward*Summary and functions chunkwise_cp_forward / chunkwise_cp_backward).
//
// Maps compose as (M2, D2) o (M1, D1) = (M2 M1, M2 D1 + D2); M is diagonal (one
// value per key row), so every state element (d, n) scans independently. A group
// of `group` = next_pow2(P) lanes holds one element's maps, one shard per lane,
// and runs a Hillis-Steele scan with segment heads:
//   forward:  shard r gets fold over [prs_r, r) of the maps, from S_init when the
//             prefix reaches rank 0 unpacked, else from zero; heads are ranks
//             with prs_r == r;
//   reverse:  shard r gets fold over (r, frs_r) taken backwards, from dS_final
//             when the suffix reaches the last rank unpacked; heads are ranks with
//             frs_r == r + 1.
// A shard containing a sequence start has M == 0, so a segment that begins
// before the slice start yields the same value as the slice itself.
// The last lane also yields the final state (forward) or dS_init (reverse).
#include "kernels.hpp"

namespace cpla {

__global__ __launch_bounds__(256) void affine_scan(ScanArgs a) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int G = a.group;
  const int s = (int)(gt % G);
  const int64_t elem = gt / G;
  const bool active = elem < a.n_elem;
  const int64_t per = (int64_t)a.dk * a.dv;
  const int64_t bh = active ? elem / per : 0;
  const int64_t e = active ? elem % per : 0;
  const int d = (int)(e / a.dv);
  const int q = a.reverse ? (a.P - 1 - s) : s;
  const bool real = active && s < a.P;

  float m = 1.f, x = 0.f;
  int head = 0;
  if (real) {
    const float* rec = a.summary + ((int64_t)q * a.BH + bh) * a.W;
    m = rec[a.diag ? d : 0];
    x = rec[a.m_slot + e];
    head = (s == 0);
    if (a.slice) head |= a.reverse ? (a.slice[q] == q + 1) : (a.slice[q] == q);
  }
  const float init = (active && a.init) ? a.init[bh * per + e] : 0.f;

  int f = head;
  for (int off = 1; off < G; off <<= 1) {
    const float m2 = __shfl_up(m, off, G);
    const float x2 = __shfl_up(x, off, G);
    const int f2 = __shfl_up(f, off, G);
    if (s >= off && !f) {
      x = m * x2 + x;
      m = m * m2;
      f = f2;
    }
  }
  // value after applying the inclusive map of lane s to the stream's initial value
  const float applied = x + m * init;
  const float prev = __shfl_up(applied, 1, G);
  if (real) {
    const float outv = head ? (s == 0 ? init : 0.f) : prev;
    a.out[((int64_t)q * a.BH + bh) * per + e] = outv;
    if (a.fin && s == a.P - 1) a.fin[bh * per + e] = applied;
  }
}

}  // namespace cpla
