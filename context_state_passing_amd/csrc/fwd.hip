// Forward shard walks: cp_forward_prepare (APPLY = false) and the local part of
// cp_forward_apply (APPLY = true).
//
// One workgroup walks one (shard, b, h): 64-token chunks in order, carrying the
// d_k x d_v fp32 state in MFMA accumulators. Wave w owns the state's d_v tiles
// w, w+4, ... (all d_k rows), so the state never leaves registers.
//
// Per chunk (see chunk_common.hpp for Gam, live, tail):
//   scores  A_ij = [same sequence, i >= j] * sum_d Q*_i[d] K*_j[d] (* exp(Gam_i - Gam_j)
//           for a scalar decay), Q* / K* = exp(+-Gam)-scaled tiles for a diagonal decay;
//   output  o_i = sum_j A_ij v_j + live_i * S0^T (q_i * exp(Gam_i))          (APPLY)
//   state   S  = diag(exp(Gam_last)) [no start] S0 + sum_{j tail} diag(exp(Gam_last - Gam_j)) k_j v_j^T
// which is the chunk algebra of S_t = diag(a_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.
#include <type_traits>

#include "chunk_common.hpp"
#include "kernels.hpp"

namespace cpla {

// S <- diag(exp(Gam_last)) keep*S + K^T V with the tail/decay token factors.
// UM > 1: UM row tiles at a time, the hi products and then the lo products, so
// that consecutive MFMAs accumulate into different tiles (for walks with
// registers to spare; the prepare walk's four waves per SIMD cover each other's
// MFMA latency instead).
template <typename E, int DK, int DV, int DECAY, int UM, int NKT_, int CPWV_, typename V, typename GT>
__device__ __forceinline__ void state_update(V (&S)[NKT_][CPWV_], const E* Kt, const E* Ktl, const E* Vt,
                                             const GT* gam, const float* el, const float* fk,
                                             const ChunkSeg& seg, int l) {
  using G = Geo<E, DK, DV>;
  const int w = wave_id(), g = l >> 4;
  __builtin_assume(w >= 0 && w < G::NW);
  const float keep = seg.any() ? 0.f : 1.f;
  if constexpr (DECAY == DECAY_SCALAR) {
    const float sc = keep * __expf((float)gam[CH - 1]);
#pragma unroll
    for (int m = 0; m < G::NKT; ++m)
#pragma unroll
      for (int cc = 0; cc < G::CPWV; ++cc) S[m][cc] *= sc;
  } else {
#pragma unroll
    for (int m = 0; m < G::NKT; ++m)
#pragma unroll
      for (int cc = 0; cc < G::CPWV; ++cc) S[m][cc] *= keep;
  }
  // V fragments, once per token block. Without a diagonal decay the token factors
  // fk (tail, and for a scalar decay exp(Gam_last - Gam_j) w_j) scale them here,
  // 2 fragments per wave rather than every K fragment; the scalar-decay V^ = fk V
  // enters the MFMA split into hi + lo parts. (A diagonal decay's factors differ
  // per key dim and sit in the staged K~ tiles, hi + lo.)
  constexpr bool VLO = DECAY == DECAY_SCALAR && Split<E>::on;
  constexpr bool LO = (DECAY == DECAY_DIAG || DECAY == DECAY_SCALAR) && Split<E>::on;
  const bool scale_tok = (DECAY == DECAY_SCALAR) || seg.any();
  Frag<E> bv[2][G::CPWV], bvl[VLO ? 2 : 1][G::CPWV];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int cc = 0; cc < G::CPWV; ++cc) {
      const int c = w + G::NW * cc;
      if (c >= G::NVT) continue;
      frag_tr(bv[kb][cc], Vt, G::LDV, 32 * kb, 16 * c, l);
      if constexpr (DECAY == DECAY_SCALAR) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = to_f(bv[kb][cc].v[e]) * fk[32 * kb + kidx(e, l)];
        if constexpr (VLO) {
          split_frag(bv[kb][cc], bvl[kb][cc], x);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) frag_set(bv[kb][cc], e, x[e]);
        }
      } else if constexpr (DECAY == DECAY_NONE) {
        if (scale_tok) frag_scale_tokens(bv[kb][cc], fk, 32 * kb, false, l);
      }
    }
  // the K fragment of row tile m, token block kb (diagonal: K~ hi and lo)
  auto k_frag = [&](Frag<E>& a, Frag<E>& al, int m, int kb) {
    frag_tr(a, Kt, G::LDK, 32 * kb, 16 * m, l);
    if constexpr (DECAY == DECAY_DIAG && Split<E>::on) {
      frag_tr(al, Ktl, G::LDK, 32 * kb, 16 * m, l);
      if (scale_tok) {
        frag_scale_tokens(a, fk, 32 * kb, false, l);
        frag_scale_tokens(al, fk, 32 * kb, false, l);
      }
    } else if constexpr (DECAY == DECAY_DIAG) {
      if (scale_tok) frag_scale_tokens(a, fk, 32 * kb, false, l);
    }
  };
  // the lo product: K~ lo times V (diagonal), K times V^ lo (scalar)
  auto mma_lo = [&](V& acc, const Frag<E>& a, const Frag<E>& al, int kb, int cc) {
    if constexpr (DECAY == DECAY_DIAG) mma(acc, al, bv[kb][cc]);
    else mma(acc, a, bvl[kb][cc]);
  };
  if constexpr (UM == 1) {
#pragma unroll
    for (int m = 0; m < G::NKT; ++m) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<E> a, al;
        k_frag(a, al, m, kb);
#pragma unroll
        for (int cc = 0; cc < G::CPWV; ++cc)
          if (w + G::NW * cc < G::NVT) {
            mma(S[m][cc], a, bv[kb][cc]);
            if constexpr (LO) mma_lo(S[m][cc], a, al, kb, cc);
          }
      }
    }
  } else {
    static_assert(G::NKT % UM == 0, "row tiles in whole groups");
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m0 = 0; m0 < G::NKT; m0 += UM) {
        Frag<E> a[UM], al[UM];
#pragma unroll
        for (int u = 0; u < UM; ++u) k_frag(a[u], al[u], m0 + u, kb);
#pragma unroll
        for (int u = 0; u < UM; ++u)
#pragma unroll
          for (int cc = 0; cc < G::CPWV; ++cc)
            if (w + G::NW * cc < G::NVT) mma(S[m0 + u][cc], a[u], bv[kb][cc]);
        if constexpr (LO) {
#pragma unroll
          for (int u = 0; u < UM; ++u)
#pragma unroll
            for (int cc = 0; cc < G::CPWV; ++cc)
              if (w + G::NW * cc < G::NVT) mma_lo(S[m0 + u][cc], a[u], al[u], kb, cc);
        }
      }
  }
  if constexpr (DECAY == DECAY_DIAG) {
    // K* = K exp(-Gam): restore exp(Gam_last - Gam_j) with a row factor exp(Gam_last[d])
#pragma unroll
    for (int m = 0; m < G::NKT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * m + 4 * g + r;
        const float f = d < DK ? el[d] : 0.f;
#pragma unroll
        for (int cc = 0; cc < G::CPWV; ++cc) S[m][cc][r] *= f;
      }
  }
}

template <typename E, int DK, int DV, int DECAY, bool APPLY, bool TAIL, bool SPLIT, bool PK>
__global__ __launch_bounds__((Geo<E, DK, DV>::NT), (APPLY ? 1 : (sizeof(E) == 4 ? 2 : 4))) void fwd_walk(FwdArgs a) {
  static_assert(APPLY || !SPLIT, "only the apply walk divides a shard");
  using G = Geo<E, DK, DV>;
  // diagonal decay: the prepare walk stages Gam rows 32..63 in the v tile's buffer
  // (written after the k tile is scaled), so two workgroups fit in a CU's LDS;
  // with d_v narrower than d_k those rows do not fit there and Gam stays whole
  constexpr bool GSPLIT = !APPLY && DECAY == DECAY_DIAG && G::TILE_V * (int)sizeof(E) >= (CH / 2) * DK * 4;
  constexpr int GAM = (DECAY == DECAY_DIAG) ? (GSPLIT ? CH / 2 : CH) * DK : CH;
  constexpr int NQT = APPLY ? 1 : 0;
  constexpr int DSP = (DECAY == DECAY_DIAG && Split<E>::on) ? 1 : 0;   // exp-scaled tiles split
  // The apply walk issues the products of GB token blocks term by term (every hi
  // part, then every lo part), so that consecutive MFMAs accumulate into
  // different tiles instead of each waiting on the one before it; d_k != d_v
  // walks have no registers to spare for the extra fragments and take one block
  // at a time.
  constexpr int GB = G::DKP == G::DVP ? 4 : 1;
  __shared__ __attribute__((aligned(16))) E s_q[NQT * G::TILE_K + 8];
  __shared__ __attribute__((aligned(16))) E s_ql[NQT * DSP * G::TILE_K + 8];
  __shared__ __attribute__((aligned(16))) E s_k[G::TILE_K];
  __shared__ __attribute__((aligned(16))) E s_kl[DSP * G::TILE_K + 8];
  __shared__ __attribute__((aligned(16))) E s_v[G::TILE_V];
  constexpr int NAL = (APPLY && Split<E>::on) ? 1 : 0;
  __shared__ __attribute__((aligned(16))) E s_a[NQT * G::TILE_A + 8];    // scores, hi part
  __shared__ __attribute__((aligned(16))) E s_al[NAL * G::TILE_A + 8];   // scores, lo part
  // Gam: fp64 for a scalar decay with fp32 inputs (see finish_gamma)
  using GT = typename std::conditional<sizeof(E) == 4 && DECAY == DECAY_SCALAR, double, float>::type;
  __shared__ GT s_gam[GAM];
  __shared__ float s_fq[CH], s_fk[CH], s_el[G::DKP];
  __shared__ float s_w[DECAY == DECAY_SCALAR ? CH : 1];   // per-token input weights

  float* const gam_hi = GSPLIT ? reinterpret_cast<float*>(s_v) : nullptr;
  const GT* const gam_last = [&]() -> const GT* {
    if constexpr (GSPLIT) return gam_hi + (CH / 2 - 1) * DK;
    else return s_gam + (CH - 1) * DK;
  }();

  const int w = wave_id(), l = lane_id(), g = l >> 4, i16 = l & 15;
  __builtin_assume(w >= 0 && w < G::NW);
  const int r = a.rank_begin + blockIdx.x;
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  // head of q and k: a scalar decay (the Mamba2 map) may share them within a group
  // of heads; the other decays read them per head
  const int64_t hqk = DECAY == DECAY_SCALAR ? (int64_t)((unsigned)h / (unsigned)a.qk_div) : h;
  const int64_t Hqk = DECAY == DECAY_SCALAR ? a.Hqk : a.H;
  // packed sequences: row b's sequence ids (one packing per batch row)
  const int32_t* const seq_row = (PK && a.seq_idx) ? a.seq_idx + b * a.T : nullptr;
  // the shard's tokens [tshard, tshard + slen): torch.chunk's division of T into P
  const int64_t tshard = shard_begin(a.T, a.P, r), slen = shard_len(a.T, a.P, r);
  const int nc = (int)chunks_of(slen);

  acc4<E> S[G::NKT][G::CPWV];   // fp32 (bf16 inputs) or fp64 (fp32 inputs)
#pragma unroll
  for (int m = 0; m < G::NKT; ++m)
#pragma unroll
    for (int cc = 0; cc < G::CPWV; ++cc) {
      const int c = w + G::NW * cc;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float x = 0.f;
        if constexpr (APPLY) {
          const int d = 16 * m + 4 * g + rr, n = 16 * c + i16;
          if (c < G::NVT && d < DK && n < DV)
            x = a.state_in[((int64_t)(r * a.B * a.H + bh) * DK + d) * DV + n];
        }
        S[m][cc][rr] = x;
      }
    }

  const E* q = reinterpret_cast<const E*>(a.q);
  const E* k = reinterpret_cast<const E*>(a.k);
  const E* v = reinterpret_cast<const E*>(a.v);
  GT gsum = 0;               // total log-decay of the shard (diag: column tid; else thread 0)
  bool any_start = false;

  // prefetch registers for the next chunk's inputs (apply); the prepare walk runs
  // two workgroups per CU and loads each chunk when it starts it
  SegRegs rseg;
  GamRegs<DK, DECAY, G::NT> rgam;
  TileRegs<E, DK, G::NT> rk, rq;
  TileRegs<E, DV, G::NT> rv;
  // tokens of chunk c inside the shard (the last chunk may be partial)
  auto valid = [&](int c) { return (int)(slen - (int64_t)c * CH < CH ? slen - (int64_t)c * CH : CH); };
  auto prefetch = [&](int c) {
    const int64_t t = tshard + (int64_t)c * CH;
    const int n = TAIL ? valid(c) : CH;
    rseg.template load<TAIL>(seq_row, t, lane_id(), n);
    rgam.template load<TAIL>(a.g, b, h, t, a.T, a.H, threadIdx.x, n);
    rgam.template load_w<TAIL>(a.w, b, h, t, a.T, a.H, threadIdx.x, n);
    rk.template load<TAIL>(k, b, hqk, t, a.T, Hqk, threadIdx.x, n);
    if constexpr (APPLY) rq.template load<TAIL>(q, b, hqk, t, a.T, Hqk, threadIdx.x, n);
    rv.template load<TAIL>(v, b, h, t, a.T, a.H, threadIdx.x, n);
  };
  if constexpr (APPLY) prefetch(0);

  // SPLIT: this workgroup emits chunks [c_emit, c_end) of the shard; the chunks
  // before them only carry the state forward (every workgroup starts at chunk 0
  // from the shard's incoming state, so the state it reaches at c_emit is exact)
  const int c_emit = SPLIT ? (int)((blockIdx.z * (int64_t)nc) / gridDim.z) : 0;
  const int c_end = SPLIT ? (int)(((blockIdx.z + 1) * (int64_t)nc) / gridDim.z) : nc;
  for (int c = 0; c < c_end; ++c) {
    const int64_t t0 = tshard + (int64_t)c * CH;
    const bool emit = !SPLIT || c >= c_emit;   // uniform across the workgroup
    const int nv = TAIL ? valid(c) : CH;
    const bool full = !TAIL || nv >= CH;   // only a shard's last chunk is partial
    if constexpr (!APPLY) prefetch(c);
    const ChunkSeg seg = rseg.finish(seq_row);
    any_start |= seg.any();
    finish_gamma<DK, DECAY, G::NT>(rgam, seg, s_gam, s_fq, s_fk, threadIdx.x, gam_hi,
                                   DECAY == DECAY_SCALAR ? s_w : nullptr);
    if constexpr (DECAY == DECAY_DIAG) {
      if (threadIdx.x < DK) {
        const float gl = gam_last[threadIdx.x];
        gsum += gl;
        s_el[threadIdx.x] = __expf(gl);   // exp(Gam_last[d]) for the state's row scaling
      }
      store_tile<E, DK, G::DKP, G::LDK, 2, DK, G::NT>(rk, s_k, s_kl, s_gam, nullptr, threadIdx.x, gam_hi);
      if constexpr (APPLY) store_tile<E, DK, G::DKP, G::LDK, 1, DK, G::NT>(rq, s_q, s_ql, s_gam, nullptr);
      if constexpr (GSPLIT) __syncthreads();   // the v tile overwrites Gam rows 32..63
    } else {
      if constexpr (DECAY == DECAY_SCALAR)
        if (threadIdx.x == 0) gsum += s_gam[CH - 1];
      store_tile<E, DK, G::DKP, G::LDK, 0, DK, G::NT>(rk, s_k, nullptr, s_gam, nullptr);
      if constexpr (APPLY) store_tile<E, DK, G::DKP, G::LDK, 0, DK, G::NT>(rq, s_q, nullptr, s_gam, nullptr);
    }
    store_tile<E, DV, G::DVP, G::LDV, 0, DK, G::NT>(rv, s_v, nullptr, s_gam, nullptr);
    if constexpr (APPLY)
      if (c + 1 < c_end) prefetch(c + 1);

    __syncthreads();

    if (APPLY && emit) {
      // ---- scores -> s_a (E), masked and decayed --------------------------------
#pragma unroll
      for (int s = 0; s < (N_SCORE_TILES + G::NW - 1) / G::NW; ++s) {
        const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
        if (s * G::NW + w >= N_SCORE_TILES) continue;
        const int idx = score_tile(s * G::NW + w);
        const int I = idx >> 2, J = idx & 3;
        acc4<E> acc = {0, 0, 0, 0};
        if (!score_tile_zero(idx)) {
          // the split cross terms in accumulators of their own, so that no MFMA
          // waits on the one before it
          acc4<E> xh = {0, 0, 0, 0}, xl = {0, 0, 0, 0};
#pragma unroll
          for (int kd = 0; kd < G::DKP / 32; ++kd) {
            Frag<E> fa, fb;
            frag_direct(fa, s_q, G::LDK, 16 * I + i16, 32 * kd, l);
            frag_direct(fb, s_k, G::LDK, 16 * J + i16, 32 * kd, l);
            if constexpr (DSP) {
              Frag<E> fal, fbl;
              frag_direct(fal, s_ql, G::LDK, 16 * I + i16, 32 * kd, l);
              frag_direct(fbl, s_kl, G::LDK, 16 * J + i16, 32 * kd, l);
              mma(acc, fa, fb);
              mma(xh, fa, fbl);
              mma(xl, fal, fb);
            } else {
              mma(acc, fa, fb);
            }
          }
          if constexpr (DSP) acc += xh + xl;
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int i = 16 * I + 4 * g + rr, j = 16 * J + i16;
          float x = 0.f;
          if (seg.same(i, j)) {
            x = (float)acc[rr];
            if constexpr (DECAY == DECAY_SCALAR) x *= __expf((float)(s_gam[i] - s_gam[j])) * s_w[j];
          }
          store_split(s_a, s_al, i * G::LDA + j, x);
        }
      }
      __syncthreads();

      // ---- o^T tiles: rows = d_v (owned tiles), columns = tokens ----------------
      E* o = reinterpret_cast<E*>(a.out);
#pragma unroll
      for (int cc = 0; cc < G::CPWV; ++cc) {
        const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
        const int cn = w + G::NW * cc;
        if (cn >= G::NVT) continue;
        Frag<E> fs[G::DKP / 32], fsl[G::DKP / 32];
#pragma unroll
        for (int kb = 0; kb < G::DKP / 32; ++kb)
          acc_to_frag_split(fs[kb], fsl[kb], S[2 * kb][cc], S[2 * kb + 1][cc]);
        Frag<E> fvt[2];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) frag_tr(fvt[jb], s_v, G::LDV, 32 * jb, 16 * cn, l);
        // GB token blocks at a time: the inter part S0^T q~ (hi.hi, hi.lo, lo.hi over
        // the blocks), then the intra part A v (score-tile blocks jb = 0 for every
        // query block, jb = 1 for query blocks 2 and 3)
#pragma unroll
        for (int I0 = 0; I0 < 4; I0 += GB) {
          acc4<E> acc[GB];
#pragma unroll
          for (int u = 0; u < GB; ++u) acc[u] = acc4<E>{0, 0, 0, 0};
#pragma unroll
          for (int kb = 0; kb < G::DKP / 32; ++kb) {
            Frag<E> fb[GB], fbl[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) {
              frag_direct_perm(fb[u], s_q, G::LDK, 16 * (I0 + u) + i16, 32 * kb, l);
              if constexpr (DSP) frag_direct_perm(fbl[u], s_ql, G::LDK, 16 * (I0 + u) + i16, 32 * kb, l);
            }
#pragma unroll
            for (int u = 0; u < GB; ++u) mma(acc[u], fs[kb], fb[u]);
            if constexpr (DSP) {
#pragma unroll
              for (int u = 0; u < GB; ++u) mma(acc[u], fs[kb], fbl[u]);
            }
            if constexpr (Split<E>::on) {
#pragma unroll
              for (int u = 0; u < GB; ++u) mma(acc[u], fsl[kb], fb[u]);
            }
          }
#pragma unroll
          for (int u = 0; u < GB; ++u) acc[u] *= s_fq[16 * (I0 + u) + i16];
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) {
            Frag<E> fb[GB], fbl[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) {
              if (jb == 1 && I0 + u < 2) continue;
              frag_direct(fb[u], s_a, G::LDA, 16 * (I0 + u) + i16, 32 * jb, l);
              if constexpr (Split<E>::on) frag_direct(fbl[u], s_al, G::LDA, 16 * (I0 + u) + i16, 32 * jb, l);
            }
#pragma unroll
            for (int u = 0; u < GB; ++u)
              if (!(jb == 1 && I0 + u < 2)) mma(acc[u], fvt[jb], fb[u]);
            if constexpr (Split<E>::on) {
#pragma unroll
              for (int u = 0; u < GB; ++u)
                if (!(jb == 1 && I0 + u < 2)) mma(acc[u], fvt[jb], fbl[u]);
            }
          }
#pragma unroll
          for (int u = 0; u < GB; ++u) {
            const int n0 = 16 * cn + 4 * g, ti = 16 * (I0 + u) + i16;
            if (n0 < DV && (full || ti < nv)) store4(o + tok_off(b, t0, h, a.T, a.H, DV) + tok_rel(ti, a.H, DV) + n0, acc[u]);
          }
        }
      }
    }

    // the state entering the chunk, saved for the backward walk: written after
    // the output tiles and before the update overwrites S (issuing these stores
    // at the start of the chunk measured slower)
    if (APPLY && emit) {
      if (a.chunk_states) {
        float* cs = a.chunk_states +
                    ((bh * row_chunks(a.T, a.P) + shard_chunk_base(a.T, a.P, r) + c) * DK) * (int64_t)DV;
#pragma unroll
        for (int m = 0; m < G::NKT; ++m)
#pragma unroll
          for (int cc = 0; cc < G::CPWV; ++cc) {
            const int cn = w + G::NW * cc;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int d = 16 * m + 4 * g + rr, n = 16 * cn + i16;
              if (cn < G::NVT && d < DK && n < DV) cs[d * DV + n] = (float)S[m][cc][rr];
            }
          }
      }
    }
    state_update<E, DK, DV, DECAY, (APPLY && GB > 1) ? (G::NKT < 4 ? G::NKT : 4) : 1>(S, s_k, s_kl, s_v, s_gam, s_el, s_fk, seg,
                                                            lane_pick<APPLY>());
    __syncthreads();
  }

  if constexpr (!APPLY) {
    // ---- summary record [M (m_slot) | delta_S (dk*dv)] -----------------------------
    float* rec = a.summary + (int64_t)(r * a.B * a.H + bh) * a.W;
    const float keep = any_start ? 0.f : 1.f;
    if constexpr (DECAY == DECAY_DIAG) {
      if (threadIdx.x < DK) rec[threadIdx.x] = keep * __expf((float)gsum);
    } else {
      if (threadIdx.x < 4) {
        float mval = (DECAY == DECAY_SCALAR) ? __expf((float)gsum) : 1.f;
        rec[threadIdx.x] = threadIdx.x == 0 ? keep * mval : 0.f;
      }
    }
    float* ds = rec + a.m_slot;
#pragma unroll
    for (int m = 0; m < G::NKT; ++m)
#pragma unroll
      for (int cc = 0; cc < G::CPWV; ++cc) {
        const int cn = w + G::NW * cc;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = 16 * m + 4 * g + rr, n = 16 * cn + i16;
          if (cn < G::NVT && d < DK && n < DV) ds[d * DV + n] = (float)S[m][cc][rr];
        }
      }
  }
}

#define CPLA_INST_FWD(E, DK, DV, DEC)                                              \
  template __global__ void fwd_walk<E, DK, DV, DEC, false, false>(FwdArgs);       \
  template __global__ void fwd_walk<E, DK, DV, DEC, true, false>(FwdArgs);        \
  template __global__ void fwd_walk<E, DK, DV, DEC, false, true>(FwdArgs);        \
  template __global__ void fwd_walk<E, DK, DV, DEC, true, true>(FwdArgs);         \
  template __global__ void fwd_walk<E, DK, DV, DEC, true, false, true>(FwdArgs);  \
  template __global__ void fwd_walk<E, DK, DV, DEC, true, true, true>(FwdArgs);   \
  template __global__ void fwd_walk<E, DK, DV, DEC, true, false, false, false>(FwdArgs); \
  template __global__ void fwd_walk<E, DK, DV, DEC, true, true, false, false>(FwdArgs);  \
  template __global__ void fwd_walk<E, DK, DV, DEC, true, false, true, false>(FwdArgs);  \
  template __global__ void fwd_walk<E, DK, DV, DEC, true, true, true, false>(FwdArgs);
#define CPLA_INST_FWD3(E, D) CPLA_INST_FWD(E, D, D, 0) CPLA_INST_FWD(E, D, D, 1) CPLA_INST_FWD(E, D, D, 2)
#define CPLA_INST_FWD3X(E, DK, DV) CPLA_INST_FWD(E, DK, DV, 0) CPLA_INST_FWD(E, DK, DV, 1) CPLA_INST_FWD(E, DK, DV, 2)
CPLA_INST_FWD3(bf16_t, 16)
CPLA_INST_FWD3(bf16_t, 64)
CPLA_INST_FWD3(bf16_t, 128)
CPLA_INST_FWD3X(bf16_t, 64, 128)
CPLA_INST_FWD3X(bf16_t, 128, 64)
CPLA_INST_FWD3(float, 16)
CPLA_INST_FWD3(float, 64)

}  // namespace cpla
