// Backward shard walks: cp_backward_prepare (APPLY = false) and the local part of
// cp_backward_apply (APPLY = true).
//
// One workgroup walks one (shard, b, h) from its last chunk to its first,
// carrying dS (gradient w.r.t. the state at the current chunk's end, d_k x d_v,
// fp32) in MFMA accumulators twice: dS with wave w owning d_v tiles w, w+4, ...,
// and its transpose with wave w owning d_k tiles w, w+4, ... (the two feed the
// contractions over d_k and over d_v). The state entering each chunk, S0, is
// read (fp32) from the chunk states the forward saved.
//
// Per chunk (Gam, live, tail as in chunk_common.hpp; A = masked decayed scores,
// dA_ij = [same sequence, i >= j] (dO_i . v_j) (* exp(Gam_i - Gam_j) for a scalar decay)):
//   dq_i = live_i exp(Gam_i) * S0 dO_i + sum_j dA_ij exp(Gam_i - Gam_j) * k_j
//   dk_j = sum_i dA_ij exp(Gam_i - Gam_j) * q_i + tail_j exp(Gam_last - Gam_j) * dS v_j
//   dv_j = sum_i A_ij dO_i + tail_j dS^T (k_j * exp(Gam_last - Gam_j))
//   dS  <- [no start] diag(exp(Gam_last)) dS + sum_i live_i (q_i * exp(Gam_i)) dO_i^T
//   dg_t = a_t rowsum(dS_t * S_{t-1}) as four non-cancelling parts:
//     T1 = live part of sum_{i >= t} q_i exp(Gam_i) * (S0 dO_i)
//     T2 = sum_{i >= t > j} exp(Gam_i - Gam_j) q_i * k_j (dO_i . v_j)
//     T3 = [no start] exp(Gam_last) * rowsum(dS * S0)
//     T4 = tail part of sum_{j < t} exp(Gam_last - Gam_j) k_j * (dS v_j)
//   diagonal decay: T1 + T2 = suffix sums of Q~ * (dq before exp(Gam)) - K~ * (intra dk),
//   per key dim; scalar decay: T2 from the fp32 product of the score and
//   score-gradient tiles (row sums left of the diagonal minus column sums below
//   it, suffix-summed), all parts summed over the key dim; dg = 0 at starts.
//
// Every fp32 intermediate that feeds an MFMA (scores, score gradients, S0, dS,
// exp-scaled q/k tiles) is split into bf16 hi + lo parts; inputs are exact.
#include <type_traits>

#include "chunk_common.hpp"
#include "kernels.hpp"

namespace cpla {

// Row shift within the 16 lanes of a DPP row; lanes with no source read 0.
template <int OFF>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 | OFF,
                                                               0xf, 0xf, true));
}

// Sum over the 16 lanes of each DPP row, in every lane of the row (quad swaps,
// then the half-row and row mirrors: VALU only, no trip through the LDS unit).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);   // row_half_mirror
  x += dpp_f<0x140>(x);   // row_mirror
  return x;
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}
// Sum over the 64 lanes, in every lane.
__device__ __forceinline__ float wave_total(float x) {
  x = row_sum(x);
  return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}
// Inclusive prefix sums over the 64 lanes: DPP scans within the rows, then the
// totals of the earlier rows (their last lanes).
__device__ __forceinline__ float wave_scan(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  const float r0 = lane_value(x, 15), r1 = lane_value(x, 31), r2 = lane_value(x, 47);
  const int row = lane_id() >> 4;
  return x + (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
}

// Inclusive prefix sums over the 16 lanes of each DPP row, per component.
__device__ __forceinline__ f32x4 row_scan(f32x4 x) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    x[rr] += row_shr<1>(x[rr]);
    x[rr] += row_shr<2>(x[rr]);
    x[rr] += row_shr<4>(x[rr]);
    x[rr] += row_shr<8>(x[rr]);
  }
  return x;
}

// Sum over the 16 lanes of each DPP row, per component, in every lane of the row.
__device__ __forceinline__ f32x4 row_total(f32x4 x) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) x[rr] = row_sum(x[rr]);
  return x;
}

// The last lane of each DPP row, per component, in every lane of the row (DPP
// row_newbcast:15): the row total of an inclusive row scan in one move.
__device__ __forceinline__ f32x4 row_last(f32x4 x) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) x[rr] = dpp_f<0x15F>(x[rr]);
  return x;
}

// Gam at token 16 I + (lane % 16) of the current block and key dims d0 .. d0+3
// (the calling lane's) from the lane's raw log-decays x of that block: the
// prefix sum over the row plus the total of the earlier blocks held in carry
// (updated for the next block).
__device__ __forceinline__ f32x4 lane_gamma(f32x4 x, f32x4& carry) {
  x = row_scan(x);
  const f32x4 out = x + carry;
  carry += row_last(x);
  return out;
}

template <typename E, int DK, int DV, int DECAY, bool APPLY, bool GF32, bool TAIL, bool SPLIT, bool PK>
__global__ __launch_bounds__((Geo<E, DK, DV>::NT), (APPLY ? 1 : (sizeof(E) == 4 ? 2 : 4))) void bwd_walk(BwdArgs a) {
  static_assert(!SPLIT || (APPLY && DECAY != DECAY_DIAG), "divided walks: apply, no or scalar decay");
  using G = Geo<E, DK, DV>;
  // dq, dk, dv in the input dtype, or in fp32 (GF32: for callers that sum them
  // further, e.g. over the heads sharing an input)
  using GE = typename std::conditional<GF32, float, E>::type;
  constexpr bool SP = Split<E>::on;
  constexpr bool DIAG = DECAY == DECAY_DIAG, SCAL = DECAY == DECAY_SCALAR;
  constexpr int NA = APPLY ? 1 : 0;
  constexpr bool HAS_DG = APPLY && DECAY != DECAY_NONE;
  // q tile (hi) and its lo part: diagonal decay stores Q~ = Q exp(Gam)
  constexpr int QLO = (DIAG && SP) ? 1 : 0;
  // k tile only in apply; lo part for the diagonal decay
  constexpr int KLO = (APPLY && DIAG && SP) ? 1 : 0;
  // Q^ = q exp(Gam_i) live_i (scalar decay), split
  constexpr int QH = (SCAL && APPLY) ? 1 : 0;
  constexpr int QHL = (SCAL && SP && APPLY) ? 1 : 0;
  // region: Gam (diag, fp32) during staging, then A/dA hi/lo and the scalar P tile.
  // The prepare walk (two workgroups per CU) stages Gam rows 32..63 in the dO
  // tile's buffer, written after the q tile is scaled (when they fit there: not
  // with d_v narrower than d_k).
  constexpr bool GSPLIT = !APPLY && DIAG && G::TILE_V * (int)sizeof(E) >= (CH / 2) * DK * 4;
  constexpr int GAM_BYTES = DIAG ? (GSPLIT ? CH / 2 : CH) * DK * 4 : 0;
  constexpr int AT_BYTES = APPLY ? (SP ? 4 : 2) * G::TILE_A * (int)sizeof(E) : 0;
  // the scalar decay's dg / dw sums: fp32 for bf16 inputs, fp64 for fp32 inputs
  using AS = typename std::conditional<sizeof(E) == 2, float, double>::type;
  // scalar decay: per score tile, the row sums left of and the column sums below
  // the diagonal of P_ij = exp(Gam_i - Gam_j) w_j (q_i.k_j)(dO_i.v_j) (16 tile
  // slots of 16 rows and 16 columns), and P's diagonal
  constexpr int P_BYTES = (APPLY && SCAL) ? (2 * 16 * 16 + CH) * (int)sizeof(AS) : 0;
  constexpr int REG_BYTES = (GAM_BYTES > AT_BYTES + P_BYTES ? GAM_BYTES : AT_BYTES + P_BYTES) + 16;
  // Apply walk, bf16 with a diagonal decay: the next chunk's raw inputs are copied
  // into LDS by DMA once the dk phase is done (q into a buffer of its own; k, v,
  // dO and g into the k, v, k-lo and score-tile regions, dead from there to the
  // end of the chunk), so their HBM latency overlaps dg and the dS update. The raw
  // dO goes to the k-lo region, so this needs d_v <= d_k + pad; wider d_v loads
  // each chunk at its start instead.
  constexpr bool PF = APPLY && DIAG && SP && G::TILE_K >= CH * DV;
  static_assert(!PF || GamRegs<DK, DECAY, G::NT>::DMA_FLOATS * 4 <= REG_BYTES, "raw g must fit");
  // Apply phases issue the products of GB token blocks term by term (every hi
  // part, then every lo part), so that consecutive MFMAs accumulate into
  // different tiles instead of each waiting on the one before it; d_k != d_v
  // walks have no registers to spare for the extra fragments and take one block
  // at a time.
  constexpr int GB = G::DKP == G::DVP ? 4 : 1;

  __shared__ __attribute__((aligned(16))) E s_q[G::TILE_K];
  __shared__ __attribute__((aligned(16))) E s_ql[QLO * G::TILE_K + 8];
  __shared__ __attribute__((aligned(16))) E s_k[NA * G::TILE_K + 8];
  __shared__ __attribute__((aligned(16))) E s_kl[KLO * G::TILE_K + 8];
  __shared__ __attribute__((aligned(16))) E s_v[NA * G::TILE_V + 8];
  __shared__ __attribute__((aligned(16))) E s_do[G::TILE_V];
  __shared__ __attribute__((aligned(16))) E s_qh[QH * G::TILE_K + 8];
  __shared__ __attribute__((aligned(16))) E s_qhl[QHL * G::TILE_K + 8];
  __shared__ __attribute__((aligned(16))) char s_reg[REG_BYTES];
  __shared__ __attribute__((aligned(16))) E s_pq[PF ? CH * DK : 8];
  constexpr int NRED = SCAL ? G::NW : 1;                          // scalar decay: per-wave T3 partials
  constexpr int NU = (APPLY && SCAL) ? G::NW * CH : 1;           // scalar dg token partials
  // Gam: fp64 for a scalar decay with fp32 inputs (see finish_gamma)
  using GT = typename std::conditional<sizeof(E) == 4 && SCAL, double, float>::type;
  __shared__ GT s_gs[DIAG ? 1 : CH];
  __shared__ float s_fq[CH], s_fk[CH], s_el[DIAG ? G::DKP : 1];
  __shared__ AS s_red[NRED], s_u1[NU], s_u4[NU];
  __shared__ float s_w[SCAL ? CH : 1];   // per-token input weights (scalar decay)

  GT* s_gam = DIAG ? reinterpret_cast<GT*>(s_reg) : s_gs;
  E* s_ah = reinterpret_cast<E*>(s_reg);
  E* s_al = s_ah + G::TILE_A;
  E* s_dah = s_ah + (SP ? 2 : 1) * G::TILE_A;
  E* s_dal = s_dah + G::TILE_A;
  AS* s_rowp = reinterpret_cast<AS*>(s_reg + AT_BYTES);
  AS* s_colp = s_rowp + 16 * 16;
  AS* s_pdiag = s_colp + 16 * 16;
  // the tile Q^ is read from in the dS update: scalar -> s_qh, else the q tile
  const E* qhat_h = SCAL ? s_qh : s_q;
  const E* qhat_l = SCAL ? s_qhl : s_ql;
  float* const gam_hi = GSPLIT ? reinterpret_cast<float*>(s_do) : nullptr;
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
  const int64_t nct = row_chunks(a.T, a.P), cbase = shard_chunk_base(a.T, a.P, r);
  // tokens of chunk c inside the shard (the last chunk may be partial)
  auto valid = [&](int c) { return (int)(slen - (int64_t)c * CH < CH ? slen - (int64_t)c * CH : CH); };

  // dS: rows = all d_k tiles, columns = owned d_v tiles.  dT = dS^T: rows = all
  // d_v tiles, columns = owned d_k tiles (lane-fixed d).
  using AV = acc4<E>;   // fp32 accumulators for bf16 inputs, fp64 for fp32 inputs
  AV dS[G::NKT][G::CPWV];
  AV dT[APPLY ? G::NVT : 1][G::CPWK];
  {
    const float* gin = APPLY ? a.grad_in + (int64_t)(r * a.B * a.H + bh) * DK * DV : nullptr;
#pragma unroll
    for (int m = 0; m < G::NKT; ++m)
#pragma unroll
      for (int cc = 0; cc < G::CPWV; ++cc) {
        const int c = w + G::NW * cc;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = 16 * m + 4 * g + rr, n = 16 * c + i16;
          dS[m][cc][rr] = (APPLY && c < G::NVT && d < DK && n < DV) ? gin[d * DV + n] : 0.f;
        }
      }
    if constexpr (APPLY) {
#pragma unroll
      for (int nt = 0; nt < G::NVT; ++nt)
#pragma unroll
        for (int cc = 0; cc < G::CPWK; ++cc) {
          const int cm = w + G::NW * cc;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int n = 16 * nt + 4 * g + rr, d = 16 * cm + i16;
            dT[nt][cc][rr] = (cm < G::NKT && d < DK && n < DV) ? gin[d * DV + n] : 0.f;
          }
        }
    }
  }

  const E* q = reinterpret_cast<const E*>(a.q);
  const E* k = reinterpret_cast<const E*>(a.k);
  const E* v = reinterpret_cast<const E*>(a.v);
  const E* dO = reinterpret_cast<const E*>(a.dO);
  GT gsum = 0;
  bool any_start = false;

  using GamR = GamRegs<DK, DECAY, G::NT>;
  using TileK = TileRegs<E, DK, G::NT>;
  using TileV = TileRegs<E, DV, G::NT>;
  float* const pf_g = reinterpret_cast<float*>(s_reg);
  E* const pf_do = s_kl;
  // raw inputs of the chunk starting at tn (n of its tokens inside the shard), by
  // DMA into the regions above
  auto prefetch = [&](int64_t tn, int tid, int n, auto tail) {
    constexpr bool TL = decltype(tail)::value;
    const int wv = wave_id();
    GamR::template dma<TL>(a.g, b, h, tn, a.T, a.H, pf_g, tid, wv, n);
    TileK::template dma<TL>(q, b, hqk, tn, a.T, Hqk, s_pq, tid, wv, n);
    TileK::template dma<TL>(k, b, hqk, tn, a.T, Hqk, s_k, tid, wv, n);
    TileV::template dma<TL>(v, b, h, tn, a.T, a.H, s_v, tid, wv, n);
    TileV::template dma<TL>(dO, b, h, tn, a.T, a.H, pf_do, tid, wv, n);
  };
  SegRegs nseg;   // sequence ids of the prefetched chunk
  // the lane's log-decays for dq/dk come from the DMA buffer (d_k 64 / 128: one
  // key tile per wave, 16-token parts) instead of a second read from HBM
  constexpr bool GL_LDS = PF && GamR::TOK == 16 && GamR::CPW == 16 && G::CPWK == 1 && G::NKT == G::NW;
  if constexpr (PF) {
    if (nc > 0) {
      const int tidf = tid_pick<APPLY, G::NT>();
      const int64_t tn = tshard + (int64_t)(nc - 1) * CH;
      const int n = TAIL ? valid(nc - 1) : CH;
      prefetch(tn, tidf, n, std::integral_constant<bool, TAIL>{});
      nseg.template load<TAIL>(seq_row, tn, tidf & 63, n);
    }
  }

  // SPLIT: this workgroup emits chunks [c_lo, c_hi) of the shard; the later ones
  // only carry the adjoint backwards (every workgroup starts at the shard's last
  // chunk from its outgoing gradient, so the adjoint it reaches at c_hi is exact)
  const int c_lo = SPLIT ? (int)((blockIdx.z * (int64_t)nc) / gridDim.z) : 0;
  const int c_hi = SPLIT ? (int)(((blockIdx.z + 1) * (int64_t)nc) / gridDim.z) : nc;
  for (int c = nc - 1; c >= c_lo; --c) {
    const bool emit = !SPLIT || c < c_hi;   // uniform across the workgroup
    const int64_t t0 = tshard + (int64_t)c * CH;
    const int nv = TAIL ? valid(c) : CH;
    const bool full = !TAIL || nv >= CH;   // only a shard's last chunk is partial
    ChunkSeg seg;
    // Every global load of the chunk's inputs is issued before the first use, so
    // the chunk waits on memory once; the registers are free again once the tiles
    // are in LDS (the apply walk's compute needs them; the prepare walk runs two
    // workgroups per CU, which cover each other's waits).
    SegRegs aseg;
    GamR agam;
    TileK aq, ak;
    TileV av_, ado;
    const int tidf = tid_pick<APPLY, G::NT>();
    // diagonal: the lane's raw log-decays g[t0 + 16 I + i16][16 cm + 4g .. +3] for
    // the dq/dk scaling, turned into Gam in the dq phase
    f32x4 gl[HAS_DG && DIAG ? G::CPWK : 1][4];
    if constexpr (PF) {
      // this wave's DMA copies must have landed before it reads them back (each
      // lane reads only bytes its own DMA lane wrote); the wait is explicit
      // because the compiler's own tracking of LDS DMA does not cover every path
      // into the loop
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      aseg = nseg;
      if constexpr (GL_LDS) {
        const int l = lane_pick<APPLY>();
#pragma unroll
        for (int I = 0; I < 4; ++I) gl[0][I] = GamR::template lane_block<TAIL>(pf_g, w, I, l, nv);
      }
      agam.template load_lds<TAIL>(pf_g, tidf, nv);
      aq.template load_lds<TAIL>(s_pq, tidf, nv);
      ak.template load_lds<TAIL>(s_k, tidf, nv);
      av_.template load_lds<TAIL>(s_v, tidf, nv);
      ado.template load_lds<TAIL>(pf_do, tidf, nv);
      __syncthreads();   // the raw regions are overwritten from here on
    } else {
      aseg.template load<TAIL>(seq_row, t0, tidf & 63, nv);
      agam.template load<TAIL>(a.g, b, h, t0, a.T, a.H, tidf, nv);
      if constexpr (APPLY) agam.template load_w<TAIL>(a.w, b, h, t0, a.T, a.H, tidf, nv);
      aq.template load<TAIL>(q, b, hqk, t0, a.T, Hqk, tidf, nv);
      if constexpr (APPLY) {
        ak.template load<TAIL>(k, b, hqk, t0, a.T, Hqk, tidf, nv);
        av_.template load<TAIL>(v, b, h, t0, a.T, a.H, tidf, nv);
      }
      ado.template load<TAIL>(dO, b, h, t0, a.T, a.H, tidf, nv);
    }
    seg = aseg.finish(seq_row);
    finish_gamma<DK, DECAY, G::NT>(agam, seg, s_gam, s_fq, s_fk, tidf, gam_hi, SCAL ? s_w : nullptr);
    any_start |= seg.any();
    const float keep = seg.any() ? 0.f : 1.f;

    // ---- stage tiles ----------------------------------------------------------------
    if constexpr (DIAG) {
      if (threadIdx.x < DK) {
        const float gl = gam_last[threadIdx.x];
        gsum += gl;
        s_el[threadIdx.x] = __expf(gl);   // exp(Gam_last[d]), read by every row scaling below
      } else if (threadIdx.x < G::DKP) {
        s_el[threadIdx.x] = 0.f;           // padded key dims: their state rows stay zero
      }
    } else if constexpr (SCAL) {
      if (threadIdx.x == 0) gsum += s_gam[CH - 1];
    }
    if constexpr (APPLY) {
      if constexpr (DIAG) {
        store_tile<E, DK, G::DKP, G::LDK, 1, DK, G::NT>(aq, s_q, s_ql, s_gam, nullptr, tidf);
        store_tile<E, DK, G::DKP, G::LDK, 2, DK, G::NT>(ak, s_k, s_kl, s_gam, nullptr, tidf);
      } else {
        if constexpr (SCAL) store_tile<E, DK, G::DKP, G::LDK, 3, DK, G::NT>(aq, s_qh, s_qhl, s_gam, s_fq, tidf);
        store_tile<E, DK, G::DKP, G::LDK, 0, DK, G::NT>(aq, s_q, nullptr, s_gam, nullptr, tidf);
        store_tile<E, DK, G::DKP, G::LDK, 0, DK, G::NT>(ak, s_k, nullptr, s_gam, nullptr, tidf);
      }
      store_tile<E, DV, G::DVP, G::LDV, 0, DK, G::NT>(ado, s_do, nullptr, s_gam, nullptr, tidf);
      store_tile<E, DV, G::DVP, G::LDV, 0, DK, G::NT>(av_, s_v, nullptr, s_gam, nullptr, tidf);
    } else {
      if constexpr (DIAG) {
        store_tile<E, DK, G::DKP, G::LDK, 1, DK, G::NT>(aq, s_q, s_ql, s_gam, nullptr, tidf, gam_hi);
        __syncthreads();   // the dO tile overwrites Gam rows 32..63
      } else {
        store_tile<E, DK, G::DKP, G::LDK, 0, DK, G::NT>(aq, s_q, nullptr, s_gam, nullptr, tidf);
      }
      store_tile<E, DV, G::DVP, G::LDV, 0, DK, G::NT>(ado, s_do, nullptr, s_gam, nullptr, tidf);
    }
    __syncthreads();

    if constexpr (DIAG) {
      // dS' = diag(exp(Gam_last)) dS, the adjoint as the chunk's tail tokens see it
      // (dv, Y' and T3 below) and the carried part of the update at the end
      const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
#pragma unroll
      for (int m = 0; m < G::NKT; ++m) {
        const AV el = widen4<AV>(load4f(s_el + 16 * m + 4 * g));
#pragma unroll
        for (int cc = 0; cc < G::CPWV; ++cc) dS[m][cc] *= el;
      }
      if constexpr (APPLY) {
#pragma unroll
        for (int cc = 0; cc < G::CPWK; ++cc) {
          const float f = s_el[16 * (w + G::NW * cc) + i16];
#pragma unroll
          for (int nt = 0; nt < G::NVT; ++nt) dT[nt][cc] *= f;
        }
      }
    }

    if constexpr (APPLY) if (emit) {
      // ---- scores and score gradients (hi/lo) for the wave's tiles -------------------
#pragma unroll
      for (int s = 0; s < (N_SCORE_TILES + G::NW - 1) / G::NW; ++s) {
        const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
        if (s * G::NW + w >= N_SCORE_TILES) continue;
        const int idx = score_tile(s * G::NW + w);
        const int I = idx >> 2, J = idx & 3;
        AV xa = {0, 0, 0, 0}, xd = {0, 0, 0, 0};
        if (!score_tile_zero(idx)) {
          // q.k (its split cross terms in accumulators of their own) and dO.v
          // interleaved step by step, so that no MFMA waits on the one before it
          constexpr int NKD = G::DKP / 32, NKN = G::DVP / 32;
          AV xh = {0, 0, 0, 0}, xl = {0, 0, 0, 0};
#pragma unroll
          for (int st = 0; st < (NKD > NKN ? NKD : NKN); ++st) {
            if (st < NKD) {
              Frag<E> fa, fb;
              frag_direct(fa, s_q, G::LDK, 16 * I + i16, 32 * st, l);
              frag_direct(fb, s_k, G::LDK, 16 * J + i16, 32 * st, l);
              if constexpr (DIAG && SP) {
                Frag<E> fal, fbl;
                frag_direct(fal, s_ql, G::LDK, 16 * I + i16, 32 * st, l);
                frag_direct(fbl, s_kl, G::LDK, 16 * J + i16, 32 * st, l);
                mma(xa, fa, fb);
                mma(xh, fa, fbl);
                mma(xl, fal, fb);
              } else {
                mma(xa, fa, fb);
              }
            }
            if (st < NKN) {
              Frag<E> fa, fb;
              frag_direct(fa, s_do, G::LDV, 16 * I + i16, 32 * st, l);
              frag_direct(fb, s_v, G::LDV, 16 * J + i16, 32 * st, l);
              mma(xd, fa, fb);
            }
          }
          if constexpr (DIAG && SP) xa += xh + xl;
        }
        // the tiles are stored transposed (row = key token j, column = query token
        // i): the lane's four rows i become one 8-byte write per part
        // causal, same-sequence mask as selects on the sequence counts (a branch per
        // element here was compiled into code that dropped some of them)
        f32x4 va, vd;
        const int j = 16 * J + i16;
        const int sj = seg.index(j);
        AS prow[4], pcol = 0;   // scalar decay: P left of / below the diagonal
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int i = 16 * I + 4 * g + rr;
          const bool ok = i >= j && seg.index(i) == sj;
          va[rr] = ok ? (float)xa[rr] : 0.f;
          vd[rr] = ok ? (float)xd[rr] : 0.f;
          if constexpr (SCAL) {
            // exp(Gam_i - Gam_j) and the input weight of token j, applied once
            const float dec = ok ? __expf((float)(s_gam[i] - s_gam[j])) * s_w[j] : 0.f;
            // P_ij = exp(Gam_i - Gam_j) w_j (q_i.k_j)(dO_i.v_j)
            const AS pv = (AS)(ok ? xa[rr] : 0) * (AS)(ok ? xd[rr] : 0) * (AS)dec;
            prow[rr] = i > j ? pv : (AS)0;
            pcol += i > j ? pv : (AS)0;
            if (i == j) s_pdiag[i] = pv;
            va[rr] *= dec;
            vd[rr] *= dec;
          }
        }
        if constexpr (SCAL) {
          // the tile's row sums (over its 16 columns: the lanes of a group) and
          // column sums (over its 16 rows: rr and the lane groups), one slot per tile
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            AS x = prow[rr];
            if constexpr (sizeof(AS) == 4) {
              x = row_sum(x);
            } else {
              x += __shfl_xor(x, 1, 64);
              x += __shfl_xor(x, 2, 64);
              x += __shfl_xor(x, 4, 64);
              x += __shfl_xor(x, 8, 64);
            }
            if (i16 == 0) s_rowp[16 * idx + 4 * g + rr] = x;
          }
          pcol += __shfl_xor(pcol, 16, 64);
          pcol += __shfl_xor(pcol, 32, 64);
          if (g == 0) s_colp[16 * idx + i16] = pcol;
        }
        store_split4(s_ah, s_al, j * G::LDA + 16 * I + 4 * g, va);
        store_split4(s_dah, s_dal, j * G::LDA + 16 * I + 4 * g, vd);
      }
      __syncthreads();

      // S0 rows of the owned d_k tiles (fp32, columns 16j + 4g .. +3), read here so
      // that the load overlaps the dv phase
      const float* cs = a.chunk_states + ((bh * nct + cbase + c) * DK) * (int64_t)DV;
      f32x4 s0r[G::CPWK][G::DVP / 16];
      {
        const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
#pragma unroll
        for (int cc = 0; cc < G::CPWK; ++cc) {
          const int dl = 16 * (w + G::NW * cc) + i16;
#pragma unroll
          for (int j = 0; j < G::DVP / 16; ++j) {
            const int n0 = 16 * j + 4 * g;
            s0r[cc][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (dl < DK && n0 < DV) s0r[cc][j] = *reinterpret_cast<const f32x4*>(cs + dl * DV + n0);
          }
          if constexpr (DIAG && !GL_LDS) {
            const int d0 = 16 * (w + G::NW * cc) + 4 * g;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
              gl[cc][I] = f32x4{0.f, 0.f, 0.f, 0.f};
              if (d0 < DK && (full || 16 * I + i16 < nv))
                gl[cc][I] = *reinterpret_cast<const f32x4*>(a.g + tok_off(b, t0, h, a.T, a.H, DK) + tok_rel(16 * I + i16, a.H, DK) + d0);
            }
          }
        }
      }

      // ---- dv^T tiles: rows = owned d_v tiles, columns = tokens j ---------------------
      GE* dvp = reinterpret_cast<GE*>(a.dv);
#pragma unroll
      for (int cc = 0; cc < G::CPWV; ++cc) {
        const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
        const int cn = w + G::NW * cc;
        if (cn >= G::NVT) continue;
        // inter part K^ dS' for the four token blocks, contracting over d_k in
        // 32-wide steps (outer) so one split dS fragment is live at a time
        AV av[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) av[J] = AV{0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < G::DKP / 32; ++kb) {
          const AV lo = dS[2 * kb][cc], hi = dS[2 * kb + 1][cc];
          Frag<E> fs, fsl;
          acc_to_frag_split(fs, fsl, lo, hi);
#pragma unroll
          for (int J0 = 0; J0 < 4; J0 += GB) {
            Frag<E> fb[GB], fbl[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) {
              frag_direct_perm(fb[u], s_k, G::LDK, 16 * (J0 + u) + i16, 32 * kb, l);
              if constexpr (DIAG && SP) frag_direct_perm(fbl[u], s_kl, G::LDK, 16 * (J0 + u) + i16, 32 * kb, l);
            }
#pragma unroll
            for (int u = 0; u < GB; ++u) mma(av[J0 + u], fs, fb[u]);
            if constexpr (DIAG && SP) {
#pragma unroll
              for (int u = 0; u < GB; ++u) mma(av[J0 + u], fs, fbl[u]);
            }
            if constexpr (SP) {
#pragma unroll
              for (int u = 0; u < GB; ++u) mma(av[J0 + u], fsl, fb[u]);
            }
          }
        }
        Frag<E> fdo[2];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) frag_tr(fdo[ib], s_do, G::LDV, 32 * ib, 16 * cn, l);
        // intra part: score-tile blocks ib = 0 (query tokens 0..31, key blocks 0 and
        // 1) and ib = 1 (every key block)
        AV accv[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) accv[J] = av[J] * s_fk[16 * J + i16];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
          for (int J0 = 0; J0 < (ib == 0 ? 2 : 4); J0 += GB) {
            constexpr int U = GB;
            Frag<E> fb[U], fbl[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
              if (ib == 0 && J0 + u >= 2) continue;
              frag_direct(fb[u], s_ah, G::LDA, 16 * (J0 + u) + i16, 32 * ib, l);
              if constexpr (SP) frag_direct(fbl[u], s_al, G::LDA, 16 * (J0 + u) + i16, 32 * ib, l);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
              if (!(ib == 0 && J0 + u >= 2)) mma(accv[J0 + u], fdo[ib], fb[u]);
            if constexpr (SP) {
#pragma unroll
              for (int u = 0; u < U; ++u)
                if (!(ib == 0 && J0 + u >= 2)) mma(accv[J0 + u], fdo[ib], fbl[u]);
            }
          }
        }
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const int tj = 16 * J + i16;
          const int n0 = 16 * cn + 4 * g;
          if (n0 < DV && (full || tj < nv)) store4(dvp + tok_off(b, t0, h, a.T, a.H, DV) + tok_rel(tj, a.H, DV) + n0, accv[J]);
        }
      }

      // ---- dq^T and dk^T tiles: rows = owned d_k tiles, columns = tokens ---------------
      GE* dqp = reinterpret_cast<GE*>(a.dq);
      GE* dkp = reinterpret_cast<GE*>(a.dk);
      AS u1p[4] = {0, 0, 0, 0}, u4p[4] = {0, 0, 0, 0};  // scalar: per-I token partials
      AS t3p = 0;                                        // scalar: T3 partial
      // diagonal dg: wv holds w_t = Q~*(dq before exp(Gam)) - K~*(intra dk) after the dq
      // loop, then r_t = z_t - w_t with z_t = K~*(tail Y'); dg_t = sum_s w_s + T3 +
      // sum_{s<t} r_s (suffix sums of w plus prefix sums of z, rearranged)
      f32x4 wv[G::CPWK][4], wtot[G::CPWK];
      float t3r[DIAG ? G::CPWK : 1];   // diagonal: T3 of the lane's key dim 16 cm + i16
#pragma unroll
      for (int cc = 0; cc < G::CPWK; ++cc) {
        const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
        const int cm = w + G::NW * cc;
        if (cm >= G::NKT) continue;
        const int dl = 16 * cm + i16;        // lane-fixed key dim of the S0 / dS^T fragments
        // X^T = S0 dO^T for the four token blocks, contracting over d_v in 32-wide
        // steps (outer) so only one split S0 fragment is live at a time. S0 is read
        // in the permuted order {32kn + 4g + e, 32kn + 16 + 4g + e}, the positions the
        // dS^T accumulators hold, so T3 is an elementwise product on the way.
        AS t3 = 0;
        AV ax[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) ax[I] = AV{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < G::DVP / 32; ++kn) {
          float x[8];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const f32x4 sv = s0r[cc][2 * kn + hh];
            const AV tv = dT[2 * kn + hh][cc];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[4 * hh + e] = sv[e];
              t3 += (AS)sv[e] * (AS)tv[e];
            }
          }
          Frag<E> fs0, fs0l;
          split_frag(fs0, fs0l, x);
#pragma unroll
          for (int I0 = 0; I0 < 4; I0 += GB) {
            Frag<E> fb[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) frag_direct_perm(fb[u], s_do, G::LDV, 16 * (I0 + u) + i16, 32 * kn, l);
#pragma unroll
            for (int u = 0; u < GB; ++u) mma(ax[I0 + u], fs0, fb[u]);
            if constexpr (SP) {
#pragma unroll
              for (int u = 0; u < GB; ++u) mma(ax[I0 + u], fs0l, fb[u]);
            }
          }
        }
        if constexpr (HAS_DG) {
          t3 += __shfl_xor(t3, 16, 64);
          t3 += __shfl_xor(t3, 32, 64);
          if constexpr (DIAG) {
            t3r[cc] = (float)t3;   // for key dim dl in every lane of column i16; dS^T carries exp(Gam_last[d])
          } else {
            if (g == 0) t3p += t3;
          }
        }
        // dq^T = (live X^T) + intra, per token block
        {
          f32x4 gcar = {0.f, 0.f, 0.f, 0.f};
          Frag<E> fkt[2], fktl[2];
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) {
            frag_tr(fkt[jb], s_k, G::LDK, 32 * jb, 16 * cm, l);
            if constexpr (DIAG && SP) frag_tr(fktl[jb], s_kl, G::LDK, 32 * jb, 16 * cm, l);
          }
          // intra part for the four token blocks, term by term over the blocks (key
          // blocks jb = 0 for every query block, jb = 1 for query blocks 2 and 3)
          AV accq[4];
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            const int ti = 16 * I + i16;
            if constexpr (SCAL) {
              const f32x4 q4 = load4f(s_q + ti * G::LDK + 16 * cm + 4 * g);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) u1p[I] += (AS)q4[rr] * (AS)ax[I][rr];
            }
            accq[I] = ax[I] * s_fq[ti];
          }
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
            for (int I0 = 2 * jb; I0 < 4; I0 += GB) {
              constexpr int U = GB;
              Frag<E> fb[U], fbl[U];
#pragma unroll
              for (int u = 0; u < U; ++u) {
                if (I0 + u >= 4) continue;
                frag_tr(fb[u], s_dah, G::LDA, 32 * jb, 16 * (I0 + u), l);
                if constexpr (SP) frag_tr(fbl[u], s_dal, G::LDA, 32 * jb, 16 * (I0 + u), l);
              }
#pragma unroll
              for (int u = 0; u < U; ++u)
                if (I0 + u < 4) mma(accq[I0 + u], fkt[jb], fb[u]);
              if constexpr (SP) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                  if (I0 + u < 4) mma(accq[I0 + u], fkt[jb], fbl[u]);
              }
              if constexpr (DIAG && SP) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                  if (I0 + u < 4) mma(accq[I0 + u], fktl[jb], fb[u]);
              }
            }
          }
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            const int ti = 16 * I + i16;
            AV acc = accq[I];
            const int d0 = 16 * cm + 4 * g;
            if constexpr (DIAG) {
              const f32x4 gm = lane_gamma(gl[cc][I], gcar);
              gl[cc][I] = gm;
              // Q~ (hi + lo) at the lane's four dims; columns past d_k hold zeros
              f32x4 q4 = load4f(s_q + ti * G::LDK + d0);
              if constexpr (SP) q4 += load4f(s_ql + ti * G::LDK + d0);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int d = d0 + rr;
                const bool ok = d < DK;
                wv[cc][I][rr] = ok ? q4[rr] * (float)acc[rr] : 0.f;
                acc[rr] *= ok ? __expf(gm[rr]) : 0.f;
              }
            }
            if (d0 < DK && (full || ti < nv)) store4(dqp + tok_off(b, t0, h, a.T, a.H, DK) + tok_rel(ti, a.H, DK) + d0, acc);
          }
        }
        // Y'^T = dS'^T V^T (dS' = dS scaled by exp(Gam_last[d]) for a diagonal decay),
        // contracting over d_v outer as above
        AV ay[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) ay[J] = AV{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < G::DVP / 32; ++kn) {
          float y[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[e] = (float)dT[2 * kn][cc][e];
            y[4 + e] = (float)dT[2 * kn + 1][cc][e];
          }
          Frag<E> fdt, fdtl;
          split_frag(fdt, fdtl, y);
#pragma unroll
          for (int J0 = 0; J0 < 4; J0 += GB) {
            Frag<E> fb[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) frag_direct_perm(fb[u], s_v, G::LDV, 16 * (J0 + u) + i16, 32 * kn, l);
#pragma unroll
            for (int u = 0; u < GB; ++u) mma(ay[J0 + u], fdt, fb[u]);
            if constexpr (SP) {
#pragma unroll
              for (int u = 0; u < GB; ++u) mma(ay[J0 + u], fdtl, fb[u]);
            }
          }
        }
        // dk^T = tail Y'^T + intra, per token block
        if constexpr (DIAG) wtot[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
          Frag<E> fqt[2], fqtl[2];
#pragma unroll
          for (int jb = 0; jb < 2; ++jb) {
            frag_tr(fqt[jb], s_q, G::LDK, 32 * jb, 16 * cm, l);
            if constexpr (DIAG && SP) frag_tr(fqtl[jb], s_ql, G::LDK, 32 * jb, 16 * cm, l);
          }
          // intra part for the four token blocks, term by term over the blocks (query
          // blocks ib = 0 for key blocks 0 and 1, ib = 1 for every key block)
          AV acck[4];
#pragma unroll
          for (int J = 0; J < 4; ++J) acck[J] = AV{0, 0, 0, 0};
#pragma unroll
          for (int ib = 0; ib < 2; ++ib) {
            const int nj = ib == 0 ? 2 : 4;
#pragma unroll
            for (int J0 = 0; J0 < nj; J0 += GB) {
              constexpr int U = GB;
              Frag<E> fb[U], fbl[U];
#pragma unroll
              for (int u = 0; u < U; ++u) {
                if (J0 + u >= nj) continue;
                frag_direct(fb[u], s_dah, G::LDA, 16 * (J0 + u) + i16, 32 * ib, l);
                if constexpr (SP) frag_direct(fbl[u], s_dal, G::LDA, 16 * (J0 + u) + i16, 32 * ib, l);
              }
#pragma unroll
              for (int u = 0; u < U; ++u)
                if (J0 + u < nj) mma(acck[J0 + u], fqt[ib], fb[u]);
              if constexpr (SP) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                  if (J0 + u < nj) mma(acck[J0 + u], fqt[ib], fbl[u]);
              }
              if constexpr (DIAG && SP) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                  if (J0 + u < nj) mma(acck[J0 + u], fqtl[ib], fb[u]);
              }
            }
          }
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            const int tj = 16 * J + i16;
            AV yv = ay[J] * s_fk[tj];
            if constexpr (SCAL) {
              const f32x4 k4 = load4f(s_k + tj * G::LDK + 16 * cm + 4 * g);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) u4p[J] += (AS)k4[rr] * (AS)yv[rr];
            }
            AV acc = acck[J];
            const int d0 = 16 * cm + 4 * g;
            if constexpr (DIAG) {
              const f32x4 gm = gl[cc][J];
              f32x4 k4 = load4f(s_k + tj * G::LDK + d0);
              if constexpr (SP) k4 += load4f(s_kl + tj * G::LDK + d0);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int d = d0 + rr;
                const bool ok = d < DK;
                const float kt = ok ? k4[rr] : 0.f;
                const float wfull = wv[cc][J][rr] - kt * (float)acc[rr];
                wtot[cc][rr] += wfull;
                wv[cc][J][rr] = kt * (float)yv[rr] - wfull;
                acc[rr] = ok ? (acc[rr] + yv[rr]) * __expf(-gm[rr]) : 0.f;
              }
            } else {
              acc += yv;
            }
            if (d0 < DK && (full || tj < nv)) store4(dkp + tok_off(b, t0, h, a.T, a.H, DK) + tok_rel(tj, a.H, DK) + d0, acc);
          }
        }
      }

      if constexpr (PF) {
        __syncthreads();   // every wave is past its last read of k, k-lo, v and the score tiles
        if (c > 0) {
          const int tidp = tid_pick<APPLY, G::NT>();
          prefetch(t0 - CH, tidp, CH, std::false_type{});   // every chunk but a shard's last is full
          nseg.load(seq_row, t0 - CH, tidp & 63);
        }
      }

      if constexpr (DIAG) {
#pragma unroll
        for (int cc = 0; cc < G::CPWK; ++cc) {
          const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
          const int cm = w + G::NW * cc;
          if (cm >= G::NKT) continue;
          const int d0 = 16 * cm + 4 * g;
          f32x4 t3v;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float t3 = __shfl(t3r[cc], 4 * g + rr, 64);   // lane 4g + rr holds key dim d0 + rr
            t3v[rr] = (d0 + rr < DK) ? keep * t3 : 0.f;
          }
          // total of w over the 64 tokens, and exclusive prefix sums of r over them
          const f32x4 base = row_total(wtot[cc]) + t3v;
          f32x4 pre_tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            const f32x4 x = row_scan(wv[cc][I]);
            f32x4 ex;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) ex[rr] = row_shr<1>(x[rr]);
            f32x4 dgv = base + ex + pre_tot;
            pre_tot += row_last(x);
            const int t = 16 * I + i16;
            if ((seg.starts >> t) & 1ull) dgv = f32x4{0.f, 0.f, 0.f, 0.f};
            if (d0 < DK && (full || t < nv)) store4(a.dg + tok_off(b, t0, h, a.T, a.H, DK) + tok_rel(t, a.H, DK) + d0, dgv);
          }
        }
      }

      if constexpr (SCAL) {
        // token partials: reduce over the lane groups, then across waves
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          AS x1 = u1p[I], x4 = u4p[I];
          x1 += __shfl_xor(x1, 16, 64);
          x1 += __shfl_xor(x1, 32, 64);
          x4 += __shfl_xor(x4, 16, 64);
          x4 += __shfl_xor(x4, 32, 64);
          if (g == 0) {
            s_u1[w * CH + 16 * I + i16] = x1;
            s_u4[w * CH + 16 * I + i16] = x4;
          }
        }
        if constexpr (sizeof(AS) == 4) t3p = wave_total(g == 0 ? t3p : (AS)0);
        else t3p = wave_sum(g == 0 ? t3p : (AS)0);
        if (l == 0) s_red[w] = t3p;
        __syncthreads();
        if (w == 0) {
          const int t = l;
          AS u1 = 0, u4 = 0;
#pragma unroll
          for (int ww = 0; ww < G::NW; ++ww) {
            u1 += s_u1[ww * CH + t];
            u4 += s_u4[ww * CH + t];
          }
          u1 *= s_fq[t];
          // T2 step: row t left of the diagonal minus column t below it, from the
          // score tiles' row sums (tiles (t/16, J), J <= t/16) and column sums
          // (tiles (I, t/16), I >= t/16)
          AS rowl = 0, colb = 0;
          const int bt = t >> 4, tt = t & 15;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (u <= bt) rowl += s_rowp[16 * (4 * bt + u) + tt];
            if (u >= bt) colb += s_colp[16 * (4 * u + bt) + tt];
          }
          AS x = u1 + rowl - colb;
          AS y4 = u4;
          if constexpr (sizeof(AS) == 4) {
            // suffix sums of x (the total less the prefix before t), exclusive
            // prefix sums of u4
            const float px = wave_scan(x);
            x = lane_value(px, 63) - px + x;
            y4 = wave_scan(u4);
          } else {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
              const AS y = __shfl_down(x, off, 64);
              if (t + off < 64) x += y;
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
              const AS y = __shfl_up(y4, off, 64);
              if (t >= off) y4 += y;
            }
          }
          y4 -= u4;
          AS t3s = 0;
#pragma unroll
          for (int ww = 0; ww < G::NW; ++ww) t3s += s_red[ww];
          const AS t3 = (AS)(keep * __expf((float)s_gam[CH - 1])) * t3s;
          AS dgv = x + y4 + t3;
          if ((seg.starts >> t) & 1ull) dgv = 0;
          if (t < nv) a.dg[(b * a.T + t0 + t) * a.H + h] = (float)dgv;
          // input-weight gradient dw_t = k_t^T dS_t v_t: the intra part is column t
          // of the P tile on and below the diagonal, the tail part is u4; both carry
          // w_t (in the score decay and the tail factor), divided out here
          if (a.dw && t < nv)
            a.dw[(b * a.T + t0 + t) * a.H + h] = (float)((colb + s_pdiag[t] + u4) / (AS)s_w[t]);
        }
      }
    }

    // ---- dS <- [no start] diag(exp(Gam_last)) dS + sum_i live_i Q^_i dO_i^T ----------
      const int l = lane_pick<APPLY>(), g = l >> 4, i16 = l & 15;
    // (and the same for dS^T)
    {
      // carried part: keep * dS' (diagonal: already scaled), keep * exp(Gam_last) dS
      // (scalar), keep * dS (none); keep = 0 when the chunk holds a start
      const float f = SCAL ? keep * __expf((float)s_gam[CH - 1]) : keep;
      if (SCAL || seg.any()) {
#pragma unroll
        for (int m = 0; m < G::NKT; ++m)
#pragma unroll
          for (int cc = 0; cc < G::CPWV; ++cc) dS[m][cc] *= f;
        if constexpr (APPLY) {
#pragma unroll
          for (int cc = 0; cc < G::CPWK; ++cc)
#pragma unroll
            for (int nt = 0; nt < G::NVT; ++nt) dT[nt][cc] *= f;
        }
      }
      // token mask for Q^ where it is not baked into a tile (diagonal / no decay, packed chunks)
      const bool mask_tok = !SCAL && seg.any();
      constexpr bool QSPLIT = SP && (DIAG || SCAL);
      // dS part: a scalar decay's token factors fq = live exp(Gam) scale the dO
      // fragments (two per token block) instead, split hi/lo, against the plain q
      // tile; a diagonal decay's depend on the key dim and sit in the Q~ tiles
      constexpr bool DOSC = SCAL;
      constexpr bool QSPLIT_S = QSPLIT && !DOSC, LO_B = DOSC && SP;
      const E* const qs_h = DOSC ? s_q : qhat_h;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<E> fdo[G::CPWV], fdol[LO_B ? G::CPWV : 1];
#pragma unroll
        for (int cc = 0; cc < G::CPWV; ++cc) {
          const int cn = w + G::NW * cc;
          if (cn >= G::NVT) continue;
          frag_tr(fdo[cc], s_do, G::LDV, 32 * kb, 16 * cn, l);
          if constexpr (DOSC) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = to_f(fdo[cc].v[e]) * s_fq[32 * kb + kidx(e, l)];
            if constexpr (LO_B) {
              split_frag(fdo[cc], fdol[cc], x);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) frag_set(fdo[cc], e, x[e]);
            }
          }
        }
        // dS[d][n] += sum_i Q^[i][d] dO[i][n]   (rows: every d tile; columns: owned n tiles).
        // Apply with GB > 1: four row tiles at a time, the hi parts and then the lo
        // parts. The prepare walk runs four waves per SIMD, which cover each other's
        // MFMA latency, and has no registers to spare: one row tile at a time.
        constexpr int UM = (!APPLY || GB == 1) ? 1 : G::NKT < 4 ? G::NKT : 4;
#pragma unroll
        for (int m0 = 0; m0 < G::NKT; m0 += UM) {
          Frag<E> fa[UM], fal[UM];
#pragma unroll
          for (int u = 0; u < UM; ++u) {
            frag_tr(fa[u], qs_h, G::LDK, 32 * kb, 16 * (m0 + u), l);
            if constexpr (QSPLIT_S) frag_tr(fal[u], qhat_l, G::LDK, 32 * kb, 16 * (m0 + u), l);
            if (mask_tok) {
              frag_scale_tokens(fa[u], s_fq, 32 * kb, false, l);
              if constexpr (QSPLIT_S) frag_scale_tokens(fal[u], s_fq, 32 * kb, false, l);
            }
          }
          if constexpr (UM == 1) {
#pragma unroll
            for (int cc = 0; cc < G::CPWV; ++cc)
              if (w + G::NW * cc < G::NVT) {
                if constexpr (QSPLIT_S) {
                  mma2a(dS[m0][cc], fa[0], fal[0], fdo[cc]);
                } else {
                  mma(dS[m0][cc], fa[0], fdo[cc]);
                  if constexpr (LO_B) mma(dS[m0][cc], fa[0], fdol[cc]);
                }
              }
          } else {
#pragma unroll
            for (int u = 0; u < UM; ++u)
#pragma unroll
              for (int cc = 0; cc < G::CPWV; ++cc)
                if (w + G::NW * cc < G::NVT) mma(dS[m0 + u][cc], fa[u], fdo[cc]);
            if constexpr (QSPLIT_S || LO_B) {
#pragma unroll
              for (int u = 0; u < UM; ++u)
#pragma unroll
                for (int cc = 0; cc < G::CPWV; ++cc)
                  if (w + G::NW * cc < G::NVT) {
                    if constexpr (QSPLIT_S) mma(dS[m0 + u][cc], fal[u], fdo[cc]);
                    else mma(dS[m0 + u][cc], fa[u], fdol[cc]);
                  }
            }
          }
        }
        // dS^T[n][d] += sum_i dO[i][n] Q^[i][d]   (rows: every n tile; columns: owned d tiles)
        if constexpr (APPLY) {
#pragma unroll
          for (int cc = 0; cc < G::CPWK; ++cc) {
            const int cm = w + G::NW * cc;
            if (cm >= G::NKT) continue;
            Frag<E> qa, qal;
            frag_tr(qa, qhat_h, G::LDK, 32 * kb, 16 * cm, l);
            if constexpr (QSPLIT) frag_tr(qal, qhat_l, G::LDK, 32 * kb, 16 * cm, l);
            else frag_zero(qal);
            if (mask_tok) {
              frag_scale_tokens(qa, s_fq, 32 * kb, false, l);
              frag_scale_tokens(qal, s_fq, 32 * kb, false, l);
            }
            constexpr int UN = GB == 1 ? 1 : G::NVT < 4 ? G::NVT : 4;
#pragma unroll
            for (int n0 = 0; n0 < G::NVT; n0 += UN) {
              Frag<E> fd[UN];
#pragma unroll
              for (int u = 0; u < UN; ++u) frag_tr(fd[u], s_do, G::LDV, 32 * kb, 16 * (n0 + u), l);
#pragma unroll
              for (int u = 0; u < UN; ++u) mma(dT[n0 + u][cc], fd[u], qa);
              if constexpr (QSPLIT) {
#pragma unroll
                for (int u = 0; u < UN; ++u) mma(dT[n0 + u][cc], fd[u], qal);
              }
            }
          }
        }
      }
    }
    __syncthreads();
  }

  if constexpr (!APPLY) {
    float* rec = a.summary + (int64_t)(r * a.B * a.H + bh) * a.W;
    const float keep = any_start ? 0.f : 1.f;
    if constexpr (DIAG) {
      if (threadIdx.x < DK) rec[threadIdx.x] = keep * __expf((float)gsum);
    } else {
      if (threadIdx.x < 4) {
        float mval = SCAL ? __expf((float)gsum) : 1.f;
        rec[threadIdx.x] = threadIdx.x == 0 ? keep * mval : 0.f;
      }
    }
    float* gm = rec + a.m_slot;
#pragma unroll
    for (int m = 0; m < G::NKT; ++m)
#pragma unroll
      for (int cc = 0; cc < G::CPWV; ++cc) {
        const int cn = w + G::NW * cc;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = 16 * m + 4 * g + rr, n = 16 * cn + i16;
          if (cn < G::NVT && d < DK && n < DV) gm[d * DV + n] = (float)dS[m][cc][rr];
        }
      }
  }
}

#define CPLA_INST_BWD(E, DK, DV, DEC)                                              \
  template __global__ void bwd_walk<E, DK, DV, DEC, false, false, false>(BwdArgs); \
  template __global__ void bwd_walk<E, DK, DV, DEC, true, false, false>(BwdArgs);  \
  template __global__ void bwd_walk<E, DK, DV, DEC, false, false, true>(BwdArgs);  \
  template __global__ void bwd_walk<E, DK, DV, DEC, true, false, true>(BwdArgs);   \
  template __global__ void bwd_walk<E, DK, DV, DEC, true, false, false, false, false>(BwdArgs); \
  template __global__ void bwd_walk<E, DK, DV, DEC, true, false, true, false, false>(BwdArgs);
#define CPLA_INST_BWD_SPLIT(E, DK, DV, DEC, GF)                                           \
  template __global__ void bwd_walk<E, DK, DV, DEC, true, GF, false, true>(BwdArgs);     \
  template __global__ void bwd_walk<E, DK, DV, DEC, true, GF, true, true>(BwdArgs);      \
  template __global__ void bwd_walk<E, DK, DV, DEC, true, GF, false, true, false>(BwdArgs); \
  template __global__ void bwd_walk<E, DK, DV, DEC, true, GF, true, true, false>(BwdArgs);
#define CPLA_INST_BWD3(E, D) CPLA_INST_BWD(E, D, D, 0) CPLA_INST_BWD(E, D, D, 1) CPLA_INST_BWD(E, D, D, 2) \
  CPLA_INST_BWD_SPLIT(E, D, D, 0, false) CPLA_INST_BWD_SPLIT(E, D, D, 1, false)
#define CPLA_INST_BWD3X(E, DK, DV) CPLA_INST_BWD(E, DK, DV, 0) CPLA_INST_BWD(E, DK, DV, 1) CPLA_INST_BWD(E, DK, DV, 2) \
  CPLA_INST_BWD_SPLIT(E, DK, DV, 0, false) CPLA_INST_BWD_SPLIT(E, DK, DV, 1, false)
CPLA_INST_BWD3(bf16_t, 16)
CPLA_INST_BWD3(bf16_t, 64)
CPLA_INST_BWD3(bf16_t, 128)
CPLA_INST_BWD3X(bf16_t, 64, 128)
CPLA_INST_BWD3X(bf16_t, 128, 64)
// fp32 gradients from bf16 inputs: the scalar decay (the Mamba2 parametrisation)
#define CPLA_INST_BWD_GF32(DK, DV)                                                   \
  template __global__ void bwd_walk<bf16_t, DK, DV, 1, true, true, false>(BwdArgs); \
  template __global__ void bwd_walk<bf16_t, DK, DV, 1, true, true, true>(BwdArgs);  \
  template __global__ void bwd_walk<bf16_t, DK, DV, 1, true, true, false, false, false>(BwdArgs); \
  template __global__ void bwd_walk<bf16_t, DK, DV, 1, true, true, true, false, false>(BwdArgs); \
  CPLA_INST_BWD_SPLIT(bf16_t, DK, DV, 1, true)
CPLA_INST_BWD_GF32(16, 16)
CPLA_INST_BWD_GF32(64, 64)
CPLA_INST_BWD_GF32(128, 128)
CPLA_INST_BWD_GF32(64, 128)
CPLA_INST_BWD_GF32(128, 64)
CPLA_INST_BWD3(float, 16)
CPLA_INST_BWD3(float, 64)

}  // namespace cpla
