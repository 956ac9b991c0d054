// Per-chunk staging shared by the forward and backward shard walks.
//
// Inside one 64-token chunk of one (b, h) row, with g the log-decay:
//   Gam_i    = sum_{s <= i} g_s          (inclusive, per key dim for a diagonal decay)
//   live_i   = no packed-sequence start at chunk positions <= i (token sees the
//              incoming state)
//   tail_j   = no start after j (token reaches the outgoing state)
// The intra-chunk decay between tokens j <= i of one sequence is
// exp(Gam_i - Gam_j). For a diagonal decay it is factorised into the operand
// tiles Q~ = Q * exp(Gam) and K~ = K * exp(-Gam); for a scalar decay it is
// applied to the 64x64 score tile and to per-token factors, which never
// exponentiate a positive exponent.
#pragma once
#include "device.hpp"
#include "shards.hpp"

namespace cpla {

enum { DECAY_NONE = 0, DECAY_SCALAR = 1, DECAY_DIAG = 2 };

template <typename E, int DK, int DV>
struct Geo {
  static constexpr int DKP = DK < 32 ? 32 : DK;   // contraction depth padded to one MFMA step
  static constexpr int DVP = DV < 32 ? 32 : DV;
  static constexpr int PAD = lds_pad<E>();
  static constexpr int LDK = DKP + PAD;           // LDS row stride of [token][dk] tiles
  static constexpr int LDV = DVP + PAD;
  static constexpr int LDA = CH + PAD;            // LDS row stride of 64x64 tiles
  static constexpr int NKT = DKP / 16;            // 16-wide tiles along dk
  static constexpr int NVT = DVP / 16;
  static constexpr int NW = waves_for(DKP);       // waves per workgroup
  static constexpr int NT = 64 * NW;              // threads per workgroup
  static constexpr int CPWK = (NKT + NW - 1) / NW;  // dk tiles owned per wave
  static constexpr int CPWV = (NVT + NW - 1) / NW;
  static constexpr int TILE_K = CH * LDK;         // elements
  static constexpr int TILE_V = CH * LDV;
  static constexpr int TILE_A = CH * LDA;
};

// Score tiles (I, J) of the 64x64 lower triangle, index I*4 + J, dealt round
// robin to the waves: wave w takes entries w, w + NW, ... of this list. Entries
// 1 = (0,1) and 11 = (2,3) are upper tiles that are read by 32-deep token
// contractions and must hold zeros.
constexpr int N_SCORE_TILES = 12;
// The list {0, 4, 5, 8, 9, 10, 12, 13, 14, 15, 1, 11} packed as 4-bit fields, so
// the lookup is register arithmetic rather than a load from a constant table
// (a global load inside the chunk loop would make the wave wait for every
// outstanding memory operation).
__device__ __forceinline__ int score_tile(int k) { return (int)((0xB1FEDCA98540ull >> (4 * k)) & 15ull); }
__device__ __forceinline__ bool score_tile_zero(int idx) { return idx == 1 || idx == 11; }

// Row base offset of token t of row (b, h) in a [B, T, H, D] tensor.
__device__ __forceinline__ int64_t tok_off(int64_t b, int64_t t, int64_t h, int64_t T, int64_t H, int D) {
  return ((b * T + t) * H + h) * (int64_t)D;
}
// Offset of token t0 + i from token t0 of the same row: the lane-dependent part of
// an address as a 32-bit product (i < 64, H * D < 2^23), added to a chunk base
// that is the same for the whole workgroup.
__device__ __forceinline__ int tok_rel(int i, int64_t H, int D) { return i * ((int)H * D); }

// ---- register prefetch ------------------------------------------------------------
// A walk issues the next chunk's global loads into these registers before it
// computes the current chunk, and writes them to LDS afterwards, so HBM latency
// overlaps MFMA and LDS work instead of stalling every chunk.

// Sequence ids of the chunk's tokens (packed sequences): one token per lane.
struct SegRegs {
  int cur, prev;
  // TAIL: n = tokens of the chunk inside the shard (fewer than 64 only in a
  // shard's last chunk); the rows past them continue the last sequence (no start)
  template <bool TAIL = false>
  __device__ __forceinline__ void load(const int32_t* seq_idx, int64_t t0, int l = lane_id(), int n = CH) {
    if (!seq_idx) return;
    const int64_t t = t0 + l;
    if (!TAIL || l < n) {
      cur = seq_idx[t];
      prev = t > 0 ? seq_idx[t - 1] : -1;   // sequence ids are >= 0: token 0 starts one
    } else {
      cur = prev = 0;
    }
  }
  __device__ __forceinline__ ChunkSeg finish(const int32_t* seq_idx) const {
    ChunkSeg s;
    s.starts = seq_idx ? (uint64_t)__ballot(cur != prev) : 0ull;
    return s;
  }
};

// Log-decays of one chunk: diagonal -> thread (d = tid % DK, part = tid / DK)
// holds TOK consecutive tokens of key column d; scalar -> thread tid < 64 holds
// token tid.
template <int DK, int DECAY, int NT>
struct GamRegs {
  // diagonal: TPC threads share a key column, each holding TOK consecutive
  // tokens; the TPC parts of a column sit in one wave (lane = part * CPW + j,
  // column = wave * CPW + j), so the running totals pass between parts by
  // shuffles instead of through LDS
  static constexpr int TPC = (DECAY == DECAY_DIAG) ? NT / DK : 1;
  static constexpr int TOK = (DECAY == DECAY_DIAG) ? CH / TPC : 1;
  static constexpr int CPW = 64 / TPC;
  static_assert(DECAY != DECAY_DIAG || (TPC <= 64 && 64 % TPC == 0), "column split must fit a wave");
  float v[TOK];
  float wt = 1.f;   // scalar decay: the token's input weight (1 without one)
  __device__ __forceinline__ static int column(int tid) { return (tid >> 6) * CPW + (tid & 63) % CPW; }
  // scalar decay with a per-token input weight: thread tid < 64 holds token tid's
  template <bool TAIL = false>
  __device__ __forceinline__ void load_w(const float* __restrict__ w, int64_t b, int64_t h, int64_t t0, int64_t T,
                                         int64_t H, int tid = threadIdx.x, int n = CH) {
    if constexpr (DECAY == DECAY_SCALAR)
      if (w && tid < (TAIL ? n : CH)) wt = w[(b * T + t0 + tid) * H + h];
  }
  __device__ __forceinline__ static int part(int tid) { return (tid & 63) / CPW; }
  // TAIL: n = tokens of the chunk inside the shard; the rows past them read as g = 0
  template <bool TAIL = false>
  __device__ __forceinline__ void load(const float* __restrict__ g, int64_t b, int64_t h, int64_t t0, int64_t T,
                                       int64_t H, int tid = threadIdx.x, int n = CH) {
    if constexpr (DECAY == DECAY_DIAG) {
      const int d = column(tid), i0 = part(tid) * TOK;
      const float* src = g + ((b * T + t0 + i0) * H + h) * DK + d;
#pragma unroll
      for (int s = 0; s < TOK; ++s) {
        if constexpr (!TAIL) {
          v[s] = src[(int64_t)s * H * DK];
        } else {   // rows past the shard: load the last valid row (in bounds), then 0
          const int row = i0 + s < n ? s : n - 1 - i0;
          const float x = src[(int64_t)row * H * DK];
          v[s] = i0 + s < n ? x : 0.f;
        }
      }
    } else if constexpr (DECAY == DECAY_SCALAR) {
      if (tid < CH) v[0] = (!TAIL || tid < n) ? g[(b * T + t0 + tid) * H + h] : 0.f;
    }
  }
  // The values load() reads, copied by LDS DMA instead. Diagonal: value s of
  // lane l of wave w lands at buf[lds_row(w, s) + l], one 64-float row per
  // (w, s), each row shifted by lds_shift(s) < 64 words so that the lane-layout
  // reads below are bank-conflict free (rows of 64 words all start in bank 0
  // otherwise); a wave's rows take (TOK + 1) * 64 floats, the last 64 absorbing
  // the shifts, so the buffer holds NT / 64 * (TOK + 1) * 64 floats. Scalar:
  // token t at buf[t].
  static constexpr int DMA_FLOATS = (DECAY == DECAY_DIAG) ? NT / 64 * (TOK + 1) * 64 : CH;
  __device__ __forceinline__ static constexpr int lds_shift(int s) { return (s & 3) + 16 * ((s >> 2) & 3); }
  __device__ __forceinline__ static int lds_row(int w, int s) { return w * (TOK + 1) * 64 + s * 64 + lds_shift(s); }
  // Diagonal with 16-token parts of 16 columns (d_k 64 or 128): the wave's 64
  // tokens x 16 columns are copied by four 16-byte DMA instructions instead, one
  // per 16-token block I, which lands as 16 rows of 16 floats at blk(w, I); the
  // blocks are 272 floats apart, so the four parts' reads of one row fall in
  // different banks. It takes the same (TOK + 1) * 64 floats per wave.
  static constexpr bool DMA16 = DECAY == DECAY_DIAG && TOK == 16 && CPW == 16;
  __device__ __forceinline__ static int blk(int w, int I) { return (4 * w + I) * 272; }
  // TAIL: with n < CH (a shard's partial last chunk) lanes past the shard copy
  // nothing and load_lds returns 0 for them
  template <bool TAIL = false>
  __device__ __forceinline__ static void dma(const float* __restrict__ g, int64_t b, int64_t h, int64_t t0,
                                             int64_t T, int64_t H, float* buf, int tid, int w, int n = CH) {
    if constexpr (DMA16) {
      const int l = tid & 63, r = l >> 2;
      const float* src = g + ((b * T + t0 + r) * H + h) * DK + 16 * w + 4 * (l & 3);
#pragma unroll
      for (int I = 0; I < 4; ++I)
        if (!TAIL || 16 * I + r < n) lds_dma<16>(src + (int64_t)(16 * I) * H * DK, buf + blk(w, I));
    } else if constexpr (DECAY == DECAY_DIAG) {
      const int i0 = part(tid) * TOK;
      const float* src = g + ((b * T + t0 + i0) * H + h) * DK + column(tid);
#pragma unroll
      for (int s = 0; s < TOK; ++s)
        if (!TAIL || i0 + s < n) lds_dma<4>(src + (int64_t)s * H * DK, buf + lds_row(w, s));
    } else if constexpr (DECAY == DECAY_SCALAR) {
      if (tid < (TAIL ? n : CH)) lds_dma<4>(g + (b * T + t0 + tid) * H + h, buf + 64 * w);
    }
  }
  template <bool TAIL = false>
  __device__ __forceinline__ void load_lds(const float* buf, int tid, int n = CH) {
    if constexpr (DECAY == DECAY_DIAG) {
      const int w = tid >> 6, l = tid & 63, i0 = part(tid) * TOK;
      if constexpr (DMA16) {
#pragma unroll
        for (int s = 0; s < TOK; ++s) v[s] = buf[blk(w, l >> 4) + 16 * s + (l & 15)];
      } else {
#pragma unroll
        for (int s = 0; s < TOK; ++s) v[s] = buf[lds_row(w, s) + l];
      }
      if constexpr (TAIL) {
#pragma unroll
        for (int s = 0; s < TOK; ++s) v[s] = i0 + s < n ? v[s] : 0.f;
      }
    } else if constexpr (DECAY == DECAY_SCALAR) {
      if (tid < CH) v[0] = (!TAIL || tid < n) ? buf[tid] : 0.f;
    }
  }
  // Diagonal, TOK == CPW == 16 (d_k of 64 or 128): the raw log-decay of token
  // 16 I + (l % 16) at key dims 16 w + 4 (l / 16) + rr (rr = 0..3), the MFMA
  // accumulator layout of wave w's key tile, from the DMA buffer.
  template <bool TAIL = false>
  __device__ __forceinline__ static f32x4 lane_block(const float* buf, int w, int I, int l, int n = CH) {
    static_assert(DMA16, "lane layout needs 16-token parts of 16 columns");
    const f32x4 x = *reinterpret_cast<const f32x4*>(buf + blk(w, I) + 16 * (l & 15) + 4 * (l >> 4));
    if constexpr (!TAIL) return x;
    return 16 * I + (l & 15) >= n ? f32x4{0.f, 0.f, 0.f, 0.f} : x;
  }
};

// The chunk's cumulative log-decay from the loaded registers, into LDS:
//   scalar: gam[i] (64 floats);  diagonal: rows i < 32 at gam[i * DK + d] and
//   rows i >= 32 at gam_hi[(i - 32) * DK + d] (gam_hi = gam + 32 * DK when null:
//   one contiguous tile; a walk short of LDS passes a buffer it reuses later);
//   none: nothing.
// and the per-token factors
//   fq[i] = live_i * (scalar ? exp(Gam_i) : 1)
//   fk[j] = tail_j * (scalar ? exp(Gam_last - Gam_j) * w_j : 1)
// and, for a scalar decay, the input weights w_j (1 without them) into wl.
// Ends with a barrier.
// GT, the type of the Gam buffer: float, or double for a scalar decay with fp32
// inputs, whose exponent differences Gam_i - Gam_j would otherwise lose up to
// |Gam| * 2^-24 to the rounding of the running sums (a relative error of that size
// in the decay factor, far above fp32's own on sums that cancel).
template <int DK, int DECAY, int NT, typename GT>
__device__ __forceinline__ void finish_gamma(GamRegs<DK, DECAY, NT>& R, const ChunkSeg& seg, GT* gam,
                                             float* fq, float* fk, int tid = threadIdx.x,
                                             float* gam_hi = nullptr, float* wl = nullptr) {
  if constexpr (DECAY == DECAY_SCALAR) {
    if (tid < CH) {
      GT x = R.v[0];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const GT y = __shfl_up(x, off, 64);
        if (tid >= off) x += y;
      }
      gam[tid] = x;
      const GT last = __shfl(x, 63, 64);
      fq[tid] = seg.live(tid) ? __expf((float)x) : 0.f;
      fk[tid] = seg.tail(tid) ? __expf((float)(last - x)) * R.wt : 0.f;
      if (wl) wl[tid] = R.wt;
    }
  } else {
    if constexpr (DECAY == DECAY_DIAG) {
      using GR = GamRegs<DK, DECAY, NT>;
      constexpr int TOK = GR::TOK;
      const int d = GR::column(tid), part = GR::part(tid), j = (tid & 63) % GR::CPW;
#pragma unroll
      for (int s = 1; s < TOK; ++s) R.v[s] += R.v[s - 1];
      // totals of the earlier parts of this column (lanes p * CPW + j of this wave)
      float off = 0.f;
#pragma unroll
      for (int p = 0; p + 1 < GR::TPC; ++p) {
        const float tp = __shfl(R.v[TOK - 1], p * GR::CPW + j, 64);
        if (p < part) off += tp;
      }
      float* const g1 = gam_hi ? gam_hi - 32 * DK : gam;
#pragma unroll
      for (int s = 0; s < TOK; ++s) {
        const int t = part * TOK + s;
        (t < 32 ? gam : g1)[t * DK + d] = R.v[s] + off;
      }
    }
    if (tid < CH) {
      fq[tid] = seg.live(tid) ? 1.f : 0.f;
      fk[tid] = seg.tail(tid) ? 1.f : 0.f;
    }
  }
  __syncthreads();
}

// One [64][D] input tile as raw 16-byte vectors, dealt round robin to threads.
template <typename E, int D, int NT>
struct TileRegs {
  static constexpr int VEC = 16 / (int)sizeof(E);
  static constexpr int VPR = D / VEC;
  static constexpr int NV = CH * VPR;
  static constexpr int PER = (NV + NT - 1) / NT;
  f32x4 r[PER];
  // TAIL: n = tokens of the chunk inside the shard; the rows past them read as zeros
  template <bool TAIL = false>
  __device__ __forceinline__ void load(const E* __restrict__ src, int64_t b, int64_t h, int64_t t0, int64_t T,
                                       int64_t H, int tid = threadIdx.x, int n = CH) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * NT;
      if (v < NV) {
        const int i = v / VPR, c = (v % VPR) * VEC;
        if constexpr (!TAIL) {
          r[p] = *reinterpret_cast<const f32x4*>(src + tok_off(b, t0 + i, h, T, H, D) + c);
        } else {   // rows past the shard: load the last valid row (in bounds), then 0
          const f32x4 x = *reinterpret_cast<const f32x4*>(src + tok_off(b, t0 + (i < n ? i : n - 1), h, T, H, D) + c);
          r[p] = i < n ? x : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
  // The vectors load() reads, copied by LDS DMA instead: vector p of thread tid
  // lands at buf[(p * NT + tid) * VEC], one contiguous kilobyte per wave and p
  // (w = the calling wave); load_lds reads them back. buf holds CH * D elements.
  template <bool TAIL = false>
  __device__ __forceinline__ static void dma(const E* __restrict__ src, int64_t b, int64_t h, int64_t t0, int64_t T,
                                             int64_t H, E* buf, int tid, int w, int n = CH) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * NT;
      const int i = v / VPR, c = (v % VPR) * VEC;
      if (v < NV && (!TAIL || i < n))
        lds_dma<16>(src + tok_off(b, t0 + i, h, T, H, D) + c, buf + (p * NT + 64 * w) * VEC);
    }
  }
  template <bool TAIL = false>
  __device__ __forceinline__ void load_lds(const E* buf, int tid, int n = CH) {
#pragma unroll
    for (int p = 0; p < PER; ++p)
      if (tid + p * NT < NV) r[p] = *reinterpret_cast<const f32x4*>(buf + (p * NT + tid) * VEC);
    if constexpr (TAIL) {
#pragma unroll
      for (int p = 0; p < PER; ++p)
        if ((tid + p * NT) / VPR >= n) r[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Write prefetched vectors to LDS (row stride LD), zero-filling columns D..DP-1.
// MODE 0: copy into `hi`; 1: x*exp(Gam[i][d]); 2: x*exp(-Gam[i][d]); 3: x*fac[i] --
// scaled modes are stored split (hi, and lo for bf16). Gam rows as finish_gamma
// wrote them (gam_hi: rows 32..63, null for one contiguous tile). No barrier.
template <typename E, int D, int DP, int LD, int MODE, int DK, int NT, typename GT = float>
__device__ __forceinline__ void store_tile(const TileRegs<E, D, NT>& R, E* hi, E* lo, const GT* gam,
                                           const float* fac, int tid = threadIdx.x,
                                           const GT* gam_hi = nullptr) {
  using TR = TileRegs<E, D, NT>;
  constexpr int VEC = TR::VEC;
  const GT* const g1 = gam_hi ? gam_hi - 32 * DK : gam;
#pragma unroll
  for (int p = 0; p < TR::PER; ++p) {
    const int v = tid + p * NT;
    if (v >= TR::NV) continue;
    const int i = v / TR::VPR, c = (v % TR::VPR) * VEC;
    if constexpr (MODE == 0) {
      *reinterpret_cast<f32x4*>(hi + i * LD + c) = R.r[p];
      continue;
    }
    float x[VEC];
    if constexpr (sizeof(E) == 2) {
      const bf16x8 y = __builtin_bit_cast(bf16x8, R.r[p]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)y[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = R.r[p][e];
    }
    const GT* const grow = (i < 32 ? gam : g1) + i * DK + c;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if constexpr (MODE == 1) x[e] *= __expf((float)grow[e]);
      if constexpr (MODE == 2) x[e] *= __expf(-(float)grow[e]);
      if constexpr (MODE == 3) x[e] *= fac[i];
    }
    if constexpr (sizeof(E) == 2) {
      Frag<bf16_t> yh, yl;
      split_frag(yh, yl, x);
      *reinterpret_cast<bf16x8*>(hi + i * LD + c) = yh.v;
      *reinterpret_cast<bf16x8*>(lo + i * LD + c) = yl.v;
    } else {
      *reinterpret_cast<f32x4*>(hi + i * LD + c) = f32x4{x[0], x[1], x[2], x[3]};
    }
  }
  if constexpr (DP > D) {
    for (int v = tid; v < CH * (DP - D); v += NT) {
      const int i = v / (DP - D), c = D + v % (DP - D);
      hi[i * LD + c] = to_e<E>(0.f);
      if constexpr (MODE != 0 && sizeof(E) == 2) lo[i * LD + c] = to_e<E>(0.f);
    }
  }
}

// Multiply fragment slot e by fac[token(e)] (token-contracted operands).
template <typename E>
__device__ __forceinline__ void frag_scale_tokens(Frag<E>& f, const float* fac, int k0, bool perm,
                                                  int l = lane_id()) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int tok = k0 + (perm ? kidx_perm(e, l) : kidx(e, l));
    f.v[e] = to_e<E>(to_f(f.v[e]) * fac[tok]);
  }
}

// Load 4 consecutive tile elements (8-byte aligned for bf16, 16 for fp32) as fp32.
__device__ __forceinline__ f32x4 load4f(const bf16_t* p) {
  const bf16x4 y = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
}
__device__ __forceinline__ f32x4 load4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Store 4 consecutive values as hi (and lo) parts into two LDS tiles at the same
// offset (8-byte aligned for bf16, 16 for fp32).
__device__ __forceinline__ void store_split4(bf16_t* hi, bf16_t* lo, int off, const f32x4& x) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const bf16x4 h = __builtin_convertvector(x, bf16x4);
  const u32x2 hb = __builtin_bit_cast(u32x2, h);
  f32x4 r = x;
  float r0 = r[0], r1 = r[1], r2 = r[2], r3 = r[3];
  bf16_residual_pair(hb[0], r0, r1);
  bf16_residual_pair(hb[1], r2, r3);
  r = f32x4{r0, r1, r2, r3};
  *reinterpret_cast<bf16x4*>(hi + off) = h;
  *reinterpret_cast<bf16x4*>(lo + off) = __builtin_convertvector(r, bf16x4);
}
__device__ __forceinline__ void store_split4(float* hi, float*, int off, const f32x4& x) {
  *reinterpret_cast<f32x4*>(hi + off) = x;
}
__device__ __forceinline__ void store_split4(float* hi, float* lo, int off, const f64x4& x) {
  store_split4(hi, lo, off, narrow4(x));
}

// Store 4 consecutive values (output feature 4g..4g+3 of a 16-wide tile).
__device__ __forceinline__ void store4(bf16_t* p, const f32x4& x) {
  bf16x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (bf16_t)x[e];
  *reinterpret_cast<bf16x4*>(p) = y;
}
__device__ __forceinline__ void store4(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ void store4(float* p, const f64x4& x) { store4(p, narrow4(x)); }

}  // namespace cpla
