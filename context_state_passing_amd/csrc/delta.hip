// The gated delta rule: a dense d_k x d_k state transition on the same
// context-parallel protocol (Megatron-Core page core.ssm.context_parallel.chunkwise:
// S_out = M S_in + delta_S and dS_in = M^T dS_out + gamma for a general M; the
// axolotl-ringmaster README's Status table names gated-DeltaNet among the
// linear-attention variants validated on it).
//
//   S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  a_t = exp(g_t),
//   o_t = S_t^T q_t,  S_{t-1} := 0 where token t starts a packed sequence.
//
// Chunk form (64 tokens; Gam = segment-local inclusive cumsum of g, live_i = no
// start at or before i, D_ij = exp(Gam_i - Gam_j) for j <= i in one sequence):
//   A = strict-lower(beta_i D_ij k_i.k_j),   [U~ | W] = (I + A)^{-1} [beta V | beta live e^Gam K]
//   U = U~ - W S,   O = live e^Gam Q S + (tril(Q K^T) . D) U,
//   S <- live_last e^{Gam_last} S + K~^T U,  K~_j = [j in the last sequence] e^{Gam_last - Gam_j} k_j.
// The solve is the WY form of the product of the chunk's transitions: the
// chunk's own map is M_c = live_last e^{Gam_last} I - K~^T W.
//
// Kernels (one workgroup of eight waves each; contractions are MFMA products of
// fp32 LDS tiles, inputs widened on load: fp32 16x16x4 for fp32 inputs, split bf16
// 16x16x32 for bf16 inputs):
//   delta_wy      per chunk:  U~, W ((I + A)^{-1} by 16 x 16 blocks, then MFMA products)
//   delta_fwalk   per shard:  chunk walk of the state; prepare folds [delta_S | M]
//                             from [0 | I], apply saves chunk states and U
//   delta_scan    per (b,h):  composition S <- M S + delta_S over shards (or its
//                             transpose backwards)
//   delta_out     per chunk:  O (d = 64, bf16: formed by the apply walk instead)
//   delta_bwalk   per shard:  reverse walk of dS; prepare gives gamma, apply saves
//                             the chunk-end gradients and dU
//   delta_grad    per chunk:  dq, dk, dv, dg, dbeta (delta_grad_wide: the same over
//                             value slices)
// d_k = d_v in {16, 32, 64}, and 128 for bf16 inputs: there the walks split the
// state's columns over workgroups and the gradients take the value dimension in
// slices, as a fp32 state with the chunk's tiles does not fit one workgroup's LDS.
// At d = 64 (bf16) the apply and reverse walks and the gradients use the same
// splits so that two workgroups share a CU.
#include <type_traits>

#include "kernels.hpp"
#include "shards.hpp"

namespace cpla {
namespace {

constexpr int NTH = DELTA_THREADS, NWV = DELTA_THREADS / 64;
static_assert(NWV % 4 == 0, "a wave's score tiles share one column tile");

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One 16 x 16 output tile: acc += sum_{k < K} a(i, k) b(k, j). Lane l supplies
// A[l % 16][k] and B[k][l % 16] for its k of the step; the accumulator holds rows
// 4 (l / 16) + r, column l % 16.
// The sum over k is split so that lane group kk = l / 16 supplies k = kk K/4 + s
// at step s: a lane's operands then run over K/4 consecutive k, which row-major
// tiles serve with 16-byte LDS reads.
template <int K, class FA, class FB>
__device__ __forceinline__ f32x4 tile_mm(const FA& a, const FB& b, f32x4 acc) {
  constexpr int S = K / 4;
  const int l = lane_id(), x = l & 15, kk = l >> 4;
  float av[S], bv[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    av[s] = a(x, kk * S + s);
    bv[s] = b(kk * S + s, x);
  }
#pragma unroll
  for (int s = 0; s < S; ++s) acc = mfma_f32(av[s], bv[s], acc);
  return acc;
}

// The same tile product for bf16 inputs: every 32-deep step of k takes the eight
// consecutive k of lane group l / 16 (the layout of v_mfma_f32_16x16x32_bf16),
// splits each fp32 operand into bf16 hi + lo and issues hi*hi, hi*lo and lo*hi, so
// the product keeps about 16 significant bits per operand (the LDS tiles and
// intermediates stay fp32) at 3 bf16 MFMAs per 32-deep step instead of 8 fp32
// ones. An operand flagged exact (AX, BX) holds bf16 values exactly (a bf16 input
// read back from its widened tile, unscaled): its lo part is zero, so it is
// converted without a split and the products with its lo part are not issued (the
// sum is the same). fp32 inputs keep the fp32 product (tile_mm).
template <int K, bool AX, bool BX, class FA, class FB>
__device__ __forceinline__ f32x4 tile_mm_split(const FA& a, const FB& b, f32x4 acc) {
  static_assert(K % 32 == 0, "32-deep steps");
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  const int l = lane_id(), x = l & 15, kg = l >> 4;
#pragma unroll
  for (int st = 0; st < K / 32; ++st) {
    float av[8], bv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      av[e] = a(x, 32 * st + 8 * kg + e);
      bv[e] = b(32 * st + 8 * kg + e, x);
    }
    Frag<bf16_t> ah, al, bh, bl;
    if constexpr (AX) ah.v = __builtin_convertvector((f32x8{av[0], av[1], av[2], av[3], av[4], av[5], av[6], av[7]}), bf16x8);
    else split_frag(ah, al, av);
    if constexpr (BX) bh.v = __builtin_convertvector((f32x8{bv[0], bv[1], bv[2], bv[3], bv[4], bv[5], bv[6], bv[7]}), bf16x8);
    else split_frag(bh, bl, bv);
    mma(acc, ah, bh);
    if constexpr (!BX) mma(acc, ah, bl);
    if constexpr (!AX) mma(acc, al, bh);
  }
  return acc;
}
// tile_mm for fp32 inputs, tile_mm_split for bf16 inputs (K a multiple of 32)
template <int K, typename E, bool AX = false, bool BX = false, class FA, class FB>
__device__ __forceinline__ f32x4 tile_mm_e(const FA& a, const FB& b, f32x4 acc) {
  if constexpr (sizeof(E) == 2 && K % 32 == 0) return tile_mm_split<K, AX, BX>(a, b, acc);
  else return tile_mm<K>(a, b, acc);
}

template <int D> struct DGeo {
  static constexpr int LD = D + 4;            // row stride of a [64][D] or [D][D] tile (floats)
  static constexpr int LC = CH + 4;           // row stride of a [64][64] tile
  static constexpr int NTC = D / 16;          // column tiles of a [*][D] tile
  static constexpr int TILE = CH * LD;        // floats of a [64][D] tile
  static constexpr int TILE_C = CH * LC;      // floats of a [64][64] tile
};


// index of (b, t0, h) in a [B,T,H] layout: the chunk's first token; the chunk's
// rows follow at 32-bit offsets i H (i < 64, H d < 2^23)
__device__ __forceinline__ int64_t row0(int64_t b, int64_t t0, int64_t h, int64_t T, int64_t H) {
  return (b * T + t0) * H + h;
}

// Input tiles staged through registers: fetch() issues a thread's global loads
// (four elements each, in the input type), put() writes them widened to fp32 into
// an LDS tile. Fetching several tiles before putting any keeps all their loads in
// flight at once, and a walk fetches its next chunk while it computes the current
// one.
template <typename E> struct Raw4 { typedef f32x4 type; };
template <> struct Raw4<bf16_t> { typedef bf16x4 type; };
__device__ __forceinline__ f32x4 widen4(const f32x4& x) { return x; }
__device__ __forceinline__ f32x4 widen4(const bf16x4& x) {
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// [64][W] columns c0 .. c0 + W - 1 of rows t0 .. t0 + 63 of a [B,T,H,D] tensor
// (W = D: whole rows); rows past n read as zero. put() writes row i at dst + i ld.
template <typename E, int D, int W = D> struct RowTile {
  static constexpr int NV = CH * W / 4, PER = (NV + NTH - 1) / NTH;
  typedef typename Raw4<E>::type R;
  R v[PER];
  __device__ __forceinline__ void fetch(const E* src, int64_t b, int64_t h, int64_t t0, int n, int64_t T,
                                        int64_t H, int c0 = 0) {
    // the chunk's first row once in 64 bits, rows within it in 32 (i < 64, H D < 2^23)
    const E* base = src + ((b * T + t0) * H + h) * D + c0;
    const int rs = (int)H * D;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = threadIdx.x + p * NTH, i = e / (W / 4), c = 4 * (e % (W / 4));
      v[p] = R{0, 0, 0, 0};
      if ((NV % NTH == 0 || e < NV) && i < n) v[p] = *reinterpret_cast<const R*>(base + (i * rs + c));
    }
  }
  __device__ __forceinline__ void put(float* dst, int ld = W + 4) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = threadIdx.x + p * NTH, i = e / (W / 4), c = 4 * (e % (W / 4));
      if (NV % NTH == 0 || e < NV) *reinterpret_cast<f32x4*>(dst + i * ld + c) = widen4(v[p]);
    }
  }
  // into a tile of the input type itself (no widening)
  __device__ __forceinline__ void put_raw(E* dst, int ld) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = threadIdx.x + p * NTH, i = e / (W / 4), c = 4 * (e % (W / 4));
      if (NV % NTH == 0 || e < NV) *reinterpret_cast<R*>(dst + i * ld + c) = v[p];
    }
  }
};

// LDS type and row stride of the raw q, k, v tiles: widened to fp32 as a rule; for
// bf16 inputs at D = 128 (and where a kernel asks for it, RAW) they stay bf16
// (exact, half the bytes), which lets the walks and delta_out own wider state
// slabs, or more workgroups share a CU. Row strides keep rows 16-byte aligned.
template <typename E, int D, bool RAW = (D > 64)> struct InTile {
  static constexpr bool raw = sizeof(E) == 2 && RAW;
  using T = typename std::conditional<raw, E, float>::type;
  static constexpr int LD = raw ? D + 8 : D + 4;
  static constexpr int TILE = CH * LD;
  // a RowTile into such a tile
  template <class RT> __device__ __forceinline__ static void put(const RT& t, T* dst) {
    if constexpr (raw) t.put_raw(dst, LD);
    else t.put(dst, LD);
  }
};

// columns c0 .. c0 + W - 1 of a row-major [D][D] fp32 matrix, put() as a [D][W + 4] tile
template <int D, int W = D> struct MatTile {
  static constexpr int NV = D * W / 4, PER = (NV + NTH - 1) / NTH;
  f32x4 v[PER];
  __device__ __forceinline__ void fetch(const float* src, int c0 = 0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = threadIdx.x + p * NTH, i = e / (W / 4), c = 4 * (e % (W / 4));
      if (NV % NTH == 0 || e < NV) v[p] = *reinterpret_cast<const f32x4*>(src + i * D + c0 + c);
    }
  }
  __device__ __forceinline__ void put(float* dst) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = threadIdx.x + p * NTH, i = e / (W / 4), c = 4 * (e % (W / 4));
      if (NV % NTH == 0 || e < NV) *reinterpret_cast<f32x4*>(dst + i * (W + 4) + c) = v[p];
    }
  }
};

// [64][D] rows t0 .. t0 + 63 of a [B,T,H,D] tensor into an fp32 LDS tile; rows
// past n read as zero.
template <typename E, int D>
__device__ __forceinline__ void load_rows(float* dst, const E* src, int64_t b, int64_t h, int64_t t0, int n,
                                          int64_t T, int64_t H) {
  RowTile<E, D> t;
  t.fetch(src, b, h, t0, n, T, H);
  t.put(dst);
}

// rows i < n of a [64][W + 4] fp32 LDS tile into columns c0 .. c0 + W - 1 of a
// [B,T,H,D] tensor of type E
template <typename E, int D, int W = D>
__device__ __forceinline__ void store_rows(E* dst, const float* src, int64_t b, int64_t h, int64_t t0, int n,
                                           int64_t T, int64_t H, int c0 = 0) {
  constexpr int PER_ROW = W / 4;
  for (int e = threadIdx.x; e < CH * PER_ROW; e += NTH) {
    const int i = e / PER_ROW, c = 4 * (e % PER_ROW);
    if (i >= n) continue;
    E* p = dst + row0(b, t0, h, T, H) * D + c0 + (i * ((int)H * D) + c);
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = (E)src[i * (W + 4) + c + u];
  }
}

// a [D][D] fp32 matrix between global (row-major) and an LDS tile
template <int D>
__device__ __forceinline__ void load_mat(float* dst, const float* src) {
  MatTile<D> t;
  t.fetch(src);
  t.put(dst);
}
// a [D][W + 4] LDS tile into columns c0 .. c0 + W - 1 of a row-major [D][D] matrix
template <int D, int W = D>
__device__ __forceinline__ void store_mat(float* dst, const float* src, int c0 = 0) {
  for (int e = threadIdx.x; e < D * W / 4; e += NTH) {
    const int i = e / (W / 4), c = 4 * (e % (W / 4));
    *reinterpret_cast<f32x4*>(dst + i * D + c0 + c) = *reinterpret_cast<const f32x4*>(src + i * (W + 4) + c);
  }
}

// Per-chunk token terms in LDS: Gam, beta, the sequence count cnt (starts at or
// before the token), eg = live e^Gam, el = tail e^{Gam_last - Gam}; sc[0] =
// live_last e^{Gam_last}. Wave 0 computes them (lane = token); ends with a barrier.
struct ChunkTerms {
  float gam[CH], beta[CH], eg[CH], el[CH];
  int cnt[CH];
  float sc[4];
};

// The per-token inputs of the terms (wave 0, lane = token), loaded by fetch() apart
// from the computation: the walks load the next chunk's with its tiles, and the
// per-chunk kernels issue them ahead of their tiles so that the terms need not wait
// for the tiles' loads.
struct TermRegs {
  float gv = 0.f, bv = 0.f;
  bool st = false;   // a sequence starts at the token
  __device__ __forceinline__ void fetch(const float* g, const float* beta, const int32_t* seq, int64_t b, int64_t h,
                                        int64_t t0, int n, int64_t T, int64_t H) {
    if (threadIdx.x < CH) {
      const int l = threadIdx.x;
      const bool ok = l < n;
      const int64_t t = t0 + l;
      const int64_t first = (b * T + t0) * H + h;   // the chunk's first token; tokens within it in 32 bits
      gv = ok ? g[first + l * (int)H] : 0.f;
      bv = ok ? beta[first + l * (int)H] : 0.f;
      st = false;
      if (seq && ok) st = seq[t] != (t > 0 ? seq[t - 1] : -1);
    }
  }
};

__device__ __forceinline__ void chunk_terms(ChunkTerms& s, const TermRegs& in) {
  if (threadIdx.x < CH) {
    const int l = threadIdx.x;
    const float gv = in.gv, bv = in.bv;
    const uint64_t starts = __ballot(in.st);
    const int cnt = __popcll(starts & ((2ull << l) - 1ull));
    // segment-local inclusive scan: add the partial of lane l - off when it is in
    // the same sequence (sequences are contiguous, so its partial is too)
    float x = gv;
#pragma unroll
    for (int off = 1; off < CH; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      const int cy = __shfl_up(cnt, off, 64);
      if (l >= off && cy == cnt) x += y;
    }
    const float last = __shfl(x, CH - 1, 64);
    const int clast = __shfl(cnt, CH - 1, 64);
    s.gam[l] = x;
    s.beta[l] = bv;
    s.cnt[l] = cnt;
    s.eg[l] = cnt == 0 ? __expf(x) : 0.f;
    s.el[l] = cnt == clast ? __expf(last - x) : 0.f;
    if (l == 0) s.sc[0] = clast == 0 ? __expf(last) : 0.f;
  }
  __syncthreads();
}

// the chunk's tokens inside shard r: (start, valid count)
__device__ __forceinline__ void chunk_of(int64_t T, int P, int64_t idx, int64_t& r, int64_t& c) {
  const int64_t nsc = chunks_of(shard_size(T, P));
  r = idx / nsc;
  c = idx % nsc;
}

// T = (I + A)^{-1} in place of a strictly lower-triangular [64][64] tile A (row
// stride CH + 4), by 16 x 16 blocks: the unit lower-triangular diagonal blocks by
// substitution, one lane of wave 0 per column (the column in registers), then the
// blocks below them block row by block row,
//   T_ij = -T_ii sum_{j <= k < i} A_ik T_kj,
// one 16 x 16 output tile per wave (an MFMA accumulator tile is laid out as the
// second operand of the next product, so -T_ii Y is formed from registers). Every
// thread of the workgroup calls it; it ends with a barrier.
__device__ __forceinline__ void unit_lower_inverse(float* s_a) {
  constexpr int LC = CH + 4;
  const int w = threadIdx.x >> 6, l = lane_id(), x = l & 15, kg = l >> 4;
  if (w == 0) {
    const int bi = kg, c = x;
    const float* ab = s_a + 16 * bi * LC + 16 * bi;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = r == c ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) v -= ab[r * LC + j] * t[j];
      t[r] = v;
    }
    asm volatile("" ::: "memory");   // the wave's reads of its blocks precede these writes
#pragma unroll
    for (int r = 0; r < 16; ++r) s_a[(16 * bi + r) * LC + 16 * bi + c] = t[r];
  }
  __syncthreads();
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const int j = w;
    if (j < i) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      for (int k = j; k < i; ++k)
        y = tile_mm<16>([&](int r, int q) { return s_a[(16 * i + r) * LC + 16 * k + q]; },
                        [&](int q, int cc) { return s_a[(16 * k + q) * LC + 16 * j + cc]; }, y);
#pragma unroll
      for (int st = 0; st < 4; ++st) z = mfma_f32(s_a[(16 * i + x) * LC + 16 * i + 4 * kg + st], y[st], z);
    }
    __syncthreads();   // block row i of A is read
    if (j < i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) s_a[(16 * i + 4 * kg + q) * LC + 16 * j + x] = -z[q];
    }
    __syncthreads();
  }
}

}  // namespace

// ---- U~ and W per chunk ------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(NTH) void delta_wy(DeltaArgs a) {
  using G = DGeo<D>;
  using IT = InTile<E, D, (D >= 64)>;
  __shared__ __attribute__((aligned(16))) typename IT::T s_k[IT::TILE], s_v[IT::TILE];
  __shared__ __attribute__((aligned(16))) float s_a[G::TILE_C];
  __shared__ ChunkTerms s_t;
  int64_t r, c;
  const int64_t idx = a.chunk_begin + blockIdx.x;
  chunk_of(a.T, a.P, idx, r, c);
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t slen = shard_len(a.T, a.P, r);
  const int n = (int)(slen - 64 * c < CH ? slen - 64 * c : CH);
  if (r >= a.P || n <= 0) return;
  const int64_t t0 = shard_begin(a.T, a.P, r) + 64 * c;
  const int32_t* seq = a.seq_idx ? a.seq_idx + b * a.T : nullptr;
  {
    RowTile<E, D> rk, rv;
    TermRegs tr;
    tr.fetch(a.g, a.beta, seq, b, h, t0, n, a.T, a.H);
    rk.fetch(reinterpret_cast<const E*>(a.k), b, h, t0, n, a.T, a.H);
    rv.fetch(reinterpret_cast<const E*>(a.v), b, h, t0, n, a.T, a.H);
    chunk_terms(s_t, tr);
    IT::put(rk, s_k);
    IT::put(rv, s_v);
  }
  __syncthreads();

  // A = strict-lower(beta_i D_ij k_i.k_j)
  const int w = threadIdx.x >> 6, l = lane_id();
  for (int t = w; t < 16; t += NWV) {
    const int ti = t >> 2, tj = t & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti)
      acc = tile_mm_e<D, E, true, true>([&](int i, int k) { return (float)s_k[(16 * ti + i) * IT::LD + k]; },
                    [&](int k, int j) { return (float)s_k[(16 * tj + j) * IT::LD + k]; }, acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
      const bool ok = j < i && s_t.cnt[i] == s_t.cnt[j];
      s_a[i * G::LC + j] = ok ? s_t.beta[i] * __expf(s_t.gam[i] - s_t.gam[j]) * acc[q] : 0.f;
    }
  }
  __syncthreads();

  // [U~ | W] = (I + A)^{-1} [beta V | beta live e^Gam K]: T = (I + A)^{-1} in place of
  // A, then the products T R by 16 x 16 tiles (T lower triangular: row tile ti
  // takes k tiles 0..ti), written straight to the workspace
  unit_lower_inverse(s_a);
  {
    constexpr int NCT = 2 * D / 16, NT_ = 4 * NCT;
    for (int t = w; t < NT_; t += NWV) {
      const int ti = t / NCT, tj = t % NCT;
      const bool isv = tj < NCT / 2;
      const typename IT::T* src = isv ? s_v : s_k;
      const int c0 = 16 * (isv ? tj : tj - NCT / 2);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kt = 0; kt <= ti; ++kt)
        acc = tile_mm<16>([&](int i, int q) { return s_a[(16 * ti + i) * G::LC + 16 * kt + q]; },
                          [&](int q, int j) {
                            const int k = 16 * kt + q;
                            return (float)src[k * IT::LD + c0 + j] * (isv ? s_t.beta[k] : s_t.beta[k] * s_t.eg[k]);
                          }, acc);
      float* dst = isv ? a.ws_ut : a.ws_w;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q;
        if (i < n) dst[row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + c0 + (l & 15))] = acc[q];
      }
    }
  }
}

// ---- forward chunk walk of one shard ------------------------------------------------------
// PREPARE: the augmented state Z = [delta_S | M] (D x 2D) from [0 | I], written to
// the shard's record as [M | delta_S]. APPLY: S from the composed incoming state;
// saves the state entering every chunk and U. The columns of Z evolve independently
// (the transition acts on the key side), so a workgroup may own a slab of SZ of
// them (blockIdx.z; at D = 128 the whole [delta_S | M] does not fit the LDS, at
// D = 64 two half-width apply walks share a CU).
template <typename E, int D, bool APPLY>
__global__ __launch_bounds__(NTH, (FwalkSlab<D, APPLY>::OCC)) void delta_fwalk(DeltaArgs a) {
  using G = DGeo<D>;
  constexpr int NZ = APPLY ? D : 2 * D;
  constexpr int SZ = FwalkSlab<D, APPLY>::SZ;
  constexpr int LZ = SZ + 4;
  using IT = InTile<E, D, (D > 64 || FwalkSlab<D, APPLY>::HALF)>;
  // the half-width bf16 apply walk (D = 64) also forms the output of its value
  // columns, O = live e^Gam Q S + P U (delta_out's work, the state and U being at
  // hand): Q and the score tile P fit beside the slab at two workgroups per CU
  constexpr bool FOLD = FwalkSlab<D, APPLY>::HALF && sizeof(E) == 2;
  __shared__ __attribute__((aligned(16))) float s_z[D * LZ], s_u[CH * LZ], s_w[G::TILE];
  __shared__ __attribute__((aligned(16))) typename IT::T s_k[IT::TILE], s_q[FOLD ? IT::TILE : 8];
  __shared__ __attribute__((aligned(16))) float s_p[FOLD ? G::TILE_C : 4];
  __shared__ ChunkTerms s_t;
  const int64_t r = a.rank_begin + blockIdx.x;
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int z0 = SZ == NZ ? 0 : SZ * blockIdx.z;                 // first column of Z owned here
  const bool takes_u = SZ == NZ || z0 < D;                        // the slab holds delta_S columns
  const int64_t tshard = shard_begin(a.T, a.P, r), slen = shard_len(a.T, a.P, r);
  const int nc = (int)chunks_of(slen);
  const int64_t cbase = shard_chunk_base(a.T, a.P, r), nct = row_chunks(a.T, a.P);
  const int32_t* seq = a.seq_idx ? a.seq_idx + b * a.T : nullptr;
  const int w = threadIdx.x >> 6, l = lane_id();

  for (int e = threadIdx.x; e < D * SZ; e += NTH) {
    const int d = e / SZ, m = e % SZ, mz = z0 + m;
    float x;
    if constexpr (APPLY) x = a.state_in[((r * a.B * a.H + bh) * D + d) * D + mz];
    else x = (mz == D + d) ? 1.f : 0.f;
    s_z[d * LZ + m] = x;
  }
  __syncthreads();   // an empty shard writes its record from s_z right away
  // each chunk's W, k and U~ are fetched into registers while the chunk before it
  // is being computed
  constexpr int UW = SZ < D ? SZ : D;            // U~ columns a slab takes
  RowTile<float, D> pw;
  RowTile<float, D, UW> pu;
  RowTile<E, D> pk, pq;
  TermRegs pt;
  auto fetch_chunk = [&](int c) {
    const int64_t t0 = tshard + 64 * c;
    const int n = (int)(slen - 64 * c < CH ? slen - 64 * c : CH);
    pt.fetch(a.g, a.beta, seq, b, h, t0, n, a.T, a.H);
    pw.fetch(a.ws_w, b, h, t0, n, a.T, a.H);
    pk.fetch(reinterpret_cast<const E*>(a.k), b, h, t0, n, a.T, a.H);
    if constexpr (FOLD) pq.fetch(reinterpret_cast<const E*>(a.q), b, h, t0, n, a.T, a.H);
    if (takes_u) pu.fetch(a.ws_ut, b, h, t0, n, a.T, a.H, z0);
  };
  if (nc > 0) fetch_chunk(0);
  for (int c = 0; c < nc; ++c) {
    const int64_t t0 = tshard + 64 * c;
    const int n = (int)(slen - 64 * c < CH ? slen - 64 * c : CH);
    pw.put(s_w);
    IT::put(pk, s_k);
    if constexpr (FOLD) IT::put(pq, s_q);
    // U~ into the slab's delta_S columns of s_u (the M part takes no input)
    if (takes_u) pu.put(s_u, LZ);
    if constexpr (SZ > UW || NZ > D) {
      const int zu = takes_u ? UW : 0;           // columns filled from U~
      for (int e = threadIdx.x; e < CH * (SZ - zu); e += NTH) s_u[(e / (SZ - zu)) * LZ + zu + e % (SZ - zu)] = 0.f;
    }
    chunk_terms(s_t, pt);
    if (c + 1 < nc) fetch_chunk(c + 1);
    if constexpr (APPLY) {
      float* cs = a.chunk_states + (bh * nct + cbase + c) * (int64_t)(D * D);
      for (int e = threadIdx.x; e < D * SZ; e += NTH) cs[(e / SZ) * D + z0 + e % SZ] = s_z[(e / SZ) * LZ + e % SZ];
    }
    // U_Z = U~_Z - W Z (and, folding the output, Q S for the same tiles and the
    // score tile P, both taken before Z is updated)
    constexpr int NUT = 4 * (SZ / 16), PUT = (NUT + NWV - 1) / NWV;
    f32x4 xo[FOLD ? PUT : 1];
    if constexpr (!FOLD) {
      for (int t = w; t < NUT; t += NWV) {
        const int ti = t / (SZ / 16), tj = t % (SZ / 16);
        f32x4 acc = tile_mm_e<D, E>([&](int i, int k) { return s_w[(16 * ti + i) * G::LD + k]; },
                            [&](int k, int j) { return s_z[k * LZ + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
          s_u[i * LZ + j] -= acc[q];
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < PUT; ++m) {
        const int t = w + NWV * m;
        if (t >= NUT) continue;
        const int ti = t / (SZ / 16), tj = t % (SZ / 16);
        f32x4 acc = tile_mm_e<D, E>([&](int i, int k) { return s_w[(16 * ti + i) * G::LD + k]; },
                            [&](int k, int j) { return s_z[k * LZ + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
          s_u[i * LZ + j] -= acc[q];
        }
        xo[m] = tile_mm_e<D, E, true, false>([&](int i, int k) { return (float)s_q[(16 * ti + i) * IT::LD + k]; },
                                             [&](int k, int j) { return s_z[k * LZ + 16 * tj + j]; },
                                             f32x4{0.f, 0.f, 0.f, 0.f});
      }
      for (int t = w; t < 16; t += NWV) {
        const int ti = t >> 2, tj = t & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (tj <= ti)
          acc = tile_mm_e<D, E, true, true>([&](int i, int k) { return (float)s_q[(16 * ti + i) * IT::LD + k]; },
                                            [&](int k, int j) { return (float)s_k[(16 * tj + j) * IT::LD + k]; }, acc);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
          const bool ok = j <= i && s_t.cnt[i] == s_t.cnt[j];
          s_p[i * G::LC + j] = ok ? __expf(s_t.gam[i] - s_t.gam[j]) * acc[q] : 0.f;
        }
      }
    }
    __syncthreads();
    if constexpr (FOLD) {
      // O = live e^Gam Q S + P U for the slab's value columns
      E* o = reinterpret_cast<E*>(a.out);
#pragma unroll
      for (int m = 0; m < PUT; ++m) {
        const int t = w + NWV * m;
        if (t >= NUT) continue;
        const int ti = t / (SZ / 16), tj = t % (SZ / 16);
        const f32x4 y = tile_mm_e<CH, E>([&](int i, int k) { return s_p[(16 * ti + i) * G::LC + k]; },
                                         [&](int k, int j) { return s_u[k * LZ + 16 * tj + j]; },
                                         f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 16 * ti + 4 * (l >> 4) + q;
          if (i < n)
            o[row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + z0 + 16 * tj + (l & 15))] =
                (E)(s_t.eg[i] * xo[m][q] + y[q]);
        }
      }
    }
    if constexpr (APPLY) {
      for (int e = threadIdx.x; e < CH * SZ; e += NTH) {
        const int i = e / SZ, m = e % SZ;
        if (i < n) a.ws_u[row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + z0 + m)] = s_u[i * LZ + m];
      }
    }
    // Z <- live_last e^Gam_last Z + K~^T U_Z
    const float sc = s_t.sc[0];
    for (int t = w; t < (D / 16) * (SZ / 16); t += NWV) {
      const int ti = t / (SZ / 16), tj = t % (SZ / 16);
      f32x4 acc = tile_mm_e<CH, E>([&](int i, int k) { return (float)s_k[k * IT::LD + 16 * ti + i] * s_t.el[k]; },
                          [&](int k, int j) { return s_u[k * LZ + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 16 * ti + 4 * (l >> 4) + q, m = 16 * tj + (l & 15);
        s_z[d * LZ + m] = sc * s_z[d * LZ + m] + acc[q];
      }
    }
    __syncthreads();
  }
  if constexpr (!APPLY) {
    // record [M | delta_S]: Z column mz < D is delta_S column mz, else M column mz - D
    float* rec = a.summary + (r * a.B * a.H + bh) * (int64_t)(2 * D * D);
    for (int e = threadIdx.x; e < D * SZ; e += NTH) {
      const int d = e / SZ, m = e % SZ, mz = z0 + m;
      const int64_t off = mz < D ? (int64_t)D * D + d * D + mz : d * D + (mz - D);
      rec[off] = s_z[d * LZ + m];
    }
  }
}

// ---- composition over shards ----------------------------------------------------------
// forward: out[r] = fold of S <- M_j S + delta_S_j over [prs_r, r) (S_init at rank 0
// unpacked); reverse: out[r] = fold of dS <- M_j^T dS + gamma_j over (r, frs_r)
// backwards (dS_final at the last rank unpacked). A shard holding a start has
// M = 0, so folding through it restarts the fold. The running value after the
// last shard is the final state / dS_init. The columns of S fold independently: a
// workgroup owns SC of them (blockIdx.y) and fetches the next shard's M while it
// folds the current one.
template <int D>
__global__ __launch_bounds__(NTH) void delta_scan(DeltaScanArgs a) {
  using G = DGeo<D>;
  constexpr int SC = DeltaSlabs<D>::SCAN, LC = SC + 4;
  __shared__ __attribute__((aligned(16))) float s_s[D * LC], s_m[D * G::LD];
  const int64_t bh = blockIdx.x;
  const int c0 = SC == D ? 0 : SC * blockIdx.y;
  const int w = threadIdx.x >> 6, l = lane_id();
  const int32_t* slice = a.slice ? a.slice + (bh / a.H) * a.P : nullptr;
  constexpr int64_t REC = 2 * D * D;
  for (int e = threadIdx.x; e < D * SC; e += NTH)
    s_s[(e / SC) * LC + e % SC] = a.init ? a.init[bh * D * D + (e / SC) * D + c0 + e % SC] : 0.f;
  MatTile<D> pm;
  auto rec_of = [&](int s) { return a.summary + ((a.reverse ? a.P - 1 - s : s) * a.BH + bh) * REC; };
  pm.fetch(rec_of(0));
  __syncthreads();
  for (int s = 0; s < a.P; ++s) {
    const int q = a.reverse ? a.P - 1 - s : s;
    if (s > 0 && slice && slice[q] == (a.reverse ? q + 1 : q)) {
      for (int e = threadIdx.x; e < D * SC; e += NTH) s_s[(e / SC) * LC + e % SC] = 0.f;
      __syncthreads();
    }
    store_mat<D, SC>(a.out + (q * a.BH + bh) * (int64_t)(D * D), s_s, c0);
    const float* rec = rec_of(s);
    pm.put(s_m);
    __syncthreads();
    if (s + 1 < a.P) pm.fetch(rec_of(s + 1));
    constexpr int NT2 = (D / 16) * (SC / 16), PW = (NT2 + NWV - 1) / NWV;
    f32x4 res[PW];
#pragma unroll
    for (int m = 0; m < PW; ++m) {
      const int t = w + NWV * m;
      if (t >= NT2) continue;
      const int ti = t / (SC / 16), tj = t % (SC / 16);
      f32x4 acc = a.reverse
          ? tile_mm<D>([&](int i, int k) { return s_m[k * G::LD + 16 * ti + i]; },
                    [&](int k, int j) { return s_s[k * LC + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f})
          : tile_mm<D>([&](int i, int k) { return s_m[(16 * ti + i) * G::LD + k]; },
                    [&](int k, int j) { return s_s[k * LC + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 16 * ti + 4 * (l >> 4) + u, j = c0 + 16 * tj + (l & 15);
        acc[u] += rec[D * D + i * D + j];
      }
      res[m] = acc;
    }
    __syncthreads();   // every read of s_s and s_m is done
#pragma unroll
    for (int m = 0; m < PW; ++m) {
      const int t = w + NWV * m;
      if (t >= NT2) continue;
      const int ti = t / (SC / 16), tj = t % (SC / 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) s_s[(16 * ti + 4 * (l >> 4) + u) * LC + 16 * tj + (l & 15)] = res[m][u];
    }
    __syncthreads();
  }
  if (a.fin) store_mat<D, SC>(a.fin + bh * (int64_t)(D * D), s_s, c0);
}

// ---- output per chunk --------------------------------------------------------------------
// O = live e^Gam Q S + P U, P = tril(Q K^T) . D; a workgroup computes the value
// columns v0 .. v0 + SV - 1 (blockIdx.z) of one chunk.
template <typename E, int D>
__global__ __launch_bounds__(NTH) void delta_out(DeltaArgs a) {
  using G = DGeo<D>;
  constexpr int SV = DeltaSlabs<D>::OUT, LV = SV + 4;
  using IT = InTile<E, D, (D >= 64)>;
  __shared__ __attribute__((aligned(16))) typename IT::T s_q[IT::TILE], s_k[IT::TILE];
  __shared__ __attribute__((aligned(16))) float s_u[CH * LV], s_s[D * LV], s_p[G::TILE_C];
  __shared__ ChunkTerms s_t;
  int64_t r, c;
  const int64_t idx = a.chunk_begin + blockIdx.x;
  chunk_of(a.T, a.P, idx, r, c);
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int v0 = SV == D ? 0 : SV * blockIdx.z;
  const int64_t slen = shard_len(a.T, a.P, r);
  const int n = (int)(slen - 64 * c < CH ? slen - 64 * c : CH);
  if (r >= a.P || n <= 0) return;
  const int64_t t0 = shard_begin(a.T, a.P, r) + 64 * c;
  const int64_t nct = row_chunks(a.T, a.P);
  const int32_t* seq = a.seq_idx ? a.seq_idx + b * a.T : nullptr;
  const int w = threadIdx.x >> 6, l = lane_id();
  {
    RowTile<E, D> rq, rk;
    RowTile<float, D, SV> ru;
    MatTile<D, SV> rs;
    TermRegs tr;
    tr.fetch(a.g, a.beta, seq, b, h, t0, n, a.T, a.H);
    rq.fetch(reinterpret_cast<const E*>(a.q), b, h, t0, n, a.T, a.H);
    rk.fetch(reinterpret_cast<const E*>(a.k), b, h, t0, n, a.T, a.H);
    ru.fetch(a.ws_u, b, h, t0, n, a.T, a.H, v0);
    rs.fetch(a.chunk_states + (bh * nct + idx) * (int64_t)(D * D), v0);
    chunk_terms(s_t, tr);
    IT::put(rq, s_q);
    IT::put(rk, s_k);
    ru.put(s_u);
    rs.put(s_s);
  }
  __syncthreads();
  for (int t = w; t < 16; t += NWV) {
    const int ti = t >> 2, tj = t & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti)
      acc = tile_mm_e<D, E, true, true>([&](int i, int k) { return (float)s_q[(16 * ti + i) * IT::LD + k]; },
                    [&](int k, int j) { return (float)s_k[(16 * tj + j) * IT::LD + k]; }, acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
      const bool ok = j <= i && s_t.cnt[i] == s_t.cnt[j];
      s_p[i * G::LC + j] = ok ? __expf(s_t.gam[i] - s_t.gam[j]) * acc[q] : 0.f;
    }
  }
  __syncthreads();
  E* o = reinterpret_cast<E*>(a.out);
  for (int t = w; t < 4 * (SV / 16); t += NWV) {
    const int ti = t / (SV / 16), tj = t % (SV / 16);
    f32x4 x = tile_mm_e<D, E, true, false>([&](int i, int k) { return (float)s_q[(16 * ti + i) * IT::LD + k]; },
                      [&](int k, int j) { return s_s[k * LV + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
    f32x4 y = tile_mm_e<CH, E>([&](int i, int k) { return s_p[(16 * ti + i) * G::LC + k]; },
                      [&](int k, int j) { return s_u[k * LV + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 16 * ti + 4 * (l >> 4) + q, j = v0 + 16 * tj + (l & 15);
      if (i < n) o[row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + j)] = (E)(s_t.eg[i] * x[q] + y[q]);
    }
  }
}

// ---- reverse chunk walk of one shard ------------------------------------------------------
// dU = P^T dO + K~ dS, dS <- live_last e^Gam_last dS + (live e^Gam Q)^T dO - W^T dU,
// from dS = 0 (PREPARE: gamma, written with a copy of the shard's M) or from the
// composed gradient (APPLY: saves the gradient at every chunk's end and dU). The
// value columns of dS and dU evolve independently: a workgroup owns SV of them
// (blockIdx.z).
template <typename E, int D, bool APPLY>
__global__ __launch_bounds__(NTH, DeltaSlabs<D>::BWALK_OCC) void delta_bwalk(DeltaArgs a) {
  using G = DGeo<D>;
  constexpr int SV = DeltaSlabs<D>::BWALK, LV = SV + 4;
  // D = 64: 32-column slabs with bf16 q, k and dU in the score tile's space (P is
  // dead once dU is formed): 73 KB, two workgroups per CU
  constexpr bool DU_IN_P = D == 64;
  static_assert(!DU_IN_P || CH * LV <= G::TILE_C, "dU fits the score tile");
  using IT = InTile<E, D, (D >= 64)>;
  __shared__ __attribute__((aligned(16))) typename IT::T s_q[IT::TILE], s_k[IT::TILE];
  __shared__ __attribute__((aligned(16))) float s_do[CH * LV], s_w[G::TILE], s_du_own[DU_IN_P ? 4 : CH * LV],
      s_ds[D * LV], s_p[G::TILE_C];
  float* const s_du = DU_IN_P ? s_p : s_du_own;
  __shared__ ChunkTerms s_t;
  const int64_t r = a.rank_begin + blockIdx.x;
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int v0 = SV == D ? 0 : SV * blockIdx.z;
  const int64_t tshard = shard_begin(a.T, a.P, r), slen = shard_len(a.T, a.P, r);
  const int nc = (int)chunks_of(slen);
  const int64_t cbase = shard_chunk_base(a.T, a.P, r), nct = row_chunks(a.T, a.P);
  const int32_t* seq = a.seq_idx ? a.seq_idx + b * a.T : nullptr;
  const int w = threadIdx.x >> 6, l = lane_id();
  for (int e = threadIdx.x; e < D * SV; e += NTH)
    s_ds[(e / SV) * LV + e % SV] =
        APPLY ? a.state_in[(r * a.B * a.H + bh) * (int64_t)(D * D) + (e / SV) * D + v0 + e % SV] : 0.f;
  __syncthreads();   // an empty shard writes its record from s_ds right away
  // each chunk's q, k, dO and W are fetched into registers while the chunk after
  // it (the walk runs backwards) is being computed
  RowTile<E, D> pq, pk;
  RowTile<E, D, SV> pdo;
  RowTile<float, D> pw;
  TermRegs pt;
  auto fetch_chunk = [&](int c) {
    const int64_t t0 = tshard + 64 * c;
    const int n = (int)(slen - 64 * c < CH ? slen - 64 * c : CH);
    pt.fetch(a.g, a.beta, seq, b, h, t0, n, a.T, a.H);
    pq.fetch(reinterpret_cast<const E*>(a.q), b, h, t0, n, a.T, a.H);
    pk.fetch(reinterpret_cast<const E*>(a.k), b, h, t0, n, a.T, a.H);
    pdo.fetch(reinterpret_cast<const E*>(a.dO), b, h, t0, n, a.T, a.H, v0);
    pw.fetch(a.ws_w, b, h, t0, n, a.T, a.H);
  };
  if (nc > 0) fetch_chunk(nc - 1);
  for (int c = nc - 1; c >= 0; --c) {
    const int64_t t0 = tshard + 64 * c;
    const int n = (int)(slen - 64 * c < CH ? slen - 64 * c : CH);
    IT::put(pq, s_q);
    IT::put(pk, s_k);
    pdo.put(s_do);
    pw.put(s_w);
    chunk_terms(s_t, pt);
    if (c > 0) fetch_chunk(c - 1);
    if constexpr (APPLY) store_mat<D, SV>(a.ws_dsc + (bh * nct + cbase + c) * (int64_t)(D * D), s_ds, v0);
    for (int t = w; t < 16; t += NWV) {
      const int ti = t >> 2, tj = t & 3;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (tj <= ti)
        acc = tile_mm_e<D, E, true, true>([&](int i, int k) { return (float)s_q[(16 * ti + i) * IT::LD + k]; },
                      [&](int k, int j) { return (float)s_k[(16 * tj + j) * IT::LD + k]; }, acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        const bool ok = j <= i && s_t.cnt[i] == s_t.cnt[j];
        s_p[i * G::LC + j] = ok ? __expf(s_t.gam[i] - s_t.gam[j]) * acc[q] : 0.f;
      }
    }
    __syncthreads();
    // dU = P^T dO + K~ dS; at D = 128 the row factor of K~ = el K is applied to the
    // product instead (k stays exact). Where dU takes the score tile's space, every
    // wave's tiles are held until all have read P.
    constexpr int NDU = 4 * (SV / 16), PDU = (NDU + NWV - 1) / NWV;
    f32x4 du_res[PDU];
#pragma unroll
    for (int m = 0; m < PDU; ++m) {
      const int t = w + NWV * m;
      if (t >= NDU) continue;
      const int ti = t / (SV / 16), tj = t % (SV / 16);
      f32x4 acc = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_p[k * G::LC + 16 * ti + i]; },
                          [&](int k, int j) { return s_do[k * LV + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
      if constexpr (D > 64) {
        const f32x4 y = tile_mm_e<D, E, true, false>([&](int i, int k) { return (float)s_k[(16 * ti + i) * IT::LD + k]; },
                      [&](int k, int j) { return s_ds[k * LV + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += s_t.el[16 * ti + 4 * (l >> 4) + q] * y[q];
      } else {
        acc = tile_mm_e<D, E>([&](int i, int k) { return (float)s_k[(16 * ti + i) * IT::LD + k] * s_t.el[16 * ti + i]; },
                      [&](int k, int j) { return s_ds[k * LV + 16 * tj + j]; }, acc);
      }
      du_res[m] = acc;
      if constexpr (!DU_IN_P) {
#pragma unroll
        for (int q = 0; q < 4; ++q) s_du[(16 * ti + 4 * (l >> 4) + q) * LV + 16 * tj + (l & 15)] = acc[q];
      }
    }
    if constexpr (DU_IN_P) {
      __syncthreads();   // every read of P is done
#pragma unroll
      for (int m = 0; m < PDU; ++m) {
        const int t = w + NWV * m;
        if (t >= NDU) continue;
        const int ti = t / (SV / 16), tj = t % (SV / 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) s_du[(16 * ti + 4 * (l >> 4) + q) * LV + 16 * tj + (l & 15)] = du_res[m][q];
      }
    }
    __syncthreads();
    if constexpr (APPLY) store_rows<float, D, SV>(a.ws_du, s_du, b, h, t0, n, a.T, a.H, v0);
    // dS <- sc dS + (eg Q)^T dO - W^T dU
    const float sc = s_t.sc[0];
    for (int t = w; t < G::NTC * (SV / 16); t += NWV) {
      const int ti = t / (SV / 16), tj = t % (SV / 16);
      f32x4 x = tile_mm_e<CH, E, false, true>([&](int i, int k) { return (float)s_q[k * IT::LD + 16 * ti + i] * s_t.eg[k]; },
                        [&](int k, int j) { return s_do[k * LV + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 y = tile_mm_e<CH, E>([&](int i, int k) { return s_w[k * G::LD + 16 * ti + i]; },
                        [&](int k, int j) { return s_du[k * LV + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 16 * ti + 4 * (l >> 4) + q, m = 16 * tj + (l & 15);
        s_ds[d * LV + m] = sc * s_ds[d * LV + m] + x[q] - y[q];
      }
    }
    __syncthreads();
  }
  if constexpr (!APPLY) {
    // record [M | gamma]: M copied from the forward record by the first slab
    float* rec = a.summary + (r * a.B * a.H + bh) * (int64_t)(2 * D * D);
    const float* frec = a.fwd_summary + (r * a.B * a.H + bh) * (int64_t)(2 * D * D);
    if (blockIdx.z == 0)
      for (int e = threadIdx.x; e < D * D; e += NTH) rec[e] = frec[e];
    for (int e = threadIdx.x; e < D * SV; e += NTH)
      rec[D * D + (e / SV) * D + v0 + e % SV] = s_ds[(e / SV) * LV + e % SV];
  }
}

// ---- gradients per chunk --------------------------------------------------------------------
// From S0 (state entering the chunk), dS (gradient at its end), U, dU, U~, W:
//   dPr = (dO U^T) . D (causal, one sequence), dq = dPr K + eg (dO S0^T),
//   dk  = dPr^T Q + el (U dS^T) + dAr K + dAr^T K + beta eg dBk,
//   [dBv | dBk] = (I + A)^{-T} [dU | -dU S0^T],  dA = strict-lower(-(dBv U~^T + dBk W^T)),
//   dAr = dA . D . beta_i,  dv = beta dBv,
//   dbeta = rowsum(dA . D . KK^T) + rowsum(dBv . V) + eg rowsum(dBk . K),
//   dGam = (row - column sums of dPr . QK^T and of dA . A) + eg rowsum(Q . dO S0^T)
//          + beta eg rowsum(dBk . K) - tk + [last] (sum tk + sc <dS, S0>),
//   tk_j = el_j rowsum(U dS^T . K)_j,  dg = suffix sums of dGam within each sequence.
template <typename E, int D>
__global__ __launch_bounds__(NTH) void delta_grad(DeltaArgs a) {
  using G = DGeo<D>;
  // eight [64][64+4] slots (a [64][D] or [D][D] tile fits one)
  __shared__ __attribute__((aligned(16))) float s_slot[8][G::TILE_C];
  __shared__ ChunkTerms s_t;
  __shared__ float s_rp[3][NWV][CH];   // per-wave row partials
  __shared__ float s_colp[NWV][CH];    // per-wave column partials
  __shared__ float s_cp[2][CH];        // column sums
  __shared__ float s_red[NWV];
  int64_t r, c;
  const int64_t idx = a.chunk_begin + blockIdx.x;
  chunk_of(a.T, a.P, idx, r, c);
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t slen = shard_len(a.T, a.P, r);
  const int n = (int)(slen - 64 * c < CH ? slen - 64 * c : CH);
  if (r >= a.P || n <= 0) return;
  const int64_t t0 = shard_begin(a.T, a.P, r) + 64 * c;
  const int64_t nct = row_chunks(a.T, a.P);
  const int32_t* seq = a.seq_idx ? a.seq_idx + b * a.T : nullptr;
  const int w = threadIdx.x >> 6, l = lane_id();
  float *s_q = s_slot[0], *s_k = s_slot[1], *s_do = s_slot[2], *s_u = s_slot[3], *s_s0 = s_slot[4],
        *s_ds = s_slot[5], *s_dp = s_slot[6], *s_dk = s_slot[7];
  {
    RowTile<E, D> rq, rk, rdo;
    RowTile<float, D> ru;
    MatTile<D> rs0, rds;
    TermRegs tr;
    tr.fetch(a.g, a.beta, seq, b, h, t0, n, a.T, a.H);
    rq.fetch(reinterpret_cast<const E*>(a.q), b, h, t0, n, a.T, a.H);
    rk.fetch(reinterpret_cast<const E*>(a.k), b, h, t0, n, a.T, a.H);
    rdo.fetch(reinterpret_cast<const E*>(a.dO), b, h, t0, n, a.T, a.H);
    ru.fetch(a.ws_u, b, h, t0, n, a.T, a.H);
    rs0.fetch(a.chunk_states + (bh * nct + idx) * (int64_t)(D * D));
    rds.fetch(a.ws_dsc + (bh * nct + idx) * (int64_t)(D * D));
    for (int e = threadIdx.x; e < 3 * NWV * CH; e += NTH) (&s_rp[0][0][0])[e] = 0.f;
    for (int e = threadIdx.x; e < NWV * CH; e += NTH) (&s_colp[0][0])[e] = 0.f;
    chunk_terms(s_t, tr);
    rq.put(s_q);
    rk.put(s_k);
    rdo.put(s_do);
    ru.put(s_u);
    rs0.put(s_s0);
    rds.put(s_ds);
  }
  __syncthreads();

  // score tiles: dPr and the decay terms of dGam (rows of wave w's column tile tj = w)
  {
    float colacc = 0.f;
    for (int t = w; t < 16; t += NWV) {
      const int ti = t >> 2, tj = t & 3;
      f32x4 qk = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
      if (tj <= ti) {
        qk = tile_mm_e<D, E, true, true>([&](int i, int k) { return s_q[(16 * ti + i) * G::LD + k]; },
                     [&](int k, int j) { return s_k[(16 * tj + j) * G::LD + k]; }, qk);
        du = tile_mm_e<D, E, true, false>([&](int i, int k) { return s_do[(16 * ti + i) * G::LD + k]; },
                     [&](int k, int j) { return s_u[(16 * tj + j) * G::LD + k]; }, du);
      }
      float rowp[4], colp = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        const bool ok = j <= i && s_t.cnt[i] == s_t.cnt[j];
        const float dpr = ok ? __expf(s_t.gam[i] - s_t.gam[j]) * du[q] : 0.f;
        s_dp[i * G::LC + j] = dpr;
        const float pa = dpr * qk[q];
        rowp[q] = pa;
        colp += pa;
      }
      // rows: sum over the 16 columns of the tile (lanes sharing l / 16)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x = rowp[q];
        x += __shfl_xor(x, 1, 64);
        x += __shfl_xor(x, 2, 64);
        x += __shfl_xor(x, 4, 64);
        x += __shfl_xor(x, 8, 64);
        if ((l & 15) == 0) s_rp[0][w][16 * ti + 4 * (l >> 4) + q] = x;
      }
      colp += __shfl_xor(colp, 16, 64);
      colp += __shfl_xor(colp, 32, 64);
      colacc += colp;
    }
    if (l < 16) s_colp[w][16 * (w & 3) + l] = colacc;   // the wave's column tile, over its row tiles
  }
  __syncthreads();
  if (threadIdx.x < CH) {
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) x += s_colp[ww][threadIdx.x];
    s_cp[0][threadIdx.x] = x;
  }

  // dq = dPr K + eg (dO S0^T); dk (part) = dPr^T Q + el (U dS^T); row partials of
  // Q . (dO S0^T) and el (U dS^T) . K
  {
    E* dq = reinterpret_cast<E*>(a.dq);
    for (int t = w; t < 4 * G::NTC; t += NWV) {
      const int ti = t / G::NTC, tj = t % G::NTC;
      f32x4 x = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_dp[(16 * ti + i) * G::LC + k]; },
                        [&](int k, int j) { return s_k[k * G::LD + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 y = tile_mm_e<D, E, true, false>([&](int i, int k) { return s_do[(16 * ti + i) * G::LD + k]; },
                        [&](int k, int j) { return s_s0[(16 * tj + j) * G::LD + k]; }, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 z = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_dp[k * G::LC + 16 * ti + i]; },
                        [&](int k, int j) { return s_q[k * G::LD + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 u = tile_mm_e<D, E>([&](int i, int k) { return s_u[(16 * ti + i) * G::LD + k]; },
                        [&](int k, int j) { return s_ds[(16 * tj + j) * G::LD + k]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        const float eg = s_t.eg[i], el = s_t.el[i];
        if (i < n) dq[row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + j)] = (E)(x[q] + eg * y[q]);
        const float ue = el * u[q];
        s_dk[i * G::LD + j] = z[q] + ue;
        float p1 = eg * y[q] * s_q[i * G::LD + j];
        float p2 = ue * s_k[i * G::LD + j];
        p1 += __shfl_xor(p1, 1, 64);
        p1 += __shfl_xor(p1, 2, 64);
        p1 += __shfl_xor(p1, 4, 64);
        p1 += __shfl_xor(p1, 8, 64);
        p2 += __shfl_xor(p2, 1, 64);
        p2 += __shfl_xor(p2, 2, 64);
        p2 += __shfl_xor(p2, 4, 64);
        p2 += __shfl_xor(p2, 8, 64);
        if ((l & 15) == 0) {
          s_rp[1][w][i] += p1;   // a wave may own several column tiles of one row
          s_rp[2][w][i] += p2;
        }
      }
    }
    // <dS, S0>
    float sp = 0.f;
    for (int e = threadIdx.x; e < D * D; e += NTH) sp += s_ds[(e / D) * G::LD + e % D] * s_s0[(e / D) * G::LD + e % D];
    sp = wave_sum(sp);
    if (l == 0) s_red[w] = sp;
  }
  __syncthreads();
  // dGam (partial) into s_cp[1]
  if (threadIdx.x < CH) {
    const int i = threadIdx.x;
    float rowpa = 0.f, qdos = 0.f, tk = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) {
      rowpa += s_rp[0][ww][i];
      qdos += s_rp[1][ww][i];
      tk += s_rp[2][ww][i];
    }
    float dgam = rowpa - s_cp[0][i] + qdos - tk;
    float tks = tk;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tks += __shfl_xor(tks, off, 64);
    if (i == CH - 1) {
      float sp = 0.f;
#pragma unroll
      for (int ww = 0; ww < NWV; ++ww) sp += s_red[ww];
      dgam += tks + s_t.sc[0] * sp;
    }
    s_cp[1][i] = dgam;
  }
  __syncthreads();

  // phase 2: slots 0 V, 2 U~, 3 W, 6 dU; 1 K, 4 S0, 7 dk kept; 5 dW
  float *s_v = s_slot[0], *s_ut = s_slot[2], *s_w = s_slot[3], *s_dU = s_slot[6], *s_dW = s_slot[5];
  {
    RowTile<E, D> rv;
    RowTile<float, D> rut, rw, rdu;
    rv.fetch(reinterpret_cast<const E*>(a.v), b, h, t0, n, a.T, a.H);
    rut.fetch(a.ws_ut, b, h, t0, n, a.T, a.H);
    rw.fetch(a.ws_w, b, h, t0, n, a.T, a.H);
    rdu.fetch(a.ws_du, b, h, t0, n, a.T, a.H);
    rv.put(s_v);
    rut.put(s_ut);
    rw.put(s_w);
    rdu.put(s_dU);
  }
  __syncthreads();
  // dW = -dU S0^T
  for (int t = w; t < 4 * G::NTC; t += NWV) {
    const int ti = t / G::NTC, tj = t % G::NTC;
    f32x4 x = tile_mm_e<D, E>([&](int i, int k) { return s_dU[(16 * ti + i) * G::LD + k]; },
                      [&](int k, int j) { return s_s0[(16 * tj + j) * G::LD + k]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int q = 0; q < 4; ++q) s_dW[(16 * ti + 4 * (l >> 4) + q) * G::LD + 16 * tj + (l & 15)] = -x[q];
  }
  __syncthreads();
  // A into slot 4 (S0 is dead)
  float* s_a = s_slot[4];
  for (int t = w; t < 16; t += NWV) {
    const int ti = t >> 2, tj = t & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti)
      acc = tile_mm_e<D, E, true, true>([&](int i, int k) { return s_k[(16 * ti + i) * G::LD + k]; },
                    [&](int k, int j) { return s_k[(16 * tj + j) * G::LD + k]; }, acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
      const bool ok = j < i && s_t.cnt[i] == s_t.cnt[j];
      s_a[i * G::LC + j] = ok ? s_t.beta[i] * __expf(s_t.gam[i] - s_t.gam[j]) * acc[q] : 0.f;
    }
  }
  __syncthreads();
  // [dBv | dBk] = (I + A)^{-T} [dU | dW] in place: T = (I + A)^{-1} in place of A (dead
  // after this), then T^T R by 16 x 16 tiles (row tile ti takes k tiles ti..3),
  // held in registers until every wave has read R
  unit_lower_inverse(s_a);
  {
    constexpr int NCT = 2 * D / 16, NT_ = 4 * NCT, PW = (NT_ + NWV - 1) / NWV;
    f32x4 res[PW];
#pragma unroll
    for (int m = 0; m < PW; ++m) {
      const int t = w + NWV * m;
      if (t >= NT_) continue;
      const int ti = t / NCT, tj = t % NCT;
      const bool isv = tj < NCT / 2;
      const float* src = isv ? s_dU : s_dW;
      const int c0 = 16 * (isv ? tj : tj - NCT / 2);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kt = ti; kt < 4; ++kt)
        acc = tile_mm<16>([&](int i, int q) { return s_a[(16 * kt + q) * G::LC + 16 * ti + i]; },
                          [&](int q, int j) { return src[(16 * kt + q) * G::LD + c0 + j]; }, acc);
      res[m] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < PW; ++m) {
      const int t = w + NWV * m;
      if (t >= NT_) continue;
      const int ti = t / NCT, tj = t % NCT;
      const bool isv = tj < NCT / 2;
      float* dst = isv ? s_dU : s_dW;
      const int c0 = 16 * (isv ? tj : tj - NCT / 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[(16 * ti + 4 * (l >> 4) + q) * G::LD + c0 + (l & 15)] = res[m][q];
    }
  }
  __syncthreads();
  // dA = strict-lower(-(dBv U~^T + dBk W^T)); dAr = dA . D . beta_i into slot 4;
  // row sums of dA . D . KK^T (dbeta) and column sums of dA . A (dGam)
  for (int e = threadIdx.x; e < 2 * NWV * CH; e += NTH) (&s_rp[0][0][0])[e] = 0.f;
  for (int e = threadIdx.x; e < NWV * CH; e += NTH) (&s_colp[0][0])[e] = 0.f;
  __syncthreads();
  {
    float colacc = 0.f;
    for (int t = w; t < 16; t += NWV) {
      const int ti = t >> 2, tj = t & 3;
      f32x4 x = {0.f, 0.f, 0.f, 0.f}, kk = {0.f, 0.f, 0.f, 0.f};
      if (tj <= ti) {
        x = tile_mm_e<D, E>([&](int i, int k) { return s_dU[(16 * ti + i) * G::LD + k]; },
                    [&](int k, int j) { return s_ut[(16 * tj + j) * G::LD + k]; }, x);
        x = tile_mm_e<D, E>([&](int i, int k) { return s_dW[(16 * ti + i) * G::LD + k]; },
                    [&](int k, int j) { return s_w[(16 * tj + j) * G::LD + k]; }, x);
        kk = tile_mm_e<D, E, true, true>([&](int i, int k) { return s_k[(16 * ti + i) * G::LD + k]; },
                     [&](int k, int j) { return s_k[(16 * tj + j) * G::LD + k]; }, kk);
      }
      float colp = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        const bool ok = j < i && s_t.cnt[i] == s_t.cnt[j];
        const float dec = ok ? __expf(s_t.gam[i] - s_t.gam[j]) : 0.f;
        const float da = ok ? -x[q] : 0.f;
        const float r1 = da * dec * kk[q];          // dA . D . KK^T
        s_a[i * G::LC + j] = da * dec * s_t.beta[i];
        colp += r1 * s_t.beta[i];                   // column sums of dA . A
        float x1 = r1;
        x1 += __shfl_xor(x1, 1, 64);
        x1 += __shfl_xor(x1, 2, 64);
        x1 += __shfl_xor(x1, 4, 64);
        x1 += __shfl_xor(x1, 8, 64);
        if ((l & 15) == 0) s_rp[0][w][i] = x1;
      }
      colp += __shfl_xor(colp, 16, 64);
      colp += __shfl_xor(colp, 32, 64);
      colacc += colp;
    }
    if (l < 16) s_colp[w][16 * (w & 3) + l] = colacc;
  }
  __syncthreads();
  if (threadIdx.x < CH) {
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) x += s_colp[ww][threadIdx.x];
    s_cp[0][threadIdx.x] = x;
  }
  __syncthreads();
  // dk = part + dAr K + dAr^T K + beta eg dBk; dv = beta dBv
  {
    E* dk = reinterpret_cast<E*>(a.dk);
    E* dv = reinterpret_cast<E*>(a.dv);
    for (int t = w; t < 4 * G::NTC; t += NWV) {
      const int ti = t / G::NTC, tj = t % G::NTC;
      f32x4 x = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_a[(16 * ti + i) * G::LC + k]; },
                        [&](int k, int j) { return s_k[k * G::LD + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
      x = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_a[k * G::LC + 16 * ti + i]; },
                  [&](int k, int j) { return s_k[k * G::LD + 16 * tj + j]; }, x);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        if (i < n) {
          const float bt = s_t.beta[i];
          const int64_t off = row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + j);
          dk[off] = (E)(s_dk[i * G::LD + j] + x[q] + bt * s_t.eg[i] * s_dW[i * G::LD + j]);
          dv[off] = (E)(bt * s_dU[i * G::LD + j]);
        }
      }
    }
  }
  // dbeta and dg (wave 0, lane = token)
  if (threadIdx.x < CH) {
    const int i = threadIdx.x;
    float r2 = 0.f, r3 = 0.f;
    for (int j = 0; j < D; ++j) {
      r2 += s_dU[i * G::LD + j] * s_v[i * G::LD + j];
      r3 += s_dW[i * G::LD + j] * s_k[i * G::LD + j];
    }
    float r1 = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) r1 += s_rp[0][ww][i];
    const float bt = s_t.beta[i], eg = s_t.eg[i];
    const float dbeta = r1 + r2 + eg * r3;
    const float dgam = s_cp[1][i] + bt * r1 - s_cp[0][i] + bt * eg * r3;
    // suffix sums within the token's sequence: lanes i + off in the same sequence
    const int cnt = s_t.cnt[i];
    float x = dgam;
#pragma unroll
    for (int off = 1; off < CH; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      const int cy = __shfl_down(cnt, off, 64);
      if (i + off < CH && cy == cnt) x += y;
    }
    const bool start = i == 0 ? (seq && cnt == 1) : cnt != s_t.cnt[i - 1];
    if (i < n) {
      a.dbeta[row0(b, t0, h, a.T, a.H) + i * (int)a.H] = dbeta;
      a.dg[row0(b, t0, h, a.T, a.H) + i * (int)a.H] = start ? 0.f : x;
    }
  }
}

// ---- gradients per chunk, value slices ------------------------------------------------------
// The formulas of delta_grad with the value dimension taken in slices of SV
// columns, for heads whose state and value-side tiles do not fit the LDS together
// (D = 128), or so that two workgroups share a CU (D = 64, 16-column slices, 80 KB).
// Every contraction over it (dO U^T, dO S0^T, U dS^T, dU S0^T, dBv U~^T, the row sums
// of dBv . V and <dS, S0>) accumulates over the slices in registers, dv = beta dBv
// is written slice by slice, and the key-side rest follows once, as in delta_grad.
template <typename E, int D>
__global__ __launch_bounds__(NTH, DeltaSlabs<D>::GRAD_OCC) void delta_grad_wide(DeltaArgs a) {
  using G = DGeo<D>;
  constexpr int SV = DeltaSlabs<D>::GRAD, LV = SV + 4, NSL = D / SV, NVT = SV / 16;
  constexpr int KT = 4 * G::NTC / NWV;         // key-shaped [64][D] tiles per wave
  constexpr int TV = CH * LV, TS = D * LV;     // a [64][SV] and a [D][SV] slice tile
  constexpr int ARENA = 5 * TV + 2 * TS;
  static_assert(ARENA >= 2 * G::TILE, "Q and the score tile, then W and dW, reuse the slice tiles");
  static_assert((4 * G::NTC) % NWV == 0 && 4 * NVT <= NWV, "tile ownership");
  __shared__ __attribute__((aligned(16))) float s_k[G::TILE], s_tm[G::TILE_C], s_ar[ARENA];
  __shared__ ChunkTerms s_t;
  __shared__ float s_rp[3][NWV][CH];   // per-wave row partials
  __shared__ float s_colp[NWV][CH];    // per-wave column partials
  __shared__ float s_cp[2][CH];        // column sums
  __shared__ float s_red[NWV];
  int64_t r, c;
  const int64_t idx = a.chunk_begin + blockIdx.x;
  chunk_of(a.T, a.P, idx, r, c);
  const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int64_t slen = shard_len(a.T, a.P, r);
  const int n = (int)(slen - 64 * c < CH ? slen - 64 * c : CH);
  if (r >= a.P || n <= 0) return;
  const int64_t t0 = shard_begin(a.T, a.P, r) + 64 * c;
  const int64_t nct = row_chunks(a.T, a.P);
  const int32_t* seq = a.seq_idx ? a.seq_idx + b * a.T : nullptr;
  const int w = threadIdx.x >> 6, l = lane_id();
  const float* cs0 = a.chunk_states + (bh * nct + idx) * (int64_t)(D * D);
  const float* cds = a.ws_dsc + (bh * nct + idx) * (int64_t)(D * D);
  float *s_do = s_ar, *s_u = s_ar + TV, *s_du = s_ar + 2 * TV, *s_ut = s_ar + 3 * TV, *s_v = s_ar + 4 * TV,
        *s_s0 = s_ar + 5 * TV, *s_ds = s_ar + 5 * TV + TS;

  // K and the terms; Q is fetched here and held in registers until the slices are
  // done, except at two workgroups per CU (fetched after them: registers)
  RowTile<E, D> rq;
  {
    RowTile<E, D> rk;
    TermRegs tr;
    tr.fetch(a.g, a.beta, seq, b, h, t0, n, a.T, a.H);
    rk.fetch(reinterpret_cast<const E*>(a.k), b, h, t0, n, a.T, a.H);
    if (DeltaSlabs<D>::GRAD_OCC <= 2) rq.fetch(reinterpret_cast<const E*>(a.q), b, h, t0, n, a.T, a.H);
    for (int e = threadIdx.x; e < 3 * NWV * CH; e += NTH) (&s_rp[0][0][0])[e] = 0.f;
    for (int e = threadIdx.x; e < NWV * CH; e += NTH) (&s_colp[0][0])[e] = 0.f;
    chunk_terms(s_t, tr);
    rk.put(s_k);
  }
  __syncthreads();
  // T = (I + A)^{-1}, A = strict-lower(beta_i D_ij k_i.k_j)
  for (int t = w; t < 16; t += NWV) {
    const int ti = t >> 2, tj = t & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti)
      acc = tile_mm_e<D, E, true, true>([&](int i, int k) { return s_k[(16 * ti + i) * G::LD + k]; },
                    [&](int k, int j) { return s_k[(16 * tj + j) * G::LD + k]; }, acc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
      const bool ok = j < i && s_t.cnt[i] == s_t.cnt[j];
      s_tm[i * G::LC + j] = ok ? s_t.beta[i] * __expf(s_t.gam[i] - s_t.gam[j]) * acc[q] : 0.f;
    }
  }
  __syncthreads();
  unit_lower_inverse(s_tm);

  // Sums over the value dimension. Score-shaped [64][64] tiles: wave w owns tiles
  // w and w + NWV (row tile t / 4, column tile t % 4, lower ones only); key-shaped
  // [64][D] tiles: wave w owns tiles t = w + NWV m, m < KT (row tile t / NTC, column
  // tile t % NTC).
  f32x4 x_dou[2], x_dbu[2], x_dos[KT], x_uds[KT], x_dus[KT];
#pragma unroll
  for (int m = 0; m < 2; ++m) x_dou[m] = x_dbu[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < KT; ++m) x_dos[m] = x_uds[m] = x_dus[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sp = 0.f, r2 = 0.f;            // <dS, S0> partial; rowsum(dBv . V) (lane = token, wave 0)
  RowTile<E, D, SV> pdo, pv;
  RowTile<float, D, SV> pu, pdu, put_;
  MatTile<D, SV> ps0, pds;
  auto fetch_slice = [&](int v0) {
    pdo.fetch(reinterpret_cast<const E*>(a.dO), b, h, t0, n, a.T, a.H, v0);
    pu.fetch(a.ws_u, b, h, t0, n, a.T, a.H, v0);
    pdu.fetch(a.ws_du, b, h, t0, n, a.T, a.H, v0);
    ps0.fetch(cs0, v0);
    pds.fetch(cds, v0);
    put_.fetch(a.ws_ut, b, h, t0, n, a.T, a.H, v0);
    pv.fetch(reinterpret_cast<const E*>(a.v), b, h, t0, n, a.T, a.H, v0);
  };
  // the next slice is fetched while this one is computed, except at D = 64, where
  // the registers it needs cost as many spills as it saves (measured; two
  // workgroups share a CU there and cover each other's loads)
  constexpr bool PREFETCH = D != 64;
  if (PREFETCH) fetch_slice(0);
  E* dv = reinterpret_cast<E*>(a.dv);
  for (int sl = 0; sl < NSL; ++sl) {
    const int v0 = SV * sl;
    if (!PREFETCH) fetch_slice(v0);
    pdo.put(s_do);
    pu.put(s_u);
    pdu.put(s_du);
    ps0.put(s_s0);
    pds.put(s_ds);
    put_.put(s_ut);
    pv.put(s_v);
    __syncthreads();
    if (PREFETCH && sl + 1 < NSL) fetch_slice(v0 + SV);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t = w + NWV * m, ti = t >> 2, tj = t & 3;
      if (tj <= ti)
        x_dou[m] = tile_mm_e<SV, E, true, false>([&](int i, int k) { return s_do[(16 * ti + i) * LV + k]; },
                                    [&](int k, int j) { return s_u[(16 * tj + j) * LV + k]; }, x_dou[m]);
    }
#pragma unroll
    for (int m = 0; m < KT; ++m) {
      const int t = w + NWV * m, ti = t / G::NTC, tj = t % G::NTC;
      x_dos[m] = tile_mm_e<SV, E, true, false>([&](int i, int k) { return s_do[(16 * ti + i) * LV + k]; },
                                  [&](int k, int j) { return s_s0[(16 * tj + j) * LV + k]; }, x_dos[m]);
      x_uds[m] = tile_mm_e<SV, E>([&](int i, int k) { return s_u[(16 * ti + i) * LV + k]; },
                                  [&](int k, int j) { return s_ds[(16 * tj + j) * LV + k]; }, x_uds[m]);
      x_dus[m] = tile_mm_e<SV, E>([&](int i, int k) { return s_du[(16 * ti + i) * LV + k]; },
                                  [&](int k, int j) { return s_s0[(16 * tj + j) * LV + k]; }, x_dus[m]);
    }
    for (int e = threadIdx.x; e < D * SV; e += NTH) sp += s_ds[(e / SV) * LV + e % SV] * s_s0[(e / SV) * LV + e % SV];
    // dBv = T^T dU over the slice (row tile ti takes k tiles ti..3; waves w < 4 NVT,
    // one tile each), dv = beta dBv
    f32x4 bv = {0.f, 0.f, 0.f, 0.f};
    const bool owns_bv = w < 4 * NVT;
    if (owns_bv) {
      const int ti = w / NVT, tj = w % NVT;
      for (int kt = ti; kt < 4; ++kt)
        bv = tile_mm<16>([&](int i, int q) { return s_tm[(16 * kt + q) * G::LC + 16 * ti + i]; },
                         [&](int q, int j) { return s_du[(16 * kt + q) * LV + 16 * tj + j]; }, bv);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q;
        if (i < n) dv[row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + v0 + 16 * tj + (l & 15))] = (E)(s_t.beta[i] * bv[q]);
      }
    }
    __syncthreads();   // every read of dU is done
    if (owns_bv) {
      const int ti = w / NVT, tj = w % NVT;
#pragma unroll
      for (int q = 0; q < 4; ++q) s_du[(16 * ti + 4 * (l >> 4) + q) * LV + 16 * tj + (l & 15)] = bv[q];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t = w + NWV * m, ti = t >> 2, tj = t & 3;
      if (tj <= ti)
        x_dbu[m] = tile_mm_e<SV, E>([&](int i, int k) { return s_du[(16 * ti + i) * LV + k]; },
                                    [&](int k, int j) { return s_ut[(16 * tj + j) * LV + k]; }, x_dbu[m]);
    }
    if (threadIdx.x < CH) {
      const int i = threadIdx.x;
#pragma unroll 8
      for (int j = 0; j < SV; ++j) r2 += s_du[i * LV + j] * s_v[i * LV + j];
    }
    __syncthreads();   // the slice tiles are read
  }
  sp = wave_sum(sp);
  if (l == 0) s_red[w] = sp;

  // Q and the score tile in the slice space: dPr = (dO U^T) . D and the decay terms
  // of dGam
  float *s_q = s_ar, *s_dp = s_ar + G::TILE;
  if (DeltaSlabs<D>::GRAD_OCC > 2) rq.fetch(reinterpret_cast<const E*>(a.q), b, h, t0, n, a.T, a.H);
  rq.put(s_q);
  RowTile<float, D> rw;
  rw.fetch(a.ws_w, b, h, t0, n, a.T, a.H);
  __syncthreads();
  {
    float colacc = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t = w + NWV * m, ti = t >> 2, tj = t & 3;
      f32x4 qk = {0.f, 0.f, 0.f, 0.f};
      if (tj <= ti)
        qk = tile_mm_e<D, E, true, true>([&](int i, int k) { return s_q[(16 * ti + i) * G::LD + k]; },
                     [&](int k, int j) { return s_k[(16 * tj + j) * G::LD + k]; }, qk);
      float rowp[4], colp = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        const bool ok = j <= i && s_t.cnt[i] == s_t.cnt[j];
        const float dpr = ok ? __expf(s_t.gam[i] - s_t.gam[j]) * x_dou[m][q] : 0.f;
        s_dp[i * G::LC + j] = dpr;
        const float pa = dpr * qk[q];
        rowp[q] = pa;
        colp += pa;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x = rowp[q];
        x += __shfl_xor(x, 1, 64);
        x += __shfl_xor(x, 2, 64);
        x += __shfl_xor(x, 4, 64);
        x += __shfl_xor(x, 8, 64);
        if ((l & 15) == 0) s_rp[0][w][16 * ti + 4 * (l >> 4) + q] = x;
      }
      colp += __shfl_xor(colp, 16, 64);
      colp += __shfl_xor(colp, 32, 64);
      colacc += colp;
    }
    if (l < 16) s_colp[w][16 * (w & 3) + l] = colacc;   // the wave's column tile, over its row tiles
  }
  __syncthreads();
  if (threadIdx.x < CH) {
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) x += s_colp[ww][threadIdx.x];
    s_cp[0][threadIdx.x] = x;
  }
  // dq = dPr K + eg (dO S0^T); dk (part, kept in registers) = dPr^T Q + el (U dS^T);
  // row partials of Q . (dO S0^T) and el (U dS^T) . K
  f32x4 dkp[KT];
  {
    E* dq = reinterpret_cast<E*>(a.dq);
#pragma unroll
    for (int m = 0; m < KT; ++m) {
      const int t = w + NWV * m, ti = t / G::NTC, tj = t % G::NTC;
      f32x4 x = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_dp[(16 * ti + i) * G::LC + k]; },
                        [&](int k, int j) { return s_k[k * G::LD + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 z = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_dp[k * G::LC + 16 * ti + i]; },
                        [&](int k, int j) { return s_q[k * G::LD + 16 * tj + j]; }, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        const float eg = s_t.eg[i], el = s_t.el[i];
        const float y = x_dos[m][q];
        if (i < n) dq[row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + j)] = (E)(x[q] + eg * y);
        const float ue = el * x_uds[m][q];
        dkp[m][q] = z[q] + ue;
        float p1 = eg * y * s_q[i * G::LD + j];
        float p2 = ue * s_k[i * G::LD + j];
        p1 += __shfl_xor(p1, 1, 64);
        p1 += __shfl_xor(p1, 2, 64);
        p1 += __shfl_xor(p1, 4, 64);
        p1 += __shfl_xor(p1, 8, 64);
        p2 += __shfl_xor(p2, 1, 64);
        p2 += __shfl_xor(p2, 2, 64);
        p2 += __shfl_xor(p2, 4, 64);
        p2 += __shfl_xor(p2, 8, 64);
        if ((l & 15) == 0) {
          s_rp[1][w][i] = p1;
          s_rp[2][w][i] = p2;
        }
      }
    }
  }
  __syncthreads();
  // dGam (partial) into s_cp[1]
  if (threadIdx.x < CH) {
    const int i = threadIdx.x;
    float rowpa = 0.f, qdos = 0.f, tk = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) {
      rowpa += s_rp[0][ww][i];
      qdos += s_rp[1][ww][i];
      tk += s_rp[2][ww][i];
    }
    float dgam = rowpa - s_cp[0][i] + qdos - tk;
    float tks = tk;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tks += __shfl_xor(tks, off, 64);
    if (i == CH - 1) {
      float spp = 0.f;
#pragma unroll
      for (int ww = 0; ww < NWV; ++ww) spp += s_red[ww];
      dgam += tks + s_t.sc[0] * spp;
    }
    s_cp[1][i] = dgam;
  }
  // W and dW = -dU S0^T in the slice space (Q and dPr are dead)
  float *s_w = s_ar, *s_dW = s_ar + G::TILE;
  rw.put(s_w);
#pragma unroll
  for (int m = 0; m < KT; ++m) {
    const int t = w + NWV * m, ti = t / G::NTC, tj = t % G::NTC;
#pragma unroll
    for (int q = 0; q < 4; ++q) s_dW[(16 * ti + 4 * (l >> 4) + q) * G::LD + 16 * tj + (l & 15)] = -x_dus[m][q];
  }
  __syncthreads();
  // dBk = T^T dW in place, held in registers until every wave has read dW
  {
    f32x4 res[KT];
#pragma unroll
    for (int m = 0; m < KT; ++m) {
      const int t = w + NWV * m, ti = t / G::NTC, tj = t % G::NTC;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kt = ti; kt < 4; ++kt)
        acc = tile_mm<16>([&](int i, int q) { return s_tm[(16 * kt + q) * G::LC + 16 * ti + i]; },
                          [&](int q, int j) { return s_dW[(16 * kt + q) * G::LD + 16 * tj + j]; }, acc);
      res[m] = acc;
    }
    for (int e = threadIdx.x; e < 2 * NWV * CH; e += NTH) (&s_rp[0][0][0])[e] = 0.f;
    for (int e = threadIdx.x; e < NWV * CH; e += NTH) (&s_colp[0][0])[e] = 0.f;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < KT; ++m) {
      const int t = w + NWV * m, ti = t / G::NTC, tj = t % G::NTC;
#pragma unroll
      for (int q = 0; q < 4; ++q) s_dW[(16 * ti + 4 * (l >> 4) + q) * G::LD + 16 * tj + (l & 15)] = res[m][q];
    }
  }
  __syncthreads();
  // dA = strict-lower(-(dBv U~^T + dBk W^T)); dAr = dA . D . beta_i in place of T;
  // row sums of dA . D . KK^T (dbeta) and column sums of dA . A (dGam)
  {
    float colacc = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int t = w + NWV * m, ti = t >> 2, tj = t & 3;
      f32x4 x = x_dbu[m], kk = {0.f, 0.f, 0.f, 0.f};
      if (tj <= ti) {
        x = tile_mm_e<D, E>([&](int i, int k) { return s_dW[(16 * ti + i) * G::LD + k]; },
                    [&](int k, int j) { return s_w[(16 * tj + j) * G::LD + k]; }, x);
        kk = tile_mm_e<D, E, true, true>([&](int i, int k) { return s_k[(16 * ti + i) * G::LD + k]; },
                     [&](int k, int j) { return s_k[(16 * tj + j) * G::LD + k]; }, kk);
      }
      float colp = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        const bool ok = j < i && s_t.cnt[i] == s_t.cnt[j];
        const float dec = ok ? __expf(s_t.gam[i] - s_t.gam[j]) : 0.f;
        const float da = ok ? -x[q] : 0.f;
        const float r1 = da * dec * kk[q];
        s_tm[i * G::LC + j] = da * dec * s_t.beta[i];
        colp += r1 * s_t.beta[i];
        float x1 = r1;
        x1 += __shfl_xor(x1, 1, 64);
        x1 += __shfl_xor(x1, 2, 64);
        x1 += __shfl_xor(x1, 4, 64);
        x1 += __shfl_xor(x1, 8, 64);
        if ((l & 15) == 0) s_rp[0][w][i] = x1;
      }
      colp += __shfl_xor(colp, 16, 64);
      colp += __shfl_xor(colp, 32, 64);
      colacc += colp;
    }
    if (l < 16) s_colp[w][16 * (w & 3) + l] = colacc;
  }
  __syncthreads();
  if (threadIdx.x < CH) {
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) x += s_colp[ww][threadIdx.x];
    s_cp[0][threadIdx.x] = x;
  }
  __syncthreads();
  // dk = part + dAr K + dAr^T K + beta eg dBk
  {
    E* dk = reinterpret_cast<E*>(a.dk);
#pragma unroll
    for (int m = 0; m < KT; ++m) {
      const int t = w + NWV * m, ti = t / G::NTC, tj = t % G::NTC;
      f32x4 x = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_tm[(16 * ti + i) * G::LC + k]; },
                        [&](int k, int j) { return s_k[k * G::LD + 16 * tj + j]; }, dkp[m]);
      x = tile_mm_e<CH, E, false, true>([&](int i, int k) { return s_tm[k * G::LC + 16 * ti + i]; },
                  [&](int k, int j) { return s_k[k * G::LD + 16 * tj + j]; }, x);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 16 * ti + 4 * (l >> 4) + q, j = 16 * tj + (l & 15);
        if (i < n)
          dk[row0(b, t0, h, a.T, a.H) * D + (i * ((int)a.H * D) + j)] = (E)(x[q] + s_t.beta[i] * s_t.eg[i] * s_dW[i * G::LD + j]);
      }
    }
  }
  // dbeta and dg (wave 0, lane = token)
  if (threadIdx.x < CH) {
    const int i = threadIdx.x;
    float r3 = 0.f;
    for (int j = 0; j < D; ++j) r3 += s_dW[i * G::LD + j] * s_k[i * G::LD + j];
    float r1 = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) r1 += s_rp[0][ww][i];
    const float bt = s_t.beta[i], eg = s_t.eg[i];
    const float dbeta = r1 + r2 + eg * r3;
    const float dgam = s_cp[1][i] + bt * r1 - s_cp[0][i] + bt * eg * r3;
    const int cnt = s_t.cnt[i];
    float x = dgam;
#pragma unroll
    for (int off = 1; off < CH; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      const int cy = __shfl_down(cnt, off, 64);
      if (i + off < CH && cy == cnt) x += y;
    }
    const bool start = i == 0 ? (seq && cnt == 1) : cnt != s_t.cnt[i - 1];
    if (i < n) {
      a.dbeta[row0(b, t0, h, a.T, a.H) + i * (int)a.H] = dbeta;
      a.dg[row0(b, t0, h, a.T, a.H) + i * (int)a.H] = start ? 0.f : x;
    }
  }
}

#define CPLA_INST_DELTA_WALKS(E, D)                                            \
  template __global__ void delta_wy<E, D>(DeltaArgs);                          \
  template __global__ void delta_fwalk<E, D, false>(DeltaArgs);                \
  template __global__ void delta_fwalk<E, D, true>(DeltaArgs);                 \
  template __global__ void delta_out<E, D>(DeltaArgs);                         \
  template __global__ void delta_bwalk<E, D, false>(DeltaArgs);                \
  template __global__ void delta_bwalk<E, D, true>(DeltaArgs);
#define CPLA_INST_DELTA(E, D)                                                  \
  CPLA_INST_DELTA_WALKS(E, D)                                                  \
  template __global__ void delta_grad<E, D>(DeltaArgs);
CPLA_INST_DELTA(float, 16)
CPLA_INST_DELTA(float, 32)
CPLA_INST_DELTA(float, 64)
CPLA_INST_DELTA(bf16_t, 16)
CPLA_INST_DELTA(bf16_t, 32)
CPLA_INST_DELTA(bf16_t, 64)
CPLA_INST_DELTA_WALKS(bf16_t, 128)
template __global__ void delta_grad_wide<bf16_t, 128>(DeltaArgs);
template __global__ void delta_grad_wide<bf16_t, 64>(DeltaArgs);
template __global__ void delta_grad_wide<float, 64>(DeltaArgs);
template __global__ void delta_grad_wide<bf16_t, 32>(DeltaArgs);
template __global__ void delta_grad_wide<float, 32>(DeltaArgs);
template __global__ void delta_scan<16>(DeltaScanArgs);
template __global__ void delta_scan<32>(DeltaScanArgs);
template __global__ void delta_scan<64>(DeltaScanArgs);
template __global__ void delta_scan<128>(DeltaScanArgs);

}  // namespace cpla
