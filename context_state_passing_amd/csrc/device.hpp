// Device primitives for the chunkwise linear-attention kernels (gfx950 only).
//
// MFMA: v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulators) and
// v_mfma_f64_16x16x4_f64 (fp32 operands widened exactly to fp64, fp64
// accumulators, eight issues per 32-deep step). A "fragment" is the 8 values a
// lane contributes to one 16x16x32 step: lane l holds operand row/column l%16
// and the 8 contraction indices {8g + e} (g = l/16), or a permuted set when the
// fragment is rebuilt from accumulators (see acc_to_frag). The fp64 form splits
// the same 8 indices over eight 16x16x4 issues. Its accumulator tile puts rows
// g, g+4, g+8, g+12 in lane group g (measured), where the fp32 tiles put rows
// 4g..4g+3; the fp64 issue therefore takes its first operand's rows permuted
// (a 4x4 transpose within each 16-lane group), which lands the product rows in
// the fp32 layout, so both element types share every layout below. With fp32
// inputs every product and every sum a walk carries from chunk to chunk is thus
// formed in fp64, and a value is rounded to fp32 only where it is stored or
// becomes an operand.
//
// LDS tiles are token-major (as the inputs sit in HBM) with 16 bytes of padding
// per row. Contractions over features read fragments directly; contractions over
// tokens read them with the gfx950 transpose load ds_read_b64_tr_b16, where lane
// c = 4r + s of each 16-lane group names row r / columns 4s..4s+3 of a 4x16
// block and lane i receives column i.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpla {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;      // chunk length (tokens)
// Waves per workgroup for a (padded) head size: 8 at 128 (two per SIMD, so one
// wave's memory or LDS wait overlaps the other's work), 4 below.
constexpr int waves_for(int dpad) { return dpad >= 128 ? 8 : 4; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The lane (thread) index behind an empty asm statement, so that the values a
// loop body derives from it are computed inside the body: in the long chunk
// walks the compiler would otherwise hoist every lane-dependent LDS and global
// address out of the chunk loop and hold each in a register for the whole walk.
// Take one per phase and pass it to the loaders below.
__device__ __forceinline__ int lane_fresh() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  __builtin_assume(l >= 0 && l < 64);
  return l;
}
template <int NT> __device__ __forceinline__ int tid_fresh() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  __builtin_assume(t >= 0 && t < NT);
  return t;
}
// fresh (FRESH = true) or plain indices, for walks that share code
template <bool FRESH> __device__ __forceinline__ int lane_pick() { return FRESH ? lane_fresh() : lane_id(); }
template <bool FRESH, int NT> __device__ __forceinline__ int tid_pick() {
  return FRESH ? tid_fresh<NT>() : (int)threadIdx.x;
}
// wave index within the workgroup, uniform (scalar register)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---- element traits -------------------------------------------------------------

template <typename E> struct Frag;
template <> struct Frag<bf16_t> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

template <typename E> __device__ __forceinline__ E to_e(float x);
template <> __device__ __forceinline__ bf16_t to_e<bf16_t>(float x) { return (bf16_t)x; }
template <> __device__ __forceinline__ float to_e<float>(float x) { return x; }
__device__ __forceinline__ float to_f(bf16_t x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

template <typename E> constexpr int lds_pad() { return 16 / (int)sizeof(E); }

// Accumulator tile (4 values per lane) of the products of E operands: fp32 for
// bf16, fp64 for fp32.
template <typename E> struct AccT;
template <> struct AccT<bf16_t> { typedef f32x4 type; };
template <> struct AccT<float> { typedef f64x4 type; };
template <typename E> using acc4 = typename AccT<E>::type;
// an fp32 vector as the accumulator type V (exact)
template <typename V> __device__ __forceinline__ V widen4(const f32x4& x) { return __builtin_convertvector(x, V); }
// accumulator values as fp32 (rounded once for fp64)
__device__ __forceinline__ f32x4 narrow4(const f32x4& x) { return x; }
__device__ __forceinline__ f32x4 narrow4(const f64x4& x) { return __builtin_convertvector(x, f32x4); }

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
// fp64 issue: lane l supplies row 4(x%4) + x/4 (x = l%16) of the first operand,
// read from the lane holding that row, so that accumulator row 4g + rr sits in
// lane group g as in the fp32 tiles
__device__ __forceinline__ void mma(f64x4& acc, const Frag<float>& a, const Frag<float>& b) {
  const int l = lane_id();
  const int src = (l & 48) | ((l & 3) << 2) | ((l >> 2) & 3);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float ar = __shfl(a.v[s], src, 64);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)ar, (double)b.v[s], acc, 0, 0, 0);
  }
}

template <typename E> __device__ __forceinline__ void frag_zero(Frag<E>& f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = to_e<E>(0.f);
}
template <typename E> __device__ __forceinline__ float frag_get(const Frag<E>& f, int e) { return to_f(f.v[e]); }
template <typename E> __device__ __forceinline__ void frag_set(Frag<E>& f, int e, float x) { f.v[e] = to_e<E>(x); }

// ---- fragment loads from LDS tiles ----------------------------------------------
// Tile: row-major, `ld` elements per row. All offsets in elements.

// lane-fixed row `row`, contraction indices k0 + 8g + e (16 contiguous bytes for bf16)
__device__ __forceinline__ void frag_direct(Frag<bf16_t>& f, const bf16_t* t, int ld, int row, int k0, int l = lane_id()) {
  const int g = l >> 4;
  f.v = *reinterpret_cast<const bf16x8*>(t + row * ld + k0 + 8 * g);
}
__device__ __forceinline__ void frag_direct(Frag<float>& f, const float* t, int ld, int row, int k0, int l = lane_id()) {
  const int g = l >> 4;
  const f32x4* p = reinterpret_cast<const f32x4*>(t + row * ld + k0 + 8 * g);
  f32x4 a = p[0], b = p[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
}
// lane-fixed row, permuted contraction indices {k0 + 4g + e, k0 + 16 + 4g + e}
__device__ __forceinline__ void frag_direct_perm(Frag<bf16_t>& f, const bf16_t* t, int ld, int row, int k0, int l = lane_id()) {
  const int g = l >> 4;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(t + row * ld + k0 + 4 * g);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(t + row * ld + k0 + 16 + 4 * g);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_direct_perm(Frag<float>& f, const float* t, int ld, int row, int k0, int l = lane_id()) {
  const int g = l >> 4;
  f32x4 a = *reinterpret_cast<const f32x4*>(t + row * ld + k0 + 4 * g);
  f32x4 b = *reinterpret_cast<const f32x4*>(t + row * ld + k0 + 16 + 4 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
}

// Direct global -> LDS copy (the gfx950 LDS DMA form of a vector load): lane i of
// the wave copies BYTES bytes from src to lds_wave + i * BYTES, without passing
// through registers. lds_wave must be the same for every lane of the wave.
// Completion is counted like any vector-memory load (vmcnt).
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* src, void* lds_wave) {
  static_assert(BYTES == 4 || BYTES == 16, "LDS DMA copies 4 or 16 bytes per lane here");
  typedef __attribute__((address_space(3))) void lds_void;
  if constexpr (BYTES == 16) __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_wave, 16, 0, 0);
  else __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_wave, 4, 0, 0);
}

// lane-fixed column col0 + l%16, contraction over rows k0 + 8g + e (transpose load)
__device__ __forceinline__ s16x4 ds_tr16(const bf16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}
__device__ __forceinline__ void frag_tr(Frag<bf16_t>& f, const bf16_t* t, int ld, int k0, int col0, int l = lane_id()) {
  const int g = l >> 4, i = l & 15;
  s16x4 a = ds_tr16(t + (k0 + 8 * g + (i >> 2)) * ld + col0 + 4 * (i & 3));
  s16x4 b = ds_tr16(t + (k0 + 8 * g + 4 + (i >> 2)) * ld + col0 + 4 * (i & 3));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  f.v = __builtin_bit_cast(bf16x8, c);
}
__device__ __forceinline__ void frag_tr(Frag<float>& f, const float* t, int ld, int k0, int col0, int l = lane_id()) {
  const int g = l >> 4, i = l & 15;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = t[(k0 + 8 * g + e) * ld + col0 + i];
}
// permuted rows {k0 + 4g + e, k0 + 16 + 4g + e}
__device__ __forceinline__ void frag_tr_perm(Frag<bf16_t>& f, const bf16_t* t, int ld, int k0, int col0, int l = lane_id()) {
  const int g = l >> 4, i = l & 15;
  s16x4 a = ds_tr16(t + (k0 + 4 * g + (i >> 2)) * ld + col0 + 4 * (i & 3));
  s16x4 b = ds_tr16(t + (k0 + 16 + 4 * g + (i >> 2)) * ld + col0 + 4 * (i & 3));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  f.v = __builtin_bit_cast(bf16x8, c);
}
__device__ __forceinline__ void frag_tr_perm(Frag<float>& f, const float* t, int ld, int k0, int col0, int l = lane_id()) {
  const int g = l >> 4, i = l & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = t[(k0 + 4 * g + e) * ld + col0 + i];
    f.v[4 + e] = t[(k0 + 16 + 4 * g + e) * ld + col0 + i];
  }
}
// contraction index of fragment slot e for the plain and the permuted orders
__device__ __forceinline__ int kidx(int e, int l = lane_id()) { return 8 * (l >> 4) + e; }
__device__ __forceinline__ int kidx_perm(int e, int l = lane_id()) { return 4 * (l >> 4) + (e & 3) + ((e >> 2) << 4); }

// Two 16x16 accumulator tiles stacked along their row index (rows r0..r0+31,
// lane-fixed column) as one operand fragment contracting over those rows, in the
// permuted order {r0 + 4g + e, r0 + 16 + 4g + e}. `s0`, `s1` scale rows.
template <typename E, typename V>
__device__ __forceinline__ void acc_to_frag(Frag<E>& f, const V& lo, const V& hi) {
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = to_e<E>((float)lo[e]); f.v[4 + e] = to_e<E>((float)hi[e]); }
}

// ---- split bf16 arithmetic ---------------------------------------------------------
// An fp32 intermediate x feeds bf16 MFMAs as hi = bf16(x), lo = bf16(x - hi); a
// product then takes hi*b + lo*b (and + hi*b_lo when the other operand is split
// too), which keeps its error near fp32 rounding instead of bf16 rounding. The
// kernel inputs themselves are exact in bf16 and need no split. With fp32
// operands the lo parts are zero and their MFMAs are skipped.
template <typename E> struct Split { static constexpr bool on = sizeof(E) == 2; };

__device__ __forceinline__ void split_frag(Frag<float>& hi, Frag<float>& lo, const float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) hi.v[e] = x[e];
}
// Residuals of a pair (x0, x1) after rounding to the packed bf16 pair h:
// x0 - h[0] and x1 - h[1], each one v_dot2c_f32_bf16 (x + h . m with m = (-1, 0)
// or (0, -1): the products are exact and the difference is representable, so the
// result is exact), instead of unpacking h and subtracting. The multipliers are
// passed in scalar registers: as an inline constant, the pair (-1, 0) is encoded
// as fp32 -1.0, whose bits are the pair (0, -1).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void bf16_residual_pair(unsigned h, float& x0, float& x1) {
  unsigned m0 = 0x0000bf80u, m1 = 0xbf800000u;
  asm("" : "+s"(m0), "+s"(m1));
  const bf16x2 hp = __builtin_bit_cast(bf16x2, h);
  x0 = __builtin_amdgcn_fdot2_f32_bf16(hp, __builtin_bit_cast(bf16x2, m0), x0, false);
  x1 = __builtin_amdgcn_fdot2_f32_bf16(hp, __builtin_bit_cast(bf16x2, m1), x1, false);
}
// bf16: hi converted in pairs, lo = bf16 of the exact residuals
__device__ __forceinline__ void split_frag(Frag<bf16_t>& hi, Frag<bf16_t>& lo, const float (&x)[8]) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  f32x8 r = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  hi.v = __builtin_convertvector(r, bf16x8);
  const u32x4 hb = __builtin_bit_cast(u32x4, hi.v);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = r[2 * i], b = r[2 * i + 1];
    bf16_residual_pair(hb[i], a, b);
    r[2 * i] = a;
    r[2 * i + 1] = b;
  }
  lo.v = __builtin_convertvector(r, bf16x8);
}
// acc += (a_hi + a_lo) (b_hi + b_lo), dropping lo*lo
template <typename E, typename V>
__device__ __forceinline__ void mma3(V& acc, const Frag<E>& ah, const Frag<E>& al, const Frag<E>& bh,
                                     const Frag<E>& bl) {
  mma(acc, ah, bh);
  if constexpr (Split<E>::on) {
    mma(acc, ah, bl);
    mma(acc, al, bh);
  }
}
// acc += (a_hi + a_lo) b
template <typename E, typename V>
__device__ __forceinline__ void mma2a(V& acc, const Frag<E>& ah, const Frag<E>& al, const Frag<E>& b) {
  mma(acc, ah, b);
  if constexpr (Split<E>::on) mma(acc, al, b);
}
// acc += a (b_hi + b_lo)
template <typename E, typename V>
__device__ __forceinline__ void mma2b(V& acc, const Frag<E>& a, const Frag<E>& bh, const Frag<E>& bl) {
  mma(acc, a, bh);
  if constexpr (Split<E>::on) mma(acc, a, bl);
}
// Two accumulator tiles (see acc_to_frag) as split hi/lo fragments.
template <typename E, typename V>
__device__ __forceinline__ void acc_to_frag_split(Frag<E>& hi, Frag<E>& lo, const V& a, const V& b) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = (float)a[e]; x[4 + e] = (float)b[e]; }
  split_frag(hi, lo, x);
}
// Store x as hi (and lo) into two LDS tiles at the same offset.
template <typename E>
__device__ __forceinline__ void store_split(E* hi, E* lo, int off, float x) {
  const E h = to_e<E>(x);
  hi[off] = h;
  if constexpr (Split<E>::on) lo[off] = to_e<E>(x - to_f(h));
}

// ---- per-chunk token structure ---------------------------------------------------
// Bit i of `starts` is set when chunk token i starts a packed sequence.
struct ChunkSeg {
  uint64_t starts;
  __device__ __forceinline__ bool any() const { return starts != 0ull; }
  // first start position (64 if none): tokens before it still see the incoming state
  __device__ __forceinline__ int first() const { return starts ? __builtin_ctzll(starts) : CH; }
  // last start position (0 if none): tokens from it on reach the outgoing state
  __device__ __forceinline__ int last() const { return starts ? 63 - __builtin_clzll(starts) : 0; }
  __device__ __forceinline__ bool live(int i) const { return i < first(); }
  __device__ __forceinline__ bool tail(int i) const { return i >= last(); }
  // number of starts at or before token t: tokens i >= j share a sequence iff
  // their counts are equal
  __device__ __forceinline__ int index(int t) const { return __popcll(starts & ((2ull << t) - 1ull)); }
  // i >= j and no start in (j, i]
  __device__ __forceinline__ bool same(int i, int j) const {
    if (i < j) return false;
    if (!starts) return true;
    uint64_t hi = (i >= 63) ? ~0ull : ((2ull << i) - 1ull);
    uint64_t lo = (2ull << j) - 1ull;
    return (starts & (hi & ~lo)) == 0ull;
  }
};

template <typename T> __device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace cpla
