// Kernel argument blocks and templates shared by the launchers (abi.cpp) and the
// kernel translation units. Device code only ever sees these plain structs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace cpla {

struct FwdArgs {
  int64_t B, T, H, W;        // W: floats per summary record
  int64_t Hqk;               // heads of q and k (H, or G: head h reads head h / qk_div)
  int P, rank_begin, m_slot, qk_div;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* w;            // scalar decay: per-token input weight [B,T,H] (fp32), or null (1)
  const int32_t* seq_idx;    // packed sequences or null
  const float* state_in;     // apply: incoming state of every shard [P,B,H,dk,dv]
  float* summary;            // prepare: [P,B,H,W]
  void* out;                 // apply: o
  float* chunk_states;       // apply: state entering every chunk (fp32), or null
};

struct BwdArgs {
  int64_t B, T, H, W;
  int64_t Hqk;               // heads of q and k (as in FwdArgs); dq and dk are per head
  int P, rank_begin, m_slot, qk_div;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* w;            // scalar decay: per-token input weight, or null (1)
  const void* dO;
  const int32_t* seq_idx;
  const float* chunk_states; // apply: saved forward states (fp32)
  const float* grad_in;      // apply: gradient arriving at every shard's end [P,B,H,dk,dv]
  float* summary;            // prepare: [P,B,H,W]
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dw;                 // apply, with w: gradient w.r.t. w [B,T,H] (fp32)
};

struct ScanArgs {
  int64_t BH, W, n_elem;     // n_elem = B*H*dk*dv
  int dk, dv, H, P, m_slot, diag, reverse;
  const float* summary;      // [P,B,H,W]
  const int32_t* slice;      // [B,P] preceding_rank_start (forward) / following_rank_stop (reverse), or null
  const float* init;         // S_init (forward) / dS_final (reverse), or null
  float* out;                // [P,B,H,dk,dv]
  float* fin;                // final state (forward) / dS_init (reverse), or null
};

// The gated delta rule (dense transition), d_k = d_v = D. Workspace tensors are
// fp32: ws_ut, ws_w, ws_u, ws_du [B,T,H,D]; chunk states and ws_dsc (the gradient
// at every chunk's end) [B,H,row_chunks,D,D].
constexpr int DELTA_THREADS = 512;   // threads per workgroup of every delta-rule kernel

// State columns per workgroup (the grid's z extent is the width over these): the
// state's columns evolve independently, and at D = 128 a whole fp32 state with the
// chunk's tiles does not fit the LDS.
template <int D> struct DeltaSlabs {
  static constexpr int OUT = D;                    // delta_out: value columns
  static constexpr int BWALK = D < 64 ? D : (D == 64 ? 32 : 64);   // delta_bwalk: value columns of dS
  static constexpr int BWALK_OCC = D == 64 ? 4 : 2;                 // delta_bwalk: waves per SIMD aimed at
  static constexpr int GRAD = D > 64 ? 32 : 16;    // delta_grad_wide: value slice
  static constexpr int GRAD_OCC = D > 64 ? 2 : 4;  // delta_grad_wide: waves per SIMD aimed at (4: two
                                                   // workgroups per CU, 128 registers per lane)
  static constexpr int SCAN = D <= 32 ? D : 32;    // delta_scan: columns of S or dS
};
template <int D, bool APPLY> struct FwalkSlab {     // delta_fwalk: columns of [delta_S | M] or S
  static constexpr int NZ = APPLY ? D : 2 * D;
  // D = 64 apply: two slabs, so that twice the workgroups run two per CU (measured:
  // the prepare walk does not gain from it)
  static constexpr bool HALF = D == 64 && APPLY;
  static constexpr int SZ = D <= 64 ? (HALF ? NZ / 2 : NZ) : D;
  static constexpr int OCC = HALF ? 4 : 2;         // waves per SIMD aimed at
};

struct DeltaArgs {
  int64_t B, T, H;
  int P, rank_begin;
  int64_t chunk_begin;       // per-chunk kernels: first chunk (row-local index) of the launch
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  const float* g;            // [B,T,H] log-decay
  const float* beta;         // [B,T,H] write strength
  const int32_t* seq_idx;    // [B,T] packed sequences or null
  const float* state_in;     // forward apply: S_in [P,B,H,D,D]; backward apply: dS_out
  const float* fwd_summary;  // backward prepare: the forward records (M is copied)
  float* summary;            // prepare: [P,B,H,2 D^2] records [M | delta_S or gamma]
  void* out;                 // o
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* chunk_states;
  float* ws_ut;
  float* ws_w;
  float* ws_u;
  float* ws_du;
  float* ws_dsc;
};

struct DeltaScanArgs {
  int64_t BH, H;
  int P, reverse;
  const float* summary;      // [P,B,H,2 D^2]
  const int32_t* slice;      // [B,P] or null
  const float* init;         // S_init / dS_final, or null
  float* out;                // [P,B,H,D,D]
  float* fin;                // final state / dS_init, or null
};

template <typename E, int D> __global__ void delta_wy(DeltaArgs a);
template <typename E, int D, bool APPLY> __global__ void delta_fwalk(DeltaArgs a);
template <int D> __global__ void delta_scan(DeltaScanArgs a);
template <typename E, int D> __global__ void delta_out(DeltaArgs a);
template <typename E, int D, bool APPLY> __global__ void delta_bwalk(DeltaArgs a);
template <typename E, int D> __global__ void delta_grad(DeltaArgs a);
template <typename E, int D> __global__ void delta_grad_wide(DeltaArgs a);

// TAIL: some shard's length is not a multiple of the chunk (a partial last chunk
// to mask); without it every guard compiles away.
// SPLIT (apply only): the shard's chunks are divided among gridDim.z workgroups;
// workgroup z emits chunks [z nc / Z, (z + 1) nc / Z) after replaying the ones
// before them from the shard's incoming state (staging and state update only).
// PK: the stream may be packed (a.seq_idx honoured); the apply walks of unpacked
// problems take PK = false, where every sequence mask folds away at compile time.
template <typename E, int DK, int DV, int DECAY, bool APPLY, bool TAIL, bool SPLIT = false, bool PK = true>
__global__ void fwd_walk(FwdArgs a);
// SPLIT (apply, no decay or scalar decay): as for fwd_walk, walking backwards:
// workgroup z emits chunks [z nc / Z, (z + 1) nc / Z) after replaying the later
// ones from the shard's outgoing gradient (staging and the adjoint update only).
template <typename E, int DK, int DV, int DECAY, bool APPLY, bool GF32, bool TAIL, bool SPLIT = false, bool PK = true>
__global__ void bwd_walk(BwdArgs a);
__global__ void affine_scan(ScanArgs a);

// Range check of a diagonal log-decay (cpla_check_decay_range).
struct DecayCheckArgs {
  int64_t B, T, H, dk, nchunks, n;   // nchunks: chunks of the handled shards; n = B*H*nchunks*dk
  int P, rank_begin;
  float limit;
  const float* g;
  int32_t* count;
};
__global__ void decay_check_zero(int32_t* count);
__global__ void decay_range(DecayCheckArgs a);

}  // namespace cpla
