// C-ABI entry points: host-side validation, then launches on the caller's stream.
//
// The four calls are the local-backend protocol of the Megatron-Core page
// core.ssm.context_parallel.chunkwise (LinearAttentionCPBackend.cp_forward_prepare,
// cp_forward_apply, cp_backward_prepare, cp_backward_apply). The composition
// step that the page's orchestrators (chunkwise_cp_forward / chunkwise_cp_backward)
// perform after gathering summaries runs here as the affine_scan kernel, since on
// one GPU every shard's summary already sits in one buffer. Validation mirrors
// _validate_summary_tensor; the stream divides into shards as torch.chunk does
// (shards.hpp), so uneven divisions are accepted.
#include <atomic>
#include <mutex>
#include <unordered_map>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cpla.h"
#include "errors.hpp"
#include "kernels.hpp"
#include "shards.hpp"

namespace cpla {

static thread_local char g_err[512];
const char* last_error_buf() { return g_err; }
void set_error_v(const char* fmt, va_list ap) { vsnprintf(g_err, sizeof(g_err), fmt, ap); }
void clear_error() { g_err[0] = 0; }

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t m_slot_of(const cpla_problem* p) { return p->decay == CPLA_DECAY_DIAG ? p->dk : 4; }

cpla_status check_problem(const cpla_problem* p) {
  if (!p) return fail(CPLA_E_INVALID, "problem is NULL");
  if (p->B <= 0 || p->T <= 0 || p->H <= 0 || p->dk <= 0 || p->dv <= 0)
    return fail(CPLA_E_SHAPE, "B, T, H, dk, dv must be positive");
  if (p->dtype != CPLA_F32 && p->dtype != CPLA_BF16) return fail(CPLA_E_DTYPE, "unknown dtype %d", p->dtype);
  if (p->decay == CPLA_DECAY_DELTA) return fail(CPLA_E_INVALID, "the delta rule goes through the _delta calls");
  if (p->decay < CPLA_DECAY_NONE || p->decay > CPLA_DECAY_DIAG) return fail(CPLA_E_INVALID, "unknown decay %d", p->decay);
  if (p->chunk != 64) return fail(CPLA_E_UNSUPPORTED, "chunk %d unsupported (64 only)", p->chunk);
  if (p->num_shards <= 0) return fail(CPLA_E_SHAPE, "num_shards must be positive");
  // any T and num_shards: torch.chunk's division (shards.hpp), partial last chunks
  if (p->num_shards > CPLA_MAX_SHARDS)
    return fail(CPLA_E_UNSUPPORTED, "num_shards=%d > %d unsupported", p->num_shards, CPLA_MAX_SHARDS);
  if (p->rank_begin < 0 || p->rank_end > p->num_shards || p->rank_begin >= p->rank_end)
    return fail(CPLA_E_INVALID, "rank range [%d, %d) outside [0, %d)", p->rank_begin, p->rank_end, p->num_shards);
  const bool bf = p->dtype == CPLA_BF16;
  if (p->dk != p->dv) {
    const bool mixed = bf && ((p->dk == 64 && p->dv == 128) || (p->dk == 128 && p->dv == 64));
    if (!mixed)
      return fail(CPLA_E_UNSUPPORTED, "dk=%lld, dv=%lld unsupported for dtype %s (dk != dv: bf16 64/128 or 128/64)",
                  (long long)p->dk, (long long)p->dv, bf ? "bf16" : "fp32");
  } else if (!(p->dk == 16 || p->dk == 64 || (bf && p->dk == 128))) {
    return fail(CPLA_E_UNSUPPORTED, "head dim %lld unsupported for dtype %s (bf16: 16, 64, 128; fp32: 16, 64)",
                (long long)p->dk, bf ? "bf16" : "fp32");
  }
  if (p->B * p->H > 65535) return fail(CPLA_E_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)(p->B * p->H));
  if (p->qk_heads < 0 || (p->qk_heads > 0 && p->H % p->qk_heads != 0))
    return fail(CPLA_E_SHAPE, "qk_heads=%d does not divide H=%lld", p->qk_heads, (long long)p->H);
  if (p->qk_heads > 0 && p->qk_heads != p->H && p->decay != CPLA_DECAY_SCALAR)
    return fail(CPLA_E_UNSUPPORTED, "q and k shared by groups of heads need a scalar decay");
  return CPLA_OK;
}

// heads of q and k (qk_heads 0 means one per head)
int64_t qk_heads_of(const cpla_problem* p) { return p->qk_heads > 0 ? p->qk_heads : p->H; }

cpla_status check_ptr(const void* ptr, const char* name, bool required) {
  if (!ptr) return required ? fail(CPLA_E_INVALID, "%s is NULL", name) : CPLA_OK;
  if (!aligned16(ptr)) return fail(CPLA_E_ALIGN, "%s is not 16-byte aligned", name);
  return CPLA_OK;
}

cpla_status check_packed(const cpla_problem* p, const cpla_packed* pk, bool need_prs, bool need_frs) {
  if (!pk) return CPLA_OK;
  cpla_status st;
  if ((st = check_ptr(pk->seq_idx, "packed->seq_idx", true)) != CPLA_OK) return st;
  if ((st = check_ptr(pk->preceding_rank_start, "packed->preceding_rank_start", need_prs)) != CPLA_OK) return st;
  if ((st = check_ptr(pk->following_rank_stop, "packed->following_rank_stop", need_frs)) != CPLA_OK) return st;
  return CPLA_OK;
}

cpla_status check_decay_ptr(const cpla_problem* p, const float* g, const char* name) {
  if (p->decay == CPLA_DECAY_NONE) {
    if (g) return fail(CPLA_E_INVALID, "%s must be NULL without decay", name);
    return CPLA_OK;
  }
  return check_ptr(g, name, true);
}

cpla_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CPLA_E_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return CPLA_OK;
}

// ---- kernel tables --------------------------------------------------------------
typedef void (*fwd_fn)(FwdArgs);
typedef void (*bwd_fn)(BwdArgs);

// some shard's length is not a multiple of the 64-token chunk
bool needs_tail(const cpla_problem* p) {
  for (int r = 0; r < p->num_shards; ++r)
    if (shard_len(p->T, p->num_shards, r) % 64 != 0) return true;
  return false;
}

// unpacked: the apply walk specialised for a stream without packed sequences
template <typename E, int KK, int VV, int DEC, bool APPLY, bool TAIL>
fwd_fn fwd_kernel(bool split, bool unpacked) {
  if constexpr (APPLY) {
    if (unpacked) return split ? fwd_walk<E, KK, VV, DEC, true, TAIL, true, false>
                               : fwd_walk<E, KK, VV, DEC, true, TAIL, false, false>;
    if (split) return fwd_walk<E, KK, VV, DEC, true, TAIL, true>;
  }
  return fwd_walk<E, KK, VV, DEC, APPLY, TAIL>;
}

template <bool APPLY, bool TAIL>
fwd_fn pick_fwd_t(int dtype, int DK, int DV, int decay, bool split, bool unpacked) {
#define CPLA_FWD_CASE(E, KK, VV)                                                    \
  if (DK == KK && DV == VV) {                                                       \
    if (decay == 0) return fwd_kernel<E, KK, VV, 0, APPLY, TAIL>(split, unpacked);  \
    if (decay == 1) return fwd_kernel<E, KK, VV, 1, APPLY, TAIL>(split, unpacked);  \
    return fwd_kernel<E, KK, VV, 2, APPLY, TAIL>(split, unpacked);                  \
  }
  if (dtype == CPLA_BF16) {
    CPLA_FWD_CASE(bf16_t, 16, 16)
    CPLA_FWD_CASE(bf16_t, 64, 64)
    CPLA_FWD_CASE(bf16_t, 128, 128)
    CPLA_FWD_CASE(bf16_t, 64, 128)
    CPLA_FWD_CASE(bf16_t, 128, 64)
  } else {
    CPLA_FWD_CASE(float, 16, 16)
    CPLA_FWD_CASE(float, 64, 64)
  }
#undef CPLA_FWD_CASE
  return nullptr;
}

// the divided (SPLIT) variants exist for the apply walk without decay or with a scalar decay
template <typename E, int KK, int VV, int DEC, bool APPLY, bool GF, bool TAIL>
bwd_fn bwd_kernel(bool split, bool unpacked) {
  if constexpr (APPLY && DEC != CPLA_DECAY_DIAG)
    if (split) return unpacked ? bwd_walk<E, KK, VV, DEC, true, GF, TAIL, true, false>
                               : bwd_walk<E, KK, VV, DEC, true, GF, TAIL, true>;
  if constexpr (APPLY)
    if (unpacked) return bwd_walk<E, KK, VV, DEC, true, GF, TAIL, false, false>;
  return bwd_walk<E, KK, VV, DEC, APPLY, GF, TAIL>;
}

template <bool APPLY, bool TAIL>
bwd_fn pick_bwd_t(int dtype, int DK, int DV, int decay, bool grad_f32, bool split, bool unpacked) {
  if (grad_f32) {   // fp32 gradients from bf16 inputs: scalar decay only
    if constexpr (!APPLY) return nullptr;
    if (dtype != CPLA_BF16 || decay != CPLA_DECAY_SCALAR) return nullptr;
    if (DK == 16 && DV == 16) return bwd_kernel<bf16_t, 16, 16, 1, true, true, TAIL>(split, unpacked);
    if (DK == 64 && DV == 64) return bwd_kernel<bf16_t, 64, 64, 1, true, true, TAIL>(split, unpacked);
    if (DK == 128 && DV == 128) return bwd_kernel<bf16_t, 128, 128, 1, true, true, TAIL>(split, unpacked);
    if (DK == 64 && DV == 128) return bwd_kernel<bf16_t, 64, 128, 1, true, true, TAIL>(split, unpacked);
    if (DK == 128 && DV == 64) return bwd_kernel<bf16_t, 128, 64, 1, true, true, TAIL>(split, unpacked);
    return nullptr;
  }
#define CPLA_BWD_CASE(E, KK, VV)                                                         \
  if (DK == KK && DV == VV) {                                                            \
    if (decay == 0) return bwd_kernel<E, KK, VV, 0, APPLY, false, TAIL>(split, unpacked); \
    if (decay == 1) return bwd_kernel<E, KK, VV, 1, APPLY, false, TAIL>(split, unpacked); \
    return bwd_kernel<E, KK, VV, 2, APPLY, false, TAIL>(false, unpacked);                \
  }
  if (dtype == CPLA_BF16) {
    CPLA_BWD_CASE(bf16_t, 16, 16)
    CPLA_BWD_CASE(bf16_t, 64, 64)
    CPLA_BWD_CASE(bf16_t, 128, 128)
    CPLA_BWD_CASE(bf16_t, 64, 128)
    CPLA_BWD_CASE(bf16_t, 128, 64)
  } else {
    CPLA_BWD_CASE(float, 16, 16)
    CPLA_BWD_CASE(float, 64, 64)
  }
#undef CPLA_BWD_CASE
  return nullptr;
}

// the kernel for a problem: the TAIL variant only when some shard ends inside a chunk
template <bool APPLY>
fwd_fn pick_fwd(const cpla_problem* p, bool split = false, bool unpacked = false) {
  return needs_tail(p) ? pick_fwd_t<APPLY, true>(p->dtype, (int)p->dk, (int)p->dv, p->decay, split, unpacked)
                       : pick_fwd_t<APPLY, false>(p->dtype, (int)p->dk, (int)p->dv, p->decay, split, unpacked);
}

// Compute units of the current device (queried once per device; 0 if unknown).
int device_cus() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  cache[dev] = n;
  return n;
}

unsigned threads_for(const cpla_problem* p);

// Workgroups of `kernel` (blocks of `threads`) resident per compute unit, from
// the runtime's occupancy query (cached per device and kernel: it depends only
// on the kernel's registers and LDS and on the block size, which the kernel fixes).
int kernel_occupancy(const void* kernel, unsigned threads) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache[dev].find(kernel);
  if (it != cache[dev].end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, (int)threads, 0) != hipSuccess || n < 1) n = 1;
  cache[dev][kernel] = n;
  return n;
}

// Workgroups per shard for an apply walk (divided kernel `kernel`): the largest
// Z in {1, 2, 4} whose Z x (shards x rows) workgroups are all resident at once
// (compute units x workgroups per unit) while no shard gets more parts than
// chunks; each extra part replays the chunks before its own, so a division only
// pays while it fills otherwise idle units.
std::atomic<int> g_forced_parts{0};   // cpla_set_apply_parts: 0 = automatic

unsigned apply_parts(const cpla_problem* p, const void* kernel) {
  const int64_t units = (int64_t)(p->rank_end - p->rank_begin) * p->B * p->H;
  const int64_t nc = chunks_of(shard_len(p->T, p->num_shards, 0));
  const int forced = g_forced_parts.load(std::memory_order_relaxed);
  if (forced > 0) {   // the forced count, halved until every part holds a chunk
    unsigned z = (unsigned)forced;
    while (z > 1 && (int64_t)z > nc) z /= 2;
    return z;
  }
  const int cus = device_cus();
  if (cus <= 0 || !kernel) return 1;
  const int64_t slots = (int64_t)cus * kernel_occupancy(kernel, threads_for(p));
  unsigned z = 1;
  while (z < 4 && 2 * z <= nc && 2 * z * units <= slots) z *= 2;
  return z;
}
template <bool APPLY>
bwd_fn pick_bwd(const cpla_problem* p, bool grad_f32 = false, bool split = false, bool unpacked = false) {
  return needs_tail(p)
             ? pick_bwd_t<APPLY, true>(p->dtype, (int)p->dk, (int)p->dv, p->decay, grad_f32, split, unpacked)
             : pick_bwd_t<APPLY, false>(p->dtype, (int)p->dk, (int)p->dv, p->decay, grad_f32, split, unpacked);
}

unsigned threads_for(const cpla_problem* p) {
  return 64u * (unsigned)waves_for(p->dk < 32 ? 32 : (int)p->dk);
}


cpla_status launch_scan(const cpla_problem* p, const float* summary, const int32_t* slice, const float* init,
                        float* out, float* fin, int reverse, hipStream_t stream) {
  ScanArgs s;
  s.BH = p->B * p->H;
  s.W = cpla_summary_width(p);
  s.dk = (int)p->dk;
  s.dv = (int)p->dv;
  s.H = (int)p->H;
  s.n_elem = s.BH * p->dk * p->dv;
  s.P = p->num_shards;
  s.m_slot = (int)m_slot_of(p);
  s.diag = p->decay == CPLA_DECAY_DIAG;
  s.reverse = reverse;
  s.summary = summary;
  s.slice = slice;
  s.init = init;
  s.out = out;
  s.fin = fin;
  const int64_t blocks = (s.n_elem + 255) / 256;
  hipLaunchKernelGGL(affine_scan, dim3((unsigned)blocks), dim3(256), 0, stream, s);
  return launched("affine_scan");
}

}  // namespace
}  // namespace cpla

using namespace cpla;

extern "C" const char* cpla_last_error(void) { return last_error_buf(); }
extern "C" int cpla_abi_version(void) { return CPLA_ABI_VERSION; }

extern "C" int cpla_set_apply_parts(int parts) {
  if (parts != 0 && parts != 1 && parts != 2 && parts != 4) return -1;
  return cpla::g_forced_parts.exchange(parts);
}

extern "C" int64_t cpla_summary_width(const cpla_problem* p) {
  if (!p) return -1;
  if (p->decay == CPLA_DECAY_DELTA) return p->dk * p->dk + p->dk * p->dv;   // [M | delta_S or gamma]
  return m_slot_of(p) + p->dk * p->dv;
}

extern "C" int64_t cpla_chunk_states_bytes(const cpla_problem* p) {
  if (!p || p->chunk != 64 || p->T <= 0 || p->num_shards <= 0) return -1;
  return p->B * p->H * row_chunks(p->T, p->num_shards) * p->dk * p->dv * (int64_t)sizeof(float);
}

namespace cpla {
namespace {
// The optional per-token input weight w (and its gradient dw) of the scalar decay.
cpla_status check_weight(const cpla_problem* p, const float* w, const float* dw) {
  if (!w && !dw) return CPLA_OK;
  if (p->decay != CPLA_DECAY_SCALAR) return fail(CPLA_E_INVALID, "input weights need a scalar decay");
  if (!w) return fail(CPLA_E_INVALID, "dw needs w");
  return check_ptr(w, "w", true);
}
}  // namespace
}  // namespace cpla

static cpla_status forward_prepare(const cpla_problem* p, const cpla_packed* packed, const void* k,
                                   const void* v, const float* g, const float* w, float* fwd_summary,
                                   hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_problem(p)) != CPLA_OK) return st;
  if ((st = check_weight(p, w, nullptr)) != CPLA_OK) return st;
  if ((st = check_packed(p, packed, false, false)) != CPLA_OK) return st;
  if ((st = check_ptr(k, "k", true)) != CPLA_OK) return st;
  if ((st = check_ptr(v, "v", true)) != CPLA_OK) return st;
  if ((st = check_decay_ptr(p, g, "g")) != CPLA_OK) return st;
  if ((st = check_ptr(fwd_summary, "fwd_summary", true)) != CPLA_OK) return st;
  FwdArgs a = {};
  a.B = p->B; a.T = p->T; a.H = p->H; a.W = cpla_summary_width(p);
  a.Hqk = qk_heads_of(p); a.qk_div = (int)(p->H / a.Hqk);
  a.P = p->num_shards; a.rank_begin = p->rank_begin; a.m_slot = (int)m_slot_of(p);
  a.k = k; a.v = v; a.g = g; a.w = w;
  a.seq_idx = packed ? packed->seq_idx : nullptr;
  a.summary = fwd_summary;
  fwd_fn fn = pick_fwd<false>(p);
  if (!fn) return fail(CPLA_E_UNSUPPORTED, "no forward kernel for this configuration");
  hipLaunchKernelGGL(fn, dim3(p->rank_end - p->rank_begin, (unsigned)(p->B * p->H)), dim3(threads_for(p)), 0, stream, a);
  return launched("cp_forward_prepare");
}

extern "C" cpla_status cp_forward_prepare(const cpla_problem* p, const cpla_packed* packed, const void* k,
                                          const void* v, const float* g, float* fwd_summary, hipStream_t stream) {
  return forward_prepare(p, packed, k, v, g, nullptr, fwd_summary, stream);
}

extern "C" cpla_status cp_forward_prepare_weighted(const cpla_problem* p, const cpla_packed* packed, const void* k,
                                                   const void* v, const float* g, const float* w,
                                                   float* fwd_summary, hipStream_t stream) {
  return forward_prepare(p, packed, k, v, g, w, fwd_summary, stream);
}

static cpla_status forward_apply(const cpla_problem* p, const cpla_packed* packed, const void* q, const void* k,
                                 const void* v, const float* g, const float* w, const float* fwd_summary,
                                 const float* initial_state, void* o, float* shard_in_state, float* final_state,
                                 void* chunk_states, hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_problem(p)) != CPLA_OK) return st;
  if ((st = check_weight(p, w, nullptr)) != CPLA_OK) return st;
  if ((st = check_packed(p, packed, true, false)) != CPLA_OK) return st;
  if ((st = check_ptr(q, "q", true)) != CPLA_OK) return st;
  if ((st = check_ptr(k, "k", true)) != CPLA_OK) return st;
  if ((st = check_ptr(v, "v", true)) != CPLA_OK) return st;
  if ((st = check_decay_ptr(p, g, "g")) != CPLA_OK) return st;
  if ((st = check_ptr(fwd_summary, "fwd_summary", true)) != CPLA_OK) return st;
  if ((st = check_ptr(initial_state, "initial_state", false)) != CPLA_OK) return st;
  if ((st = check_ptr(o, "o", true)) != CPLA_OK) return st;
  if ((st = check_ptr(shard_in_state, "shard_in_state", true)) != CPLA_OK) return st;
  if ((st = check_ptr(final_state, "final_state", false)) != CPLA_OK) return st;
  if ((st = check_ptr(chunk_states, "chunk_states", false)) != CPLA_OK) return st;
  if (packed && initial_state) return fail(CPLA_E_INVALID, "initial_state must be NULL with packed sequences");
  st = launch_scan(p, fwd_summary, packed ? packed->preceding_rank_start : nullptr, initial_state, shard_in_state,
                   final_state, 0, stream);
  if (st != CPLA_OK) return st;
  FwdArgs a = {};
  a.B = p->B; a.T = p->T; a.H = p->H; a.W = cpla_summary_width(p);
  a.Hqk = qk_heads_of(p); a.qk_div = (int)(p->H / a.Hqk);
  a.P = p->num_shards; a.rank_begin = p->rank_begin; a.m_slot = (int)m_slot_of(p);
  a.q = q; a.k = k; a.v = v; a.g = g; a.w = w;
  a.seq_idx = packed ? packed->seq_idx : nullptr;
  a.state_in = shard_in_state;
  a.out = o;
  a.chunk_states = reinterpret_cast<float*>(chunk_states);
  const bool unpacked = packed == nullptr;
  const unsigned parts = apply_parts(p, reinterpret_cast<const void*>(pick_fwd<true>(p, true, unpacked)));
  fwd_fn fn = pick_fwd<true>(p, parts > 1, unpacked);
  if (!fn) return fail(CPLA_E_UNSUPPORTED, "no forward kernel for this configuration");
  hipLaunchKernelGGL(fn, dim3(p->rank_end - p->rank_begin, (unsigned)(p->B * p->H), parts), dim3(threads_for(p)), 0,
                     stream, a);
  return launched("cp_forward_apply");
}

extern "C" cpla_status cp_forward_apply(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                        const void* k, const void* v, const float* g, const float* fwd_summary,
                                        const float* initial_state, void* o, float* shard_in_state,
                                        float* final_state, void* chunk_states, hipStream_t stream) {
  return forward_apply(p, packed, q, k, v, g, nullptr, fwd_summary, initial_state, o, shard_in_state, final_state,
                       chunk_states, stream);
}

// ---- cp_forward_apply without allocation --------------------------------------------
// The composed incoming states of every shard ([P, B, H, dk, dv] fp32: written by
// the prefix scan, read by the shard walks of the same call) live in this
// file-scope device array instead of a caller buffer: one copy per GPU, held
// until the process ends. In host code the array's name is not a device address;
// the address comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in noalloc_ptr below.
constexpr int64_t NOALLOC_SCRATCH_BYTES = int64_t(32) << 20;
static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_BYTES / 4];

namespace {
// Device address of `scratch` on the current device (nullptr and an error set on failure).
float* noalloc_ptr() {
  static std::mutex mu;
  static float* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    fail(CPLA_E_HIP, "cp_forward_apply_noalloc: no current device (or device index >= 64)");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(CPLA_E_HIP, "cp_forward_apply_noalloc: hipGetSymbolAddress of the scratch failed: %s",
           hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = static_cast<float*>(ptr);
  }
  return ptrs[dev];
}
}  // namespace

extern "C" int64_t cpla_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

extern "C" cpla_status cpla_check_decay_range(const cpla_problem* p, const float* g, int32_t* count,
                                              hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_problem(p)) != CPLA_OK) return st;
  if (p->decay != CPLA_DECAY_DIAG) return CPLA_OK;   // scalar decays are applied without a factorisation
  if ((st = check_ptr(g, "g", true)) != CPLA_OK) return st;
  if ((st = check_ptr(count, "count", true)) != CPLA_OK) return st;
  const int64_t cps = chunks_of(shard_size(p->T, p->num_shards));
  DecayCheckArgs a = {};
  a.B = p->B; a.T = p->T; a.H = p->H; a.dk = p->dk;
  a.nchunks = (int64_t)(p->rank_end - p->rank_begin) * cps;
  a.n = a.B * a.H * a.nchunks * a.dk;
  a.P = p->num_shards; a.rank_begin = p->rank_begin;
  a.limit = CPLA_DIAG_GAMMA_MIN;
  a.g = g;
  a.count = count;
  hipLaunchKernelGGL(decay_check_zero, dim3(1), dim3(1), 0, stream, count);
  if ((st = launched("decay_check_zero")) != CPLA_OK) return st;
  hipLaunchKernelGGL(decay_range, dim3((unsigned)((a.n + 255) / 256)), dim3(256), 0, stream, a);
  if ((st = launched("decay_range")) != CPLA_OK) return st;
  int32_t host = 0;
  hipError_t e = hipMemcpyAsync(&host, count, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(CPLA_E_HIP, "cpla_check_decay_range: %s", hipGetErrorString(e));
  if (host > 0)
    return fail(CPLA_E_INVALID,
                "diagonal decay out of range: in %d (chunk, key dim) pairs the running log-decay of a 64-token "
                "chunk falls below %.0f, where the factorised decay exp(+-sum) leaves fp32",
                host, (double)CPLA_DIAG_GAMMA_MIN);
  return CPLA_OK;
}

extern "C" cpla_status cp_forward_apply_noalloc(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                                const void* k, const void* v, const float* g,
                                                const float* fwd_summary, const float* initial_state, void* o,
                                                float* final_state, void* chunk_states, hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_problem(p)) != CPLA_OK) return st;
  const int64_t need = (int64_t)p->num_shards * p->B * p->H * p->dk * p->dv * (int64_t)sizeof(float);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(CPLA_E_UNSUPPORTED,
                "cp_forward_apply_noalloc: the composed states of %d shards x %lld rows need %lld bytes; "
                "its scratch holds %lld (use cp_forward_apply)",
                p->num_shards, (long long)(p->B * p->H), (long long)need, (long long)NOALLOC_SCRATCH_BYTES);
  float* const ptr = noalloc_ptr();
  if (!ptr) return CPLA_E_HIP;
  return forward_apply(p, packed, q, k, v, g, nullptr, fwd_summary, initial_state, o, ptr, final_state,
                       chunk_states, stream);
}

extern "C" cpla_status cp_forward_apply_weighted(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                                 const void* k, const void* v, const float* g, const float* w,
                                                 const float* fwd_summary, const float* initial_state, void* o,
                                                 float* shard_in_state, float* final_state, void* chunk_states,
                                                 hipStream_t stream) {
  return forward_apply(p, packed, q, k, v, g, w, fwd_summary, initial_state, o, shard_in_state, final_state,
                       chunk_states, stream);
}

extern "C" cpla_status cp_backward_prepare(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                           const float* g, const void* dO, float* bwd_summary, hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_problem(p)) != CPLA_OK) return st;
  if ((st = check_packed(p, packed, false, false)) != CPLA_OK) return st;
  if ((st = check_ptr(q, "q", true)) != CPLA_OK) return st;
  if ((st = check_decay_ptr(p, g, "g")) != CPLA_OK) return st;
  if ((st = check_ptr(dO, "dO", true)) != CPLA_OK) return st;
  if ((st = check_ptr(bwd_summary, "bwd_summary", true)) != CPLA_OK) return st;
  BwdArgs a = {};
  a.B = p->B; a.T = p->T; a.H = p->H; a.W = cpla_summary_width(p);
  a.Hqk = qk_heads_of(p); a.qk_div = (int)(p->H / a.Hqk);
  a.P = p->num_shards; a.rank_begin = p->rank_begin; a.m_slot = (int)m_slot_of(p);
  a.q = q; a.g = g; a.dO = dO;
  a.seq_idx = packed ? packed->seq_idx : nullptr;
  a.summary = bwd_summary;
  bwd_fn fn = pick_bwd<false>(p);
  if (!fn) return fail(CPLA_E_UNSUPPORTED, "no backward kernel for this configuration");
  hipLaunchKernelGGL(fn, dim3(p->rank_end - p->rank_begin, (unsigned)(p->B * p->H)), dim3(threads_for(p)), 0, stream, a);
  return launched("cp_backward_prepare");
}

static cpla_status backward_apply(const cpla_problem* p, const cpla_packed* packed, const void* q, const void* k,
                                  const void* v, const float* g, const float* w, const void* dO,
                                  const void* chunk_states, const float* bwd_summary, const float* d_final_state,
                                  void* dq, void* dk, void* dv, float* dg, float* dw, float* shard_out_grad,
                                  float* d_initial_state, int32_t grad_dtype, hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_problem(p)) != CPLA_OK) return st;
  if (grad_dtype != p->dtype && grad_dtype != CPLA_F32)
    return fail(CPLA_E_DTYPE, "grad_dtype must be the input dtype or CPLA_F32");
  const bool grad_f32 = grad_dtype != p->dtype;
  if ((st = check_weight(p, w, dw)) != CPLA_OK) return st;
  if ((st = check_ptr(dw, "dw", false)) != CPLA_OK) return st;
  if ((st = check_packed(p, packed, false, true)) != CPLA_OK) return st;
  if ((st = check_ptr(q, "q", true)) != CPLA_OK) return st;
  if ((st = check_ptr(k, "k", true)) != CPLA_OK) return st;
  if ((st = check_ptr(v, "v", true)) != CPLA_OK) return st;
  if ((st = check_decay_ptr(p, g, "g")) != CPLA_OK) return st;
  if ((st = check_ptr(dO, "dO", true)) != CPLA_OK) return st;
  if ((st = check_ptr(chunk_states, "chunk_states", true)) != CPLA_OK) return st;
  if ((st = check_ptr(bwd_summary, "bwd_summary", true)) != CPLA_OK) return st;
  if ((st = check_ptr(d_final_state, "d_final_state", false)) != CPLA_OK) return st;
  if ((st = check_ptr(dq, "dq", true)) != CPLA_OK) return st;
  if ((st = check_ptr(dk, "dk", true)) != CPLA_OK) return st;
  if ((st = check_ptr(dv, "dv", true)) != CPLA_OK) return st;
  if ((st = check_decay_ptr(p, dg, "dg")) != CPLA_OK) return st;
  if ((st = check_ptr(shard_out_grad, "shard_out_grad", true)) != CPLA_OK) return st;
  if ((st = check_ptr(d_initial_state, "d_initial_state", false)) != CPLA_OK) return st;
  if (packed && (d_final_state || d_initial_state))
    return fail(CPLA_E_INVALID, "d_final_state and d_initial_state must be NULL with packed sequences");
  st = launch_scan(p, bwd_summary, packed ? packed->following_rank_stop : nullptr, d_final_state, shard_out_grad,
                   d_initial_state, 1, stream);
  if (st != CPLA_OK) return st;
  BwdArgs a = {};
  a.B = p->B; a.T = p->T; a.H = p->H; a.W = cpla_summary_width(p);
  a.Hqk = qk_heads_of(p); a.qk_div = (int)(p->H / a.Hqk);
  a.P = p->num_shards; a.rank_begin = p->rank_begin; a.m_slot = (int)m_slot_of(p);
  a.q = q; a.k = k; a.v = v; a.g = g; a.w = w; a.dO = dO;
  a.seq_idx = packed ? packed->seq_idx : nullptr;
  a.chunk_states = reinterpret_cast<const float*>(chunk_states);
  a.grad_in = shard_out_grad;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dw = dw;
  // divided walks for small grids (no decay or a scalar decay)
  const unsigned parts =
      p->decay == CPLA_DECAY_DIAG ? 1u
                                  : apply_parts(p, reinterpret_cast<const void*>(
                                                       pick_bwd<true>(p, grad_f32, true, packed == nullptr)));
  bwd_fn fn = pick_bwd<true>(p, grad_f32, parts > 1, packed == nullptr);
  if (!fn) return fail(CPLA_E_UNSUPPORTED, "no backward kernel for this configuration");
  hipLaunchKernelGGL(fn, dim3(p->rank_end - p->rank_begin, (unsigned)(p->B * p->H), parts), dim3(threads_for(p)), 0,
                     stream, a);
  return launched("cp_backward_apply");
}

extern "C" cpla_status cp_backward_apply(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                         const void* k, const void* v, const float* g, const void* dO,
                                         const void* chunk_states, const float* bwd_summary,
                                         const float* d_final_state, void* dq, void* dk, void* dv, float* dg,
                                         float* shard_out_grad, float* d_initial_state, hipStream_t stream) {
  return backward_apply(p, packed, q, k, v, g, nullptr, dO, chunk_states, bwd_summary, d_final_state, dq, dk, dv,
                        dg, nullptr, shard_out_grad, d_initial_state, p ? p->dtype : 0, stream);
}

extern "C" cpla_status cp_backward_apply_weighted(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                                  const void* k, const void* v, const float* g, const float* w,
                                                  const void* dO, const void* chunk_states,
                                                  const float* bwd_summary, const float* d_final_state, void* dq,
                                                  void* dk, void* dv, float* dg, float* dw,
                                                  float* shard_out_grad, float* d_initial_state,
                                                  int32_t grad_dtype, hipStream_t stream) {
  return backward_apply(p, packed, q, k, v, g, w, dO, chunk_states, bwd_summary, d_final_state, dq, dk, dv, dg, dw,
                        shard_out_grad, d_initial_state, grad_dtype, stream);
}

// ---- the gated delta rule (dense transition) ------------------------------------------------
namespace cpla {
namespace {

cpla_status check_delta(const cpla_problem* p) {
  if (!p) return fail(CPLA_E_INVALID, "problem is NULL");
  if (p->B <= 0 || p->T <= 0 || p->H <= 0 || p->dk <= 0 || p->dv <= 0)
    return fail(CPLA_E_SHAPE, "B, T, H, dk, dv must be positive");
  if (p->dtype != CPLA_F32 && p->dtype != CPLA_BF16) return fail(CPLA_E_DTYPE, "unknown dtype %d", p->dtype);
  if (p->decay != CPLA_DECAY_DELTA) return fail(CPLA_E_INVALID, "the _delta calls need decay CPLA_DECAY_DELTA");
  if (p->chunk != 64) return fail(CPLA_E_UNSUPPORTED, "chunk %d unsupported (64 only)", p->chunk);
  if (p->num_shards <= 0) return fail(CPLA_E_SHAPE, "num_shards must be positive");
  if (p->num_shards > CPLA_MAX_SHARDS)
    return fail(CPLA_E_UNSUPPORTED, "num_shards=%d > %d unsupported", p->num_shards, CPLA_MAX_SHARDS);
  if (p->rank_begin < 0 || p->rank_end > p->num_shards || p->rank_begin >= p->rank_end)
    return fail(CPLA_E_INVALID, "rank range [%d, %d) outside [0, %d)", p->rank_begin, p->rank_end, p->num_shards);
  if (p->dk != p->dv) return fail(CPLA_E_UNSUPPORTED, "dk != dv unsupported");
  if (p->qk_heads != 0 && p->qk_heads != p->H)
    return fail(CPLA_E_UNSUPPORTED, "qk_heads=%d: the delta rule takes q and k per head", p->qk_heads);
  if (!(p->dk == 16 || p->dk == 32 || p->dk == 64 || (p->dk == 128 && p->dtype == CPLA_BF16)))
    return fail(CPLA_E_UNSUPPORTED, "head dim %lld unsupported for the delta rule (16, 32, 64; 128 for bf16)",
                (long long)p->dk);
  if (p->B * p->H > 65535) return fail(CPLA_E_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)(p->B * p->H));
  return CPLA_OK;
}

// workspace: U~, W, U, dU [B,T,H,D] then the chunk states and chunk-end gradients
// [B,H,row_chunks,D,D], all fp32
int64_t delta_ws_floats(const cpla_problem* p) {
  const int64_t tok = p->B * p->T * p->H * p->dk, ch = p->B * p->H * row_chunks(p->T, p->num_shards) * p->dk * p->dk;
  return 4 * tok + 2 * ch;
}

void bind_ws(const cpla_problem* p, void* ws, DeltaArgs& a) {
  const int64_t tok = p->B * p->T * p->H * p->dk, ch = p->B * p->H * row_chunks(p->T, p->num_shards) * p->dk * p->dk;
  float* f = static_cast<float*>(ws);
  a.ws_ut = f;
  a.ws_w = f + tok;
  a.ws_u = f + 2 * tok;
  a.ws_du = f + 3 * tok;
  a.chunk_states = f + 4 * tok;
  a.ws_dsc = f + 4 * tok + ch;
}

DeltaArgs delta_args(const cpla_problem* p, const cpla_packed* packed, void* ws) {
  DeltaArgs a = {};
  a.B = p->B; a.T = p->T; a.H = p->H;
  a.P = p->num_shards; a.rank_begin = p->rank_begin;
  const int64_t nsc = chunks_of(shard_size(p->T, p->num_shards));
  a.chunk_begin = p->rank_begin * nsc;
  a.seq_idx = packed ? packed->seq_idx : nullptr;
  bind_ws(p, ws, a);
  return a;
}

// chunks of the launch's ranks (row-local indices [chunk_begin, chunk_end))
unsigned delta_chunks(const cpla_problem* p) {
  const int64_t nsc = chunks_of(shard_size(p->T, p->num_shards));
  int64_t end = (int64_t)p->rank_end * nsc;
  const int64_t nct = row_chunks(p->T, p->num_shards);
  if (end > nct) end = nct;
  const int64_t beg = (int64_t)p->rank_begin * nsc;
  return (unsigned)(end > beg ? end - beg : 0);
}

enum DeltaPhase { DP_FWD_PREPARE, DP_FWD_APPLY_WALK, DP_FWD_OUT, DP_BWD_PREPARE, DP_BWD_APPLY_WALK, DP_BWD_GRAD };

template <typename E, int D>
void delta_launch(DeltaPhase ph, const cpla_problem* p, const DeltaArgs& a, hipStream_t stream) {
  const unsigned nr = p->rank_end - p->rank_begin, bh = (unsigned)(p->B * p->H), nch = delta_chunks(p);
  const dim3 nt(DELTA_THREADS);
  switch (ph) {
    case DP_FWD_PREPARE:
      if (nch) hipLaunchKernelGGL((delta_wy<E, D>), dim3(nch, bh), nt, 0, stream, a);
      hipLaunchKernelGGL((delta_fwalk<E, D, false>),
                         dim3(nr, bh, FwalkSlab<D, false>::NZ / FwalkSlab<D, false>::SZ), nt, 0, stream, a);
      break;
    case DP_FWD_APPLY_WALK:
      hipLaunchKernelGGL((delta_fwalk<E, D, true>),
                         dim3(nr, bh, FwalkSlab<D, true>::NZ / FwalkSlab<D, true>::SZ), nt, 0, stream, a);
      break;
    case DP_FWD_OUT:
      // the half-width bf16 apply walk (D = 64) has written o itself
      if constexpr (!(FwalkSlab<D, true>::HALF && sizeof(E) == 2))
        if (nch) hipLaunchKernelGGL((delta_out<E, D>), dim3(nch, bh, D / DeltaSlabs<D>::OUT), nt, 0, stream, a);
      break;
    case DP_BWD_PREPARE:
      hipLaunchKernelGGL((delta_bwalk<E, D, false>), dim3(nr, bh, D / DeltaSlabs<D>::BWALK), nt, 0, stream, a);
      break;
    case DP_BWD_APPLY_WALK:
      hipLaunchKernelGGL((delta_bwalk<E, D, true>), dim3(nr, bh, D / DeltaSlabs<D>::BWALK), nt, 0, stream, a);
      break;
    case DP_BWD_GRAD:
      if (nch) {
        // value slices: needed at D = 128, two workgroups per CU at D = 32, 64
        if constexpr (D >= 32)
          hipLaunchKernelGGL((delta_grad_wide<E, D>), dim3(nch, bh), nt, 0, stream, a);
        else hipLaunchKernelGGL((delta_grad<E, D>), dim3(nch, bh), nt, 0, stream, a);
      }
      break;
  }
}

template <typename E>
void delta_launch_d(DeltaPhase ph, const cpla_problem* p, const DeltaArgs& a, hipStream_t stream) {
  if (p->dk == 16) delta_launch<E, 16>(ph, p, a, stream);
  else if (p->dk == 32) delta_launch<E, 32>(ph, p, a, stream);
  else if (p->dk == 64) delta_launch<E, 64>(ph, p, a, stream);
  else if constexpr (sizeof(E) == 2) delta_launch<E, 128>(ph, p, a, stream);   // 128: bf16 only (checked)
}

cpla_status delta_run(DeltaPhase ph, const cpla_problem* p, const DeltaArgs& a, hipStream_t stream, const char* what) {
  if (p->dtype == CPLA_BF16) delta_launch_d<bf16_t>(ph, p, a, stream);
  else delta_launch_d<float>(ph, p, a, stream);
  return launched(what);
}

// one workgroup per (b, h) and slab of the state's columns
template <int D>
void delta_scan_launch(const DeltaScanArgs& s, hipStream_t stream) {
  hipLaunchKernelGGL(delta_scan<D>, dim3((unsigned)s.BH, D / DeltaSlabs<D>::SCAN), dim3(DELTA_THREADS), 0, stream, s);
}

cpla_status delta_scan_run(const cpla_problem* p, const float* summary, const int32_t* slice, const float* init,
                           float* out, float* fin, int reverse, hipStream_t stream) {
  DeltaScanArgs s = {};
  s.BH = p->B * p->H;
  s.H = p->H;
  s.P = p->num_shards;
  s.reverse = reverse;
  s.summary = summary;
  s.slice = slice;
  s.init = init;
  s.out = out;
  s.fin = fin;
  if (p->dk == 16) delta_scan_launch<16>(s, stream);
  else if (p->dk == 32) delta_scan_launch<32>(s, stream);
  else if (p->dk == 64) delta_scan_launch<64>(s, stream);
  else delta_scan_launch<128>(s, stream);
  return launched("delta_scan");
}

}  // namespace
}  // namespace cpla

extern "C" int64_t cpla_delta_workspace_bytes(const cpla_problem* p) {
  if (check_delta(p) != CPLA_OK) return -1;
  return delta_ws_floats(p) * (int64_t)sizeof(float);
}

extern "C" cpla_status cp_forward_prepare_delta(const cpla_problem* p, const cpla_packed* packed, const void* k,
                                                const void* v, const float* g, const float* beta,
                                                float* fwd_summary, void* workspace, hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_delta(p)) != CPLA_OK) return st;
  if ((st = check_packed(p, packed, false, false)) != CPLA_OK) return st;
  if ((st = check_ptr(k, "k", true)) != CPLA_OK) return st;
  if ((st = check_ptr(v, "v", true)) != CPLA_OK) return st;
  if ((st = check_ptr(g, "g", true)) != CPLA_OK) return st;
  if ((st = check_ptr(beta, "beta", true)) != CPLA_OK) return st;
  if ((st = check_ptr(fwd_summary, "fwd_summary", true)) != CPLA_OK) return st;
  if ((st = check_ptr(workspace, "workspace", true)) != CPLA_OK) return st;
  DeltaArgs a = delta_args(p, packed, workspace);
  a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.summary = fwd_summary;
  return delta_run(DP_FWD_PREPARE, p, a, stream, "cp_forward_prepare_delta");
}

extern "C" cpla_status cp_forward_apply_delta(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                              const void* k, const void* v, const float* g, const float* beta,
                                              const float* fwd_summary, const float* initial_state, void* o,
                                              float* shard_in_state, float* final_state, void* workspace,
                                              hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_delta(p)) != CPLA_OK) return st;
  if ((st = check_packed(p, packed, true, false)) != CPLA_OK) return st;
  const void* req[] = {q, k, v, g, beta, fwd_summary, o, shard_in_state, workspace};
  const char* names[] = {"q", "k", "v", "g", "beta", "fwd_summary", "o", "shard_in_state", "workspace"};
  for (int i = 0; i < 9; ++i)
    if ((st = check_ptr(req[i], names[i], true)) != CPLA_OK) return st;
  if ((st = check_ptr(initial_state, "initial_state", false)) != CPLA_OK) return st;
  if ((st = check_ptr(final_state, "final_state", false)) != CPLA_OK) return st;
  if (packed && initial_state) return fail(CPLA_E_INVALID, "initial_state must be NULL with packed sequences");
  st = delta_scan_run(p, fwd_summary, packed ? packed->preceding_rank_start : nullptr, initial_state, shard_in_state,
                      final_state, 0, stream);
  if (st != CPLA_OK) return st;
  DeltaArgs a = delta_args(p, packed, workspace);
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.state_in = shard_in_state;
  a.out = o;
  if ((st = delta_run(DP_FWD_APPLY_WALK, p, a, stream, "cp_forward_apply_delta (walk)")) != CPLA_OK) return st;
  return delta_run(DP_FWD_OUT, p, a, stream, "cp_forward_apply_delta (output)");
}

extern "C" cpla_status cp_backward_prepare_delta(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                                 const void* k, const float* g, const float* beta, const void* dO,
                                                 const float* fwd_summary, float* bwd_summary, void* workspace,
                                                 hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_delta(p)) != CPLA_OK) return st;
  if ((st = check_packed(p, packed, false, false)) != CPLA_OK) return st;
  const void* req[] = {q, k, g, beta, dO, fwd_summary, bwd_summary, workspace};
  const char* names[] = {"q", "k", "g", "beta", "dO", "fwd_summary", "bwd_summary", "workspace"};
  for (int i = 0; i < 8; ++i)
    if ((st = check_ptr(req[i], names[i], true)) != CPLA_OK) return st;
  DeltaArgs a = delta_args(p, packed, workspace);
  a.q = q; a.k = k; a.g = g; a.beta = beta; a.dO = dO;
  a.fwd_summary = fwd_summary;
  a.summary = bwd_summary;
  return delta_run(DP_BWD_PREPARE, p, a, stream, "cp_backward_prepare_delta");
}

extern "C" cpla_status cp_backward_apply_delta(const cpla_problem* p, const cpla_packed* packed, const void* q,
                                               const void* k, const void* v, const float* g, const float* beta,
                                               const void* dO, const float* bwd_summary,
                                               const float* d_final_state, void* dq, void* dk, void* dv, float* dg,
                                               float* dbeta, float* shard_out_grad, float* d_initial_state,
                                               void* workspace, hipStream_t stream) {
  clear_error();
  cpla_status st;
  if ((st = check_delta(p)) != CPLA_OK) return st;
  if ((st = check_packed(p, packed, false, true)) != CPLA_OK) return st;
  const void* req[] = {q, k, v, g, beta, dO, bwd_summary, dq, dk, dv, dg, dbeta, shard_out_grad, workspace};
  const char* names[] = {"q", "k", "v", "g", "beta", "dO", "bwd_summary", "dq", "dk", "dv", "dg", "dbeta",
                         "shard_out_grad", "workspace"};
  for (int i = 0; i < 14; ++i)
    if ((st = check_ptr(req[i], names[i], true)) != CPLA_OK) return st;
  if ((st = check_ptr(d_final_state, "d_final_state", false)) != CPLA_OK) return st;
  if ((st = check_ptr(d_initial_state, "d_initial_state", false)) != CPLA_OK) return st;
  if (packed && (d_final_state || d_initial_state))
    return fail(CPLA_E_INVALID, "d_final_state and d_initial_state must be NULL with packed sequences");
  st = delta_scan_run(p, bwd_summary, packed ? packed->following_rank_stop : nullptr, d_final_state, shard_out_grad,
                      d_initial_state, 1, stream);
  if (st != CPLA_OK) return st;
  DeltaArgs a = delta_args(p, packed, workspace);
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.dO = dO;
  a.state_in = shard_out_grad;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta;
  if ((st = delta_run(DP_BWD_APPLY_WALK, p, a, stream, "cp_backward_apply_delta (walk)")) != CPLA_OK) return st;
  return delta_run(DP_BWD_GRAD, p, a, stream, "cp_backward_apply_delta (gradients)");
}
