// Mamba2 (SSD) parametrisation of the scalar-decay path, and its C-ABI calls.
//
// The axolotl-ringmaster README lists Mamba2 SSM context parallelism beside
// linear-attention state passing (Status table; Layout: state_passing.py, an
// exact CP linear scan shared by Mamba2 and linear attention), and the chunkwise
// interfaces of the Megatron-Core page core.ssm.context_parallel.chunkwise are
// those of its SSM module. Mamba2's selective state space (state h [N x P] per
// head, per-token decay exp(dt A_h), input dt B x^T, output h^T C, with B and C
// shared by the heads of a group) is this library's weighted scalar-decay
// recurrence
//   S_t = exp(g_t) S_{t-1} + w_t k_t v_t^T,   o_t = S_t^T q_t
// under the map, for head h of group gr = h / (H / G):
//   q[b,t,h,:] = C[b,t,gr,:]   k[b,t,h,:] = B[b,t,gr,:]   v = x   w = dt   g[b,t,h] = A[h] dt[b,t,h]
// (dt enters as the fp32 weight, so nothing is rounded on the way in).
// ssd_inputs writes g (and, if asked, per-head copies q, k; the walks can read B
// and C in place through the problem's qk_heads = G); ssd_grads and ssd_dA take
// the fp32 gradients of the weighted backward (dq, dk, dv, dg, dw) back to x, dt,
// A, B and C:
//   dx = dv,   d_dt = dw + A dg,   dA_h = sum_{b,t} dt dg,
//   dB[gr] = sum_{h in gr} dk,   dC[gr] = sum_{h in gr} dq
// (the head sums in fp32, each output rounded once).
// All three are elementwise / reduction passes bound by HBM bandwidth; every
// thread moves four features (one 8-byte bf16 or 16-byte fp32 vector).
#include <stdint.h>

#include "cpla.h"
#include "errors.hpp"
#include "kernels.hpp"

namespace cpla {

struct SsdArgs {
  int64_t B, T, H, G, N, P;
  const float* dt;
  const float* A;
  const void* Bm;
  const void* Cm;
  void* q;
  void* k;
  float* g;
  const float* dq;
  const float* dk;
  const float* dv;
  const float* dg;
  const float* dw;
  void* dx;
  float* ddt;
  float* dA;
  void* dB;
  void* dC;
};

namespace {

__device__ __forceinline__ f32x4 ld4(const bf16_t* p) {
  const bf16x4 y = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(bf16_t* p, const f32x4& x) {
  bf16x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (bf16_t)x[e];
  *reinterpret_cast<bf16x4*>(p) = y;
}
__device__ __forceinline__ void st4(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ void cp4(bf16_t* d, const bf16_t* s) {
  *reinterpret_cast<bf16x4*>(d) = *reinterpret_cast<const bf16x4*>(s);
}
__device__ __forceinline__ void cp4(float* d, const float* s) {
  *reinterpret_cast<f32x4*>(d) = *reinterpret_cast<const f32x4*>(s);
}

// One thread per (b, t, h): g only (the walks read B and C in place).
__global__ __launch_bounds__(256) void ssd_decay(SsdArgs a) {
  const int64_t bth = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (bth >= a.B * a.T * a.H) return;
  a.g[bth] = a.A[bth % a.H] * a.dt[bth];
}

// One thread per (b, t, h, four features): g and the per-head copies of B and C.
template <typename E>
__global__ __launch_bounds__(256) void ssd_inputs(SsdArgs a) {
  const int64_t nv = a.N / 4;
  const int64_t total = a.B * a.T * a.H * nv;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t bth = i / nv, f = (i % nv) * 4;
  const int64_t h = bth % a.H, bt = bth / a.H;
  const int64_t gr = h / (a.H / a.G);
  const int64_t src = (bt * a.G + gr) * a.N + f, dst = bth * a.N + f;
  cp4(reinterpret_cast<E*>(a.q) + dst, reinterpret_cast<const E*>(a.Cm) + src);
  cp4(reinterpret_cast<E*>(a.k) + dst, reinterpret_cast<const E*>(a.Bm) + src);
  if (f == 0) a.g[bth] = a.A[h] * a.dt[bth];
}

// One thread per (b, t, group, four features f of max(N, P)): the group's dB and
// dC rows (f < N), its heads' dx (f < P), and their d_dt (from the thread
// holding features 0..3).
template <typename E>
__global__ __launch_bounds__(256) void ssd_grads(SsdArgs a) {
  const int64_t nv = (a.N > a.P ? a.N : a.P) / 4;
  const int64_t total = a.B * a.T * a.G * nv;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t btg = i / nv, f = (i % nv) * 4;
  const int64_t gr = btg % a.G, bt = btg / a.G;
  const int64_t hpg = a.H / a.G;
  const bool in_n = f < a.N, in_p = f < a.P;
  f32x4 sb = {0.f, 0.f, 0.f, 0.f}, sc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t j = 0; j < hpg; ++j) {
    const int64_t h = gr * hpg + j, bth = bt * a.H + h;
    if (in_n) {
      sb += ld4(a.dk + bth * a.N + f);
      sc += ld4(a.dq + bth * a.N + f);
    }
    if (in_p) st4(reinterpret_cast<E*>(a.dx) + bth * a.P + f, ld4(a.dv + bth * a.P + f));
    if (f == 0) a.ddt[bth] = a.dw[bth] + a.A[h] * a.dg[bth];
  }
  if (in_n) {
    const int64_t off = btg * a.N + f;
    st4(reinterpret_cast<E*>(a.dB) + off, sb);
    st4(reinterpret_cast<E*>(a.dC) + off, sc);
  }
}

// One workgroup per head: dA_h = sum over (b, t) of dt * dg in a fixed order
// (four strided partial sums per thread, so their loads are in flight together,
// then a tree), so the result is the same on every run.
constexpr int DA_THREADS = 1024;
__global__ __launch_bounds__(DA_THREADS) void ssd_dA(SsdArgs a) {
  __shared__ float red[DA_THREADS];
  const int64_t h = blockIdx.x, n = a.B * a.T;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int64_t bt = threadIdx.x;
  for (; bt + 3 * DA_THREADS < n; bt += 4 * DA_THREADS) {
    s0 += a.dt[bt * a.H + h] * a.dg[bt * a.H + h];
    s1 += a.dt[(bt + DA_THREADS) * a.H + h] * a.dg[(bt + DA_THREADS) * a.H + h];
    s2 += a.dt[(bt + 2 * DA_THREADS) * a.H + h] * a.dg[(bt + 2 * DA_THREADS) * a.H + h];
    s3 += a.dt[(bt + 3 * DA_THREADS) * a.H + h] * a.dg[(bt + 3 * DA_THREADS) * a.H + h];
  }
  for (; bt < n; bt += DA_THREADS) s0 += a.dt[bt * a.H + h] * a.dg[bt * a.H + h];
  red[threadIdx.x] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  for (int w = DA_THREADS / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dA[h] = red[0];
}

cpla_status check_ssd(const cpla_ssd_problem* p) {
  if (!p) return fail(CPLA_E_INVALID, "problem is NULL");
  if (p->B <= 0 || p->T <= 0 || p->H <= 0 || p->G <= 0 || p->N <= 0)
    return fail(CPLA_E_SHAPE, "B, T, H, G, N must be positive");
  if (p->H % p->G != 0) return fail(CPLA_E_SHAPE, "H=%lld is not a multiple of G=%lld", (long long)p->H, (long long)p->G);
  if (p->dtype != CPLA_F32 && p->dtype != CPLA_BF16) return fail(CPLA_E_DTYPE, "unknown dtype %d", p->dtype);
  const int64_t nv = p->N / 4;
  if (p->N % 4 != 0 || nv > 64 || (nv & (nv - 1)) != 0)
    return fail(CPLA_E_UNSUPPORTED, "N=%lld unsupported (4 times a power of two up to 256)", (long long)p->N);
  if (p->P <= 0 || p->P % 4 != 0 || p->P > 256)
    return fail(CPLA_E_UNSUPPORTED, "P=%lld unsupported (a positive multiple of 4 up to 256)", (long long)p->P);
  return CPLA_OK;
}

cpla_status ptr_ok(const void* ptr, const char* name) {
  if (!ptr) return fail(CPLA_E_INVALID, "%s is NULL", name);
  if (((uintptr_t)ptr & 15u) != 0) return fail(CPLA_E_ALIGN, "%s is not 16-byte aligned", name);
  return CPLA_OK;
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace
}  // namespace cpla

using namespace cpla;

extern "C" cpla_status cpla_ssd_inputs(const cpla_ssd_problem* p, const float* dt, const float* A, const void* Bm,
                                       const void* Cm, void* q, void* k, float* g, hipStream_t stream) {
  clear_error();
  cpla_status st = check_ssd(p);
  if (st != CPLA_OK) return st;
  if (!q != !k) return fail(CPLA_E_INVALID, "q and k must both be NULL (B and C read in place) or both given");
  const bool copies = q != nullptr;
  const void* in[] = {dt, A, g, Bm, Cm, q, k};
  const char* nm[] = {"dt", "A", "g", "B", "C", "q", "k"};
  for (int i = 0; i < (copies ? 7 : 3); ++i)
    if ((st = ptr_ok(in[i], nm[i])) != CPLA_OK) return st;
  SsdArgs a{};
  a.B = p->B; a.T = p->T; a.H = p->H; a.G = p->G; a.N = p->N; a.P = p->P;
  a.dt = dt; a.A = A; a.Bm = Bm; a.Cm = Cm; a.q = q; a.k = k; a.g = g;
  if (!copies) {
    hipLaunchKernelGGL(ssd_decay, dim3(blocks_for(p->B * p->T * p->H)), dim3(256), 0, stream, a);
  } else {
    const unsigned nb = blocks_for(p->B * p->T * p->H * (p->N / 4));
    if (p->dtype == CPLA_BF16) hipLaunchKernelGGL(ssd_inputs<bf16_t>, dim3(nb), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(ssd_inputs<float>, dim3(nb), dim3(256), 0, stream, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CPLA_E_HIP, "ssd_inputs launch: %s", hipGetErrorString(e));
  return CPLA_OK;
}

extern "C" cpla_status cpla_ssd_input_grads(const cpla_ssd_problem* p, const float* dt, const float* A,
                                            const float* dq, const float* dk, const float* dv, const float* dg,
                                            const float* dw, void* dx, float* d_dt, float* dA, void* dB, void* dC,
                                            hipStream_t stream) {
  clear_error();
  cpla_status st = check_ssd(p);
  if (st != CPLA_OK) return st;
  const void* in[] = {dt, A, dq, dk, dv, dg, dw, dx, d_dt, dA, dB, dC};
  const char* nm[] = {"dt", "A", "dq", "dk", "dv", "dg", "dw", "dx", "d_dt", "dA", "dB", "dC"};
  for (int i = 0; i < 12; ++i)
    if ((st = ptr_ok(in[i], nm[i])) != CPLA_OK) return st;
  SsdArgs a{};
  a.B = p->B; a.T = p->T; a.H = p->H; a.G = p->G; a.N = p->N; a.P = p->P;
  a.dt = dt; a.A = A; a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dw = dw;
  a.dx = dx; a.ddt = d_dt; a.dA = dA; a.dB = dB; a.dC = dC;
  const unsigned nb = blocks_for(p->B * p->T * p->G * ((p->N > p->P ? p->N : p->P) / 4));
  if (p->dtype == CPLA_BF16) hipLaunchKernelGGL(ssd_grads<bf16_t>, dim3(nb), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(ssd_grads<float>, dim3(nb), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(ssd_dA, dim3((unsigned)p->H), dim3(DA_THREADS), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CPLA_E_HIP, "ssd gradient launch: %s", hipGetErrorString(e));
  return CPLA_OK;
}
