// Attainable-peak probes for the benchmark harness: a streaming device copy (the
// HBM rate a kernel that reads and writes every byte once can reach) and MFMA
// issue loops (the matrix-core rate a kernel with enough independent
// accumulator chains can reach). They measure the machine, not the method, and
// live in their own library (libcpla_peaks.so) so that the method's library
// carries only the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int COPY_THREADS = 256;
constexpr int MFMA_THREADS = 256;   // four waves per workgroup
constexpr int CHAINS = 8;           // independent accumulators per wave

// Grid-stride copy of n16 16-byte vectors, U in flight per thread; NT: the
// nontemporal (streaming) forms of the loads and stores.
template <int U, bool NT>
__global__ __launch_bounds__(COPY_THREADS) void peak_copy(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                          int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * COPY_THREADS;
  int64_t i = (int64_t)blockIdx.x * COPY_THREADS + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (NT) __builtin_nontemporal_store(x[u], dst + i + u * stride);
      else dst[i + u * stride] = x[u];
    }
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// KIND 0: v_mfma_f32_16x16x32_bf16; 1: v_mfma_f32_16x16x4_f32; 2: v_mfma_f64_16x16x4_f64;
// 3: v_mfma_f32_32x32x16_bf16.
// Each wave issues CHAINS independent accumulations per iteration; the sums are
// stored (one float per thread) so that nothing is optimised away.
template <int KIND>
__global__ __launch_bounds__(MFMA_THREADS) void peak_mfma(float* __restrict__ out, int iters) {
  const float x = 1.0f + 1e-3f * (float)(threadIdx.x & 63);
  float sum = 0.f;
  if constexpr (KIND == 0) {
    // a different second operand per chain: with one shared operand the compiler
    // rotates the accumulators through other registers every iteration
    bf16x8 a, b[CHAINS];
    for (int e = 0; e < 8; ++e) a[e] = (__bf16)(x * (e + 1));
    for (int c = 0; c < CHAINS; ++c)
      for (int e = 0; e < 8; ++e) b[c][e] = (__bf16)(1e-4f * (e + 1 + c));
    f32x4 acc[CHAINS];
    for (int c = 0; c < CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[c], acc[c], 0, 0, 0);
    for (int c = 0; c < CHAINS; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else if constexpr (KIND == 1) {
    const float a = x;
    float b[CHAINS];
    for (int c = 0; c < CHAINS; ++c) b[c] = 1e-4f * x * (c + 1);
    f32x4 acc[CHAINS];
    for (int c = 0; c < CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b[c], acc[c], 0, 0, 0);
    for (int c = 0; c < CHAINS; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else if constexpr (KIND == 3) {
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    bf16x8 a, b[CHAINS / 2];
    for (int e = 0; e < 8; ++e) a[e] = (__bf16)(x * (e + 1));
    for (int c = 0; c < CHAINS / 2; ++c)
      for (int e = 0; e < 8; ++e) b[c][e] = (__bf16)(1e-4f * (e + 1 + c));
    f32x16 acc[CHAINS / 2];
    for (int c = 0; c < CHAINS / 2; ++c)
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CHAINS / 2; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[c], acc[c], 0, 0, 0);
    for (int c = 0; c < CHAINS / 2; ++c)
      for (int e = 0; e < 16; ++e) sum += acc[c][e];
  } else {
    const double a = x;
    double b[CHAINS];
    for (int c = 0; c < CHAINS; ++c) b[c] = 1e-4 * x * (c + 1);
    f64x4 acc[CHAINS];
    for (int c = 0; c < CHAINS; ++c) acc[c] = f64x4{0.0, 0.0, 0.0, 0.0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b[c], acc[c], 0, 0, 0);
    for (int c = 0; c < CHAINS; ++c) sum += (float)(acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3]);
  }
  out[(int64_t)blockIdx.x * MFMA_THREADS + threadIdx.x] = sum;
}

}  // namespace

// Copy `bytes` (a multiple of 16; both pointers 16-byte aligned device memory)
// from src to dst on `stream` with `blocks` workgroups of 256 threads. Returns
// 0, or -1 for bad arguments, or the HIP error code of the launch.
// `variant`: 0 four vectors in flight per thread, 1 eight, 2 eight with nontemporal
// loads and stores.
extern "C" int cpla_peak_copy(const void* src, void* dst, int64_t bytes, int blocks, int variant,
                              hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || (bytes & 15) || blocks <= 0 || (((uintptr_t)src | (uintptr_t)dst) & 15))
    return -1;
  const f32x4* s = static_cast<const f32x4*>(src);
  f32x4* d = static_cast<f32x4*>(dst);
  const dim3 grid((unsigned)blocks), block(COPY_THREADS);
  if (variant == 0) hipLaunchKernelGGL((peak_copy<4, false>), grid, block, 0, stream, s, d, bytes / 16);
  else if (variant == 1) hipLaunchKernelGGL((peak_copy<8, false>), grid, block, 0, stream, s, d, bytes / 16);
  else if (variant == 2) hipLaunchKernelGGL((peak_copy<8, true>), grid, block, 0, stream, s, d, bytes / 16);
  else return -1;
  return (int)hipGetLastError();
}

// Run the MFMA issue loop `kind` (0 bf16 16x16x32, 1 fp32 16x16x4, 2 fp64
// 16x16x4, 3 bf16 32x32x16) on `blocks` workgroups of four waves, `iters`
// iterations per wave; `out` (device, blocks * 256 floats) receives the sums. The
// flops executed are blocks * 4 * iters * cpla_peak_mfma_flops(kind).
extern "C" int cpla_peak_mfma(int kind, float* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks <= 0 || iters <= 0) return -1;
  const dim3 grid((unsigned)blocks), block(MFMA_THREADS);
  if (kind == 0) hipLaunchKernelGGL(peak_mfma<0>, grid, block, 0, stream, out, iters);
  else if (kind == 1) hipLaunchKernelGGL(peak_mfma<1>, grid, block, 0, stream, out, iters);
  else if (kind == 2) hipLaunchKernelGGL(peak_mfma<2>, grid, block, 0, stream, out, iters);
  else if (kind == 3) hipLaunchKernelGGL(peak_mfma<3>, grid, block, 0, stream, out, iters);
  else return -1;
  return (int)hipGetLastError();
}

// Flops of one iteration of loop `kind` per wave (its issues x 2 m n k), 0 for an
// unknown kind.
extern "C" int64_t cpla_peak_mfma_flops(int kind) {
  if (kind == 0) return CHAINS * 2 * 16 * 16 * 32;
  if (kind == 1 || kind == 2) return CHAINS * 2 * 16 * 16 * 4;
  if (kind == 3) return CHAINS / 2 * 2 * 32 * 32 * 16;
  return 0;
}
