// Measured peaks of the chip: the dense MFMA issue rate (bf16 / fp16 inputs,
// fp32 accumulate) and HBM streaming rates (copy, read).  These kernels sit
// beside the attention library and share nothing with it; they give the
// ceilings the attention kernels are compared with on the same box and
// clocks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsa_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChains = 4;   // independent accumulators per wave: covers the MFMA issue latency

template <typename V>
__device__ __forceinline__ f32x16 mfma(V a, V b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma<bf16x8>(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma<f16x8>(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <typename V, typename E>
__global__ __launch_bounds__(kThreads) void peak_mfma_kernel(int iters, float a, float* out) {
  V x;
  for (int i = 0; i < 8; ++i) x[i] = (E)a;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma<V>(x, x, c0);
    c1 = mfma<V>(x, x, c1);
    c2 = mfma<V>(x, x, c2);
    c3 = mfma<V>(x, x, c3);
  }
  if (threadIdx.x == 0) out[blockIdx.x] = c0[0] + c1[0] + c2[0] + c3[0];
}

__global__ __launch_bounds__(kThreads) void peak_copy_kernel(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  // four independent 16-byte loads in flight per lane before the stores
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 v0 = __builtin_nontemporal_load(src + i);
    u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + stride);
    __builtin_nontemporal_store(v2, dst + i + 2 * stride);
    __builtin_nontemporal_store(v3, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kThreads) void peak_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                             unsigned* out) {
  __shared__ unsigned wx[kThreads / 64];
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 v0 = __builtin_nontemporal_load(src + i);
    u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= v0 ^ v1 ^ v2 ^ v3;
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = wx[0] ^ wx[1] ^ wx[2] ^ wx[3];
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -2; }

}  // namespace

extern "C" __attribute__((visibility("default")))
int tsa_peak_mfma(int dtype, int n_blocks, int iters, float a, float* out, double* flops_out,
                  void* stream) {
  if ((dtype != 0 && dtype != 1) || n_blocks < 1 || n_blocks > 65536 || iters < 1 ||
      iters > (1 << 20) || !out || !flops_out)
    return -1;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == 0)
    peak_mfma_kernel<bf16x8, __bf16><<<n_blocks, kThreads, 0, st>>>(iters, a, out);
  else
    peak_mfma_kernel<f16x8, _Float16><<<n_blocks, kThreads, 0, st>>>(iters, a, out);
  *flops_out = (double)n_blocks * (kThreads / 64) * kChains * iters * (2.0 * 32 * 32 * 16);
  return launched();
}

extern "C" __attribute__((visibility("default")))
int tsa_peak_copy(const void* src, void* dst, size_t bytes, int n_blocks, void* stream) {
  if (!src || !dst || bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16 || n_blocks < 1 ||
      n_blocks > 65536)
    return -1;
  const char* s = (const char*)src;
  const char* d = (const char*)dst;
  if (bytes && s < d + bytes && d < s + bytes) return -1;
  if (bytes == 0) return 0;
  peak_copy_kernel<<<n_blocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, (u32x4*)dst,
                                                                   bytes / 16);
  return launched();
}

extern "C" __attribute__((visibility("default")))
int tsa_peak_read(const void* src, size_t bytes, int n_blocks, unsigned* out, void* stream) {
  if (!src || !out || bytes % 16 || (uintptr_t)src % 16 || n_blocks < 1 || n_blocks > 65536)
    return -1;
  peak_read_kernel<<<n_blocks, kThreads, 0, (hipStream_t)stream>>>((const u32x4*)src, bytes / 16,
                                                                   out);
  return launched();
}
