// Ceilings measured on the running GPU, so that kernel fractions can be stated against
// what the part sustains as well as against its datasheet peaks:
//   * read stream: every byte of a buffer read once with 16-byte vector loads, eight
//     in flight per thread (no writes beyond one word per workgroup), grid-strided or
//     one contiguous slice per workgroup;
//   * matrix rate: back-to-back MFMA 32x32x16 bf16 products on register operands, eight
//     independent accumulators per wave, no memory traffic.
// Neither is part of the verify step; they exist for its measurement.

#include "vs_internal.hpp"

namespace vs {

namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_pk;

__global__ void __launch_bounds__(256)
peak_read_kernel(const u32x4 *buf, size_t n16, uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  // eight independent 16-byte loads in flight per thread and iteration
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][u & 3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    acc ^= a[0] ^ a[3];
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x & 1023], acc);
}

// one contiguous slice per workgroup, read front to back (4 KB per step, eight steps
// in flight)
__global__ void __launch_bounds__(256)
peak_read_slice_kernel(const u32x4 *buf, size_t n16, uint32_t *sink) {
  const size_t per = n16 / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = (blockIdx.x + 1 == gridDim.x) ? n16 : lo + per;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = buf[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][u & 3];
  }
  for (; i < hi; i += 256) {
    const u32x4 a = buf[i];
    acc ^= a[0] ^ a[3];
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x & 1023], acc);
}

__global__ void __launch_bounds__(256)
peak_mfma_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0f + 0.001f * (float)(lane + e));
    b[e] = (__bf16)(1.0f - 0.001f * (float)(lane - e));
  }
  f32x16_pk c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) c[k][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[k][j];
  if (s == 1.2345f) sink[blockIdx.x] = s;   // keeps the products live; never true in practice
}

}  // namespace

hipError_t launch_peak_read(const void *buf, size_t bytes, uint32_t *sink, int n_wg,
                            int pattern, hipStream_t st) {
  if (pattern == 1)
    hipLaunchKernelGGL(peak_read_slice_kernel, dim3(n_wg), dim3(256), 0, st,
                       (const u32x4 *)buf, bytes / 16, sink);
  else
    hipLaunchKernelGGL(peak_read_kernel, dim3(n_wg), dim3(256), 0, st, (const u32x4 *)buf,
                       bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(int n_wg, int iters, float *sink, hipStream_t st) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(n_wg), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

}  // namespace vs
