// Measured ceilings for the rooflines: the HBM read bandwidth a plain streaming kernel
// reaches on this GPU, and the bf16 MFMA rate of back-to-back v_mfma_f32_32x32x16_bf16.
// The library's kernels are reported against these as well as against the published
// peaks (8 TB/s, 2.5 PFLOP/s dense bf16).
#include "dg_common.h"

namespace {

// XOR of every 16-byte word of the buffer, eight loads in flight per thread; each
// workgroup writes its XOR to sink[blockIdx.x] (a few KiB of writes against the GiBs read).
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t *p, int64_t n16, uint32_t *sink) {
  __shared__ uint32_t red[256];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(p + i + j * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  red[threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

// Four independent accumulator chains per wave, operands in registers (bf16 1.0 in A and
// B, so every product is exact): after iters rounds every accumulator element is
// 16 * iters. Lane 0 of each wave writes its 64-element sum to sink[wave].
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float *sink) {
  const u32x4_t one = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma_32x32x16(one, one, c0);
    c1 = mfma_32x32x16(one, one, c1);
    c2 = mfma_32x32x16(one, one, c2);
    c3 = mfma_32x32x16(one, one, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

hipError_t dg_launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, st, (const u32x4_t *)buf, bytes / 16,
                     sink);
  return hipGetLastError();
}

hipError_t dg_launch_mfma_peak(int iters, float *sink, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}
