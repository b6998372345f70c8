// Measurement kernel: the matrix-core peak of this GPU for the attention kernels' product
// (v_mfma_f32_32x32x16_bf16) and the shader clock it runs at.  Each wave keeps four
// independent accumulators and issues their products round-robin for `iters` steps, so
// the matrix pipe of every SIMD always has independent work.  The first wave of each
// workgroup records its shader-clock cycles (s_memtime) and 100 MHz reference ticks
// (s_memrealtime) over the loop, from which the clock under this load follows.
// A second kernel reads two buffers front to back (grid-stride, 16-byte loads, two per
// buffer in flight per thread): the rate of a plain contiguous read of the same bytes as a
// memory-bound stage, the ceiling that stage's access pattern is measured against.
#include "prism_internal.h"

namespace prism {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 2) void k_mfma_peak(int iters, unsigned long long* __restrict__ clocks,
                                                      float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float((lane + e) & 7) * 0.125f);
    b[e] = (__bf16)(float((lane * 3 + e) & 7) * 0.0625f);
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (s == -1.f) sink[blockIdx.x] = s;  // never true: keeps the products live
}

constexpr int kStreamWgs = PRISM_BENCH_STREAM_SINK / 4;  // one checksum per wavefront
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ a, const u32x4* __restrict__ b,
                                                     size_t n, uint32_t* __restrict__ sink) {
  const size_t stride = size_t(gridDim.x) * 256;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  for (; i + stride < n; i += 2 * stride) {
    const u32x4 a0 = a[i], a1 = a[i + stride], b0 = b[i], b1 = b[i + stride];
    acc ^= a0 ^ a1 ^ b0 ^ b1;
  }
  for (; i < n; i += stride) acc ^= a[i] ^ b[i];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= uint32_t(__shfl_xor(int(x), o, 64));
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;  // XOR of every word the wave read
}

}  // namespace

hipError_t launch_stream_read(const void* a, const void* b, size_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(kStreamWgs), dim3(256), 0, s, static_cast<const u32x4*>(a),
                     static_cast<const u32x4*>(b), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_peak(int workgroups, int iters, unsigned long long* clocks, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_peak, dim3(workgroups), dim3(256), 0, s, iters, clocks, sink);
  return hipGetLastError();
}

}  // namespace prism
