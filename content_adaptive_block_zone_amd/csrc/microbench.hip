// Measurement kernel: the matrix-core peak of this GPU for the attention kernels' product
// (v_mfma_f32_32x32x16_bf16) and the shader clock it runs at.  Each wave keeps four
// independent accumulators and issues their products round-robin for `iters` steps, so
// the matrix pipe of every SIMD always has independent work.  The first wave of each
// workgroup records its shader-clock cycles (s_memtime) and 100 MHz reference ticks
// (s_memrealtime) over the loop, from which the clock under this load follows.
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

}  // namespace

hipError_t launch_mfma_peak(int workgroups, int iters, unsigned long long* clocks, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_peak, dim3(workgroups), dim3(256), 0, s, iters, clocks, sink);
  return hipGetLastError();
}

}  // namespace prism
