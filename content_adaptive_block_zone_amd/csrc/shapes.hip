// Shape assignment (Prism abstract: finer partitioning along axes of rapid visual
// variation and strong audio-visual coupling; Table 9 caption: gate a-bar and audio
// directional variance; Table 10 caption: b*_d ~ g_d^-alpha and the quantization of
// Eq. 7).  One workgroup per (batch*head): the head-mean A2V norm is reduced first,
// then each thread scores every feasible candidate for its zones in float32.
#include <cmath>

#include "prism_internal.h"

namespace prism {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void k_assign(const float* __restrict__ stats, int nZ, ShapeTab tab,
                                               prism_shape_params p, float lam0,
                                               int32_t* __restrict__ shape_id,
                                               float* __restrict__ margin) {
  __shared__ float red[8];
  const int bh = blockIdx.x;
  const float* st = stats + size_t(bh) * nZ * 8;
  float mn = 0.f, nn = 0.f;
  for (int z = threadIdx.x; z < nZ; z += NT) {
    mn = fmaf(st[z * 8 + 6], st[z * 8 + 7], mn);
    nn += st[z * 8 + 7];
  }
  mn = block_sum<NT>(mn, red);
  nn = block_sum<NT>(nn, red);
  const float mbar = mn / nn;
  const float inv_tau = 1.f / (p.tau_hi - p.tau_lo);
  for (int z = threadIdx.x; z < nZ; z += NT) {
    const float* s = st + z * 8;
    const float ratio = s[6] / fmaxf(mbar, p.eps);
    const float abar = fminf(fmaxf((ratio - p.tau_lo) * inv_tau, 0.f), 1.f);
    const float asum = s[3] + s[4] + s[5] + p.eps;
    float L[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const float vhat = s[3 + d] / asum;
      const float gd = fmaxf((1.f - abar) * s[d] + abar * vhat, p.g_min);
      L[d] = log2f(gd);
    }
    const float mean = (L[0] + L[1] + L[2]) / 3.f;
    float lam[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) lam[d] = lam0 - p.alpha * (L[d] - mean);
    float d1 = INFINITY, d2 = INFINITY;
    int best = 0;
    for (int c = 0; c < tab.n; ++c) {
      if (!tab.feasible[c]) continue;
      const float e0 = tab.lg[c][0] - lam[0], e1 = tab.lg[c][1] - lam[1], e2 = tab.lg[c][2] - lam[2];
      const float D = e0 * e0 + e1 * e1 + e2 * e2;
      if (D < d1) {
        d2 = d1;
        d1 = D;
        best = c;
      } else if (D < d2) {
        d2 = D;
      }
    }
    shape_id[size_t(bh) * nZ + z] = best;
    if (margin) margin[size_t(bh) * nZ + z] = isinf(d2) ? 1.f : (d2 - d1) / fmaxf(d2, 1e-12f);
  }
}

}  // namespace

hipError_t launch_assign_shapes(const float* stats, int BH, const Geo& g, const ShapeTab& tab,
                                const prism_shape_params& p, int32_t* shape_id, float* margin,
                                hipStream_t s) {
  const float lam0 = float(std::log2(double(tab.vol)) / 3.0);
  hipLaunchKernelGGL(k_assign, dim3(BH), dim3(NT), 0, s, stats, g.nZ, tab, p, lam0, shape_id, margin);
  return hipGetLastError();
}

}  // namespace prism
