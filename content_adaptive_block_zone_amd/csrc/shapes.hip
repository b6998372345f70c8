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

// Mixed volumes: one workgroup per (batch*head).  The activity of zone z is its video
// activity relative to the mean over the head's zones plus its audio gate; the volume is
// 4*unit below tau_256, 2*unit below tau_128, else unit (falling back to a smaller volume
// when none of the chosen volume tiles the zone), and the shape is the Eq. 7 choice among
// the candidates of that volume.  The margin is the smaller of the shape margin and the
// relative distance of the activity to each threshold.
__global__ __launch_bounds__(NT) void k_assign_multi(const float* __restrict__ stats, const float* __restrict__ vact,
                                                     int nZ, ShapeTab tab, prism_shape_params p, float tau_128,
                                                     float tau_256, int32_t* __restrict__ shape_id,
                                                     float* __restrict__ margin) {
  __shared__ float red[8];
  const int bh = blockIdx.x;
  const float* st = stats + size_t(bh) * nZ * 8;
  const float* va = vact + size_t(bh) * nZ;
  float mn = 0.f, nn = 0.f, vs = 0.f, vc = 0.f;
  for (int z = threadIdx.x; z < nZ; z += NT) {
    mn = fmaf(st[z * 8 + 6], st[z * 8 + 7], mn);
    nn += st[z * 8 + 7];
    if (st[z * 8 + 7] > 0.f) {
      vs += va[z];
      vc += 1.f;
    }
  }
  mn = block_sum<NT>(mn, red);
  nn = block_sum<NT>(nn, red);
  vs = block_sum<NT>(vs, red);
  vc = block_sum<NT>(vc, red);
  const float mbar = mn / nn;
  const float vmean = vs / fmaxf(vc, 1.f);
  const float inv_tau = 1.f / (p.tau_hi - p.tau_lo);
  // volumes present with at least one feasible candidate
  bool has2 = false, has4 = false;
  for (int c = 0; c < tab.n; ++c) {
    has2 |= tab.feasible[c] && tab.cvol[c] == 2 * tab.vol;
    has4 |= tab.feasible[c] && tab.cvol[c] == 4 * tab.vol;
  }
  for (int z = threadIdx.x; z < nZ; z += NT) {
    const float* s = st + z * 8;
    const float ratio = s[6] / fmaxf(mbar, p.eps);
    const float abar = fminf(fmaxf((ratio - p.tau_lo) * inv_tau, 0.f), 1.f);
    const float rho = vmean > 0.f ? va[z] / vmean : 0.f;
    const float act = rho + abar;
    int want = act < tau_256 ? 4 : (act < tau_128 ? 2 : 1);
    if (want == 4 && !has4) want = 2;
    if (want == 2 && !has2) want = 1;
    const int vol = want * tab.vol;
    const float lam0 = log2f(float(vol)) / 3.f;
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
      if (!tab.feasible[c] || tab.cvol[c] != vol) continue;
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
    if (margin) {
      float m = isinf(d2) ? 1.f : (d2 - d1) / fmaxf(d2, 1e-12f);
      m = fminf(m, fabsf(act - tau_128) / tau_128);
      m = fminf(m, fabsf(act - tau_256) / tau_256);
      margin[size_t(bh) * nZ + z] = m;
    }
  }
}

// Block-level valid counts at each block's first unit (the whole block's count), 0 at its
// other units, from the per-unit counts of the permutation.  One thread per unit.
__global__ void k_block_heads(const int32_t* __restrict__ unit_valid, const int32_t* __restrict__ shape_id, Geo g,
                              ShapeTab tab, int nb, size_t total, int32_t* __restrict__ block_valid) {
  const size_t t = blockIdx.x * size_t(blockDim.x) + threadIdx.x;
  if (t >= total) return;
  const int bh = int(t / nb), u = int(t % nb);
  const int upz = g.Vz / tab.vol;
  const int z = u / upz, uz = u % upz;
  const int gu = tab.cvol[shape_id[size_t(bh) * g.nZ + z]] / tab.vol;
  int n = 0;
  if (uz % gu == 0)
    for (int k = 0; k < gu; ++k) n += unit_valid[t + k];
  block_valid[t] = n;
}

}  // namespace

hipError_t launch_assign_shapes_multi(const float* stats, const float* vact, int BH, const Geo& g,
                                      const ShapeTab& tab, const prism_shape_params& p, float tau_128,
                                      float tau_256, int32_t* shape_id, float* margin, hipStream_t s) {
  hipLaunchKernelGGL(k_assign_multi, dim3(BH), dim3(NT), 0, s, stats, vact, g.nZ, tab, p, tau_128, tau_256,
                     shape_id, margin);
  return hipGetLastError();
}

hipError_t launch_block_heads(const int32_t* unit_valid, const int32_t* shape_id, int BH, const Geo& g,
                              const ShapeTab& tab, int32_t* block_valid, hipStream_t s) {
  const int nb = g.nZ * (g.Vz / tab.vol);
  const size_t total = size_t(BH) * nb;
  hipLaunchKernelGGL(k_block_heads, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, unit_valid, shape_id, g,
                     tab, nb, total, block_valid);
  return hipGetLastError();
}

hipError_t launch_assign_shapes(const float* stats, int BH, const Geo& g, const ShapeTab& tab,
                                const prism_shape_params& p, int32_t* shape_id, float* margin,
                                hipStream_t s) {
  const float lam0 = float(std::log2(double(tab.vol)) / 3.0);
  hipLaunchKernelGGL(k_assign, dim3(BH), dim3(NT), 0, s, stats, g.nZ, tab, p, lam0, shape_id, margin);
  return hipGetLastError();
}

}  // namespace prism
