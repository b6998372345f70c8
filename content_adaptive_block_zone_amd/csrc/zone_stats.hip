// Zone statistics (Prism abstract: per-zone variance of the video features taken per
// channel, and norms of the audio-to-video cross-attention output; Table 9 caption:
// r_{v,d}, the audio coupling gate and the audio directional variance).
//
// One workgroup per (batch*head, zone).  The zone is streamed row by row: a group of
// D/8 lanes owns one (t, h) row of the zone and walks it along w, each lane holding 8
// channels, four tokens per step with all their loads issued together (the kernel is
// bound by memory latency, so the loads in flight per lane matter more than anything
// else).  Increments along w stay in registers; the neighbour rows along h and t are read
// again, close enough in time to hit in cache, so HBM traffic stays near one pass over V
// and the A2V output.  The
// per-token A2V norm goes to a zone-local LDS map, from which the audio increments are
// taken after the streaming pass.  Per-channel sums are reduced across the row groups of
// a wavefront with lane shuffles, then across the four wavefronts in LDS.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int NT = 256;
constexpr int NWAVE = NT / 64;

// GLOBAL: instead of taking each channel's share of its semivariance per axis and
// averaging the shares, take the per-axis semivariance averaged over all channels
// jointly and its share (the "global variance" variant of Eq. 1, Table 9 caption).
// FROM_NORM: aux is the per-token A2V norm map, float [BH][N], instead of the A2V output
// rows [BH][N][D] whose norms the kernel would take itself.
template <typename T, int D, bool GLOBAL, bool FROM_NORM>
__global__ __launch_bounds__(NT) void k_zone_stats(const T* __restrict__ v, const void* __restrict__ aux,
                                                   float* __restrict__ stats, float* __restrict__ vact, Geo g) {
  const T* a2v = static_cast<const T*>(aux);
  const float* anorm = static_cast<const float*>(aux);
  constexpr int G = D / 8;      // lanes per token
  constexpr int RPP = NT / G;   // rows in flight per pass
  constexpr int U = 4;          // tokens along w per step
  __shared__ float s_a[kMaxZoneVol];
  __shared__ float s_red[NWAVE][3][D];
  __shared__ float s_share[3][D];
  __shared__ float s_tmp[8];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int z = blockIdx.x % g.nZ;
  const int bh = blockIdx.x / g.nZ;
  const int iw = z % g.nzw, ih = (z / g.nzw) % g.nzh, it = z / (g.nzw * g.nzh);
  const int t0 = it * g.zt, h0 = ih * g.zh, w0 = iw * g.zw;
  const int et = min(g.zt, g.T - t0), eh = min(g.zh, g.H - h0), ew = min(g.zw, g.W - w0);
  const size_t base = size_t(bh) * g.N * D;
  const size_t row_stride_h = size_t(g.W) * D, row_stride_t = size_t(g.H) * g.W * D;
  const int cg = tid % G, rg = tid / G;

  float ssd[3][8];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int k = 0; k < 8; ++k) ssd[a][k] = 0.f;

  // rows are numbered t-fastest, so the row groups of one pass read each other's t- and
  // h-neighbour rows at about the same time and the rereads hit in cache
  for (int row = rg; row < et * eh; row += RPP) {
    const int lt = row % et, lh = row / et;
    const size_t off = base + (size_t((t0 + lt) * g.H + h0 + lh) * g.W + w0) * D + cg * 8;
    const T* vr = v + off;
    const T* ar = a2v + off;
    const float* nr = anorm + size_t(bh) * g.N + size_t((t0 + lt) * g.H + h0 + lh) * g.W + w0;
    const bool has_t = lt + 1 < et, has_h = lh + 1 < eh;
    // A neighbour row that does not exist is replaced by the row itself, and a token past
    // the zone's end by the last one: their increments are exactly zero (the ragged tail
    // is also multiplied by 0), so every load and update is unconditional and the loads
    // of a step stay in flight together.
    const size_t dh = has_h ? row_stride_h : 0, dt = has_t ? row_stride_t : 0;
    float prev[8];
    for (int lw0 = 0; lw0 < ew; lw0 += U) {
      float x[U][8], yh[U][8], yt[U][8], u[U][8];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const size_t o = size_t(min(lw0 + j, ew - 1)) * D;
        load8(vr + o, x[j]);
        load8(vr + o + dh, yh[j]);
        load8(vr + o + dt, yt[j]);
        if constexpr (!FROM_NORM) load8_once(ar + o, u[j]);  // each A2V row is read once
      }
      if (lw0 == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) prev[k] = x[0][k];
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int lw = lw0 + j;
        const float m = lw < ew ? 1.f : 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float dw = x[j][k] - prev[k];
          const float dhh = (x[j][k] - yh[j][k]) * m;
          const float dtt = (x[j][k] - yt[j][k]) * m;
          ssd[2][k] = fmaf(dw, dw, ssd[2][k]);
          ssd[1][k] = fmaf(dhh, dhh, ssd[1][k]);
          ssd[0][k] = fmaf(dtt, dtt, ssd[0][k]);
          prev[k] = x[j][k];
        }
        if constexpr (FROM_NORM) {
          if (cg == 0 && lw < ew) s_a[(lt * g.zh + lh) * g.zw + lw] = nr[lw];
        } else {
          float sq = 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) sq = fmaf(u[j][k], u[j][k], sq);
#pragma unroll
          for (int o = G / 2; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
          if (cg == 0 && lw < ew) s_a[(lt * g.zh + lh) * g.zw + lw] = sqrtf(sq);
        }
      }
    }
  }

  // ---- video: per-channel semivariance, share per axis, mean over channels
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float t = ssd[a][k];
#pragma unroll
      for (int o = G; o < 64; o <<= 1) t += __shfl_xor(t, o, 64);
      if (lane < G) s_red[wv][a][cg * 8 + k] = t;
    }
  __syncthreads();
  const float np_t = float(max(et - 1, 0) * eh * ew);
  const float np_h = float(et * max(eh - 1, 0) * ew);
  const float np_w = float(et * eh * max(ew - 1, 0));
  const float npair[3] = {np_t, np_h, np_w};
  float vs = 0.f;  // channel sum of the per-axis semivariances (zone activity)
  for (int c = tid; c < D; c += NT) {
    float gam[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < NWAVE; ++r) s += s_red[r][a][c];
      gam[a] = npair[a] > 0.f ? 0.5f * s / npair[a] : 0.f;
    }
    vs += gam[0] + gam[1] + gam[2];
    if (GLOBAL) {
#pragma unroll
      for (int a = 0; a < 3; ++a) s_share[a][c] = gam[a];
    } else {
      const float den = gam[0] + gam[1] + gam[2] + 1e-12f;
#pragma unroll
      for (int a = 0; a < 3; ++a) s_share[a][c] = gam[a] / den;
    }
  }
  __syncthreads();
  float sh[3] = {0.f, 0.f, 0.f};
  for (int c = tid; c < D; c += NT) {
#pragma unroll
    for (int a = 0; a < 3; ++a) sh[a] += s_share[a][c];
  }

  // ---- audio: norm map increments and zone mean
  float sa[3] = {0.f, 0.f, 0.f}, asum = 0.f;
  const int nval = et * eh * ew;
  const int plane = g.zh * g.zw;
  for (int p = tid; p < nval; p += NT) {
    const int lt = p / (eh * ew), lh = (p / ew) % eh, lw = p % ew;
    const int idx = (lt * g.zh + lh) * g.zw + lw;
    const float a = s_a[idx];
    asum += a;
    if (lt + 1 < et) { const float dd = a - s_a[idx + plane]; sa[0] = fmaf(dd, dd, sa[0]); }
    if (lh + 1 < eh) { const float dd = a - s_a[idx + g.zw]; sa[1] = fmaf(dd, dd, sa[1]); }
    if (lw + 1 < ew) { const float dd = a - s_a[idx + 1]; sa[2] = fmaf(dd, dd, sa[2]); }
  }
  float res[7];
#pragma unroll
  for (int a = 0; a < 3; ++a) res[a] = block_sum<NT>(sh[a], s_tmp);
#pragma unroll
  for (int a = 0; a < 3; ++a) res[3 + a] = block_sum<NT>(sa[a], s_tmp);
  res[6] = block_sum<NT>(asum, s_tmp);
  if (vact) {  // uniform over the workgroup
    vs = block_sum<NT>(vs, s_tmp);
    if (tid == 0) vact[size_t(bh) * g.nZ + z] = vs / float(D);
  }
  if (tid == 0) {
    float* out = stats + (size_t(bh) * g.nZ + z) * 8;
    if (GLOBAL) {  // shares of the channel-mean semivariances
      const float den = (res[0] + res[1] + res[2]) / float(D) + 1e-12f;
      out[0] = res[0] / float(D) / den;
      out[1] = res[1] / float(D) / den;
      out[2] = res[2] / float(D) / den;
    } else {       // channel-mean of the per-channel shares
      out[0] = res[0] / float(D);
      out[1] = res[1] / float(D);
      out[2] = res[2] / float(D);
    }
    out[3] = np_t > 0.f ? 0.5f * res[3] / np_t : 0.f;
    out[4] = np_h > 0.f ? 0.5f * res[4] / np_h : 0.f;
    out[5] = np_w > 0.f ? 0.5f * res[5] / np_w : 0.f;
    out[6] = res[6] / float(nval);
    out[7] = float(nval);
  }
}

template <typename T, bool GLOBAL, bool FROM_NORM>
hipError_t launch_t(const void* v, const void* aux, int BH, int d, const Geo& g, float* stats, float* vact,
                    hipStream_t s) {
  dim3 grid(unsigned(BH) * unsigned(g.nZ)), block(NT);
  const T* pv = static_cast<const T*>(v);
  switch (d) {
    case 32: hipLaunchKernelGGL((k_zone_stats<T, 32, GLOBAL, FROM_NORM>), grid, block, 0, s, pv, aux, stats, vact, g); break;
    case 64: hipLaunchKernelGGL((k_zone_stats<T, 64, GLOBAL, FROM_NORM>), grid, block, 0, s, pv, aux, stats, vact, g); break;
    case 128: hipLaunchKernelGGL((k_zone_stats<T, 128, GLOBAL, FROM_NORM>), grid, block, 0, s, pv, aux, stats, vact, g); break;
    case 256: hipLaunchKernelGGL((k_zone_stats<T, 256, GLOBAL, FROM_NORM>), grid, block, 0, s, pv, aux, stats, vact, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const void* v, const void* aux, int BH, int d, const Geo& g, bool global_variance,
                     bool from_norm, float* stats, float* vact, hipStream_t s) {
  if (from_norm)
    return global_variance ? launch_t<T, true, true>(v, aux, BH, d, g, stats, vact, s)
                           : launch_t<T, false, true>(v, aux, BH, d, g, stats, vact, s);
  return global_variance ? launch_t<T, true, false>(v, aux, BH, d, g, stats, vact, s)
                         : launch_t<T, false, false>(v, aux, BH, d, g, stats, vact, s);
}

}  // namespace

hipError_t launch_zone_stats(const void* v, const void* aux, prism_dtype dt, int BH, int d, const Geo& g,
                             bool global_variance, bool from_norm, float* stats, float* vact, hipStream_t s) {
  if (dt == PRISM_BF16) return launch_dt<bf16_t>(v, aux, BH, d, g, global_variance, from_norm, stats, vact, s);
  return launch_dt<float>(v, aux, BH, d, g, global_variance, from_norm, stats, vact, s);
}

}  // namespace prism
