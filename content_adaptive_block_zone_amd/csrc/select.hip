// Block pooling and hybrid Top-k/Top-p block selection (Prism abstract: block-level
// features and a hybrid selection that fixes each query block's sparsity; Figure 2
// caption; Table 7 caption: Top-p keeps the smallest set of key blocks whose cumulative
// attention weight exceeds the threshold).
//
//   k_pool    mean of each block's valid rows (float32)           HBM-bound
//   k_scores  scale * Qbar Kbar^T per head, 64x64 register tiles  fp32 ALU
//   k_select  per query block: softmax over live key blocks, then the hybrid count found
//             by bitwise search on the float bits of the probabilities (no sort): the
//             Top-p threshold is the largest probability v whose "sum of probabilities
//             >= v" still exceeds p; the Top-k clamp is a count search.  The kept set is
//             emitted in ascending block order and marked in a bitmap for the reverse
//             index.
//   k_rev_*   deterministic transpose of the selection via that bitmap: count, scan, fill.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int NT = 256;

struct SelWs {
  float* qbar;
  float* kbar;
  float* scores;
  uint32_t* bitmap;
  int32_t* rcnt;
};

__host__ __device__ inline int words32(int nb) { return (nb + 31) / 32; }

SelWs carve(void* ws, int BH, int nb, int d) {
  char* p = static_cast<char*>(ws);
  SelWs w;
  w.qbar = reinterpret_cast<float*>(p);
  p += align256(size_t(BH) * nb * d * 4);
  w.kbar = reinterpret_cast<float*>(p);
  p += align256(size_t(BH) * nb * d * 4);
  w.scores = reinterpret_cast<float*>(p);
  p += align256(size_t(BH) * nb * nb * 4);
  w.bitmap = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(BH) * nb * words32(nb) * 4);
  w.rcnt = reinterpret_cast<int32_t*>(p);
  return w;
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t val) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
    p[i] = val;
}

// One workgroup per (block, head, tensor): D/8 lanes cover a row in 16-byte (bf16) or
// 32-byte (fp32) chunks and the row groups take rows rg, rg + NT/G, ..., four rows per
// step with their loads issued together; per-channel sums are reduced across the row
// groups of a wavefront with lane shuffles, then across wavefronts in LDS.
template <typename T, int D>
__global__ __launch_bounds__(NT) void k_pool(const T* __restrict__ qp, const T* __restrict__ kp,
                                             const int32_t* __restrict__ bvalid, int nb, int vol,
                                             float* __restrict__ qbar, float* __restrict__ kbar) {
  constexpr int G = D / 8;       // lanes per row
  constexpr int RG = NT / G;     // row groups
  constexpr int U = 4;           // rows per step
  __shared__ float s_red[NT / 64][D];
  const int I = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, cg = tid % G, rg = tid / G;
  const T* x = (blockIdx.z == 0 ? qp : kp) + (size_t(bh) * nb + I) * vol * D + cg * 8;
  float* out = (blockIdx.z == 0 ? qbar : kbar) + (size_t(bh) * nb + I) * D;
  const int n = bvalid[size_t(bh) * nb + I];
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  // rows past the valid count reread the last valid row and count zero times, so the
  // loads of a step are unconditional and stay in flight together
  for (int r0 = rg; r0 < n; r0 += U * RG) {
    float v[U][8];
#pragma unroll
    for (int j = 0; j < U; ++j) load8(x + size_t(min(r0 + j * RG, n - 1)) * D, v[j]);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const float m = r0 + j * RG < n ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(v[j][k], m, acc[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float t = acc[k];
#pragma unroll
    for (int o = G; o < 64; o <<= 1) t += __shfl_xor(t, o, 64);
    if (lane < G) s_red[wv][cg * 8 + k] = t;
  }
  __syncthreads();
  for (int c = tid; c < D; c += NT) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) t += s_red[w][c];
    out[c] = n > 0 ? t / float(n) : 0.f;
  }
}

template <typename T>
void launch_pool(const void* qp, const void* kp, const int32_t* bvalid, int BH, int nb, int vol, int d,
                 float* qbar, float* kbar, hipStream_t s) {
  const T* q = static_cast<const T*>(qp);
  const T* k = static_cast<const T*>(kp);
  const dim3 grid(nb, BH, 2);
  switch (d) {
    case 32: hipLaunchKernelGGL((k_pool<T, 32>), grid, dim3(NT), 0, s, q, k, bvalid, nb, vol, qbar, kbar); break;
    case 64: hipLaunchKernelGGL((k_pool<T, 64>), grid, dim3(NT), 0, s, q, k, bvalid, nb, vol, qbar, kbar); break;
    case 128: hipLaunchKernelGGL((k_pool<T, 128>), grid, dim3(NT), 0, s, q, k, bvalid, nb, vol, qbar, kbar); break;
    default: hipLaunchKernelGGL((k_pool<T, 256>), grid, dim3(NT), 0, s, q, k, bvalid, nb, vol, qbar, kbar); break;
  }
}

// scores[bh][I][J] = scale * sum_c qbar[bh][I][c] kbar[bh][J][c]
__global__ __launch_bounds__(256) void k_scores(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                int nb, int d, float scale, float* __restrict__ scores) {
  __shared__ float As[16][64];
  __shared__ float Bs[16][64];
  const int bh = blockIdx.z;
  const int I0 = blockIdx.y * 64, J0 = blockIdx.x * 64;
  const float* Q = qbar + size_t(bh) * nb * d;
  const float* K = kbar + size_t(bh) * nb * d;
  const int t = threadIdx.x, ty = t / 16, tx = t % 16;
  const int lr = t / 4, lc = (t % 4) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 16) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (I0 + lr < nb) a = *reinterpret_cast<const float4*>(Q + size_t(I0 + lr) * d + k0 + lc);
    if (J0 + lr < nb) b = *reinterpret_cast<const float4*>(K + size_t(J0 + lr) * d + k0 + lc);
    __syncthreads();
    As[lc + 0][lr] = a.x; As[lc + 1][lr] = a.y; As[lc + 2][lr] = a.z; As[lc + 3][lr] = a.w;
    Bs[lc + 0][lr] = b.x; Bs[lc + 1][lr] = b.y; Bs[lc + 2][lr] = b.z; Bs[lc + 3][lr] = b.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float4 av = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
      const float ar[4] = {av.x, av.y, av.z, av.w}, br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int I = I0 + ty * 4 + i;
    if (I >= nb) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int J = J0 + tx * 4 + j;
      if (J < nb) scores[(size_t(bh) * nb + I) * nb + J] = acc[i][j] * scale;
    }
  }
}

__device__ __forceinline__ uint32_t key_of(float p) { return __float_as_uint(p); }

__global__ __launch_bounds__(NT) void k_select(const float* __restrict__ scores, const int32_t* __restrict__ bvalid,
                                               int nb, prism_select_params prm, int k_max,
                                               int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
                                               float* __restrict__ sel_margin, uint32_t* __restrict__ bitmap) {
  extern __shared__ float sP[];  // nb probabilities (-1 for dead key blocks)
  __shared__ float redf[8];
  __shared__ int redi[8];
  const int I = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int32_t* bv = bvalid + size_t(bh) * nb;
  int32_t* out = sel_idx + (size_t(bh) * nb + I) * k_max;
  if (bv[I] == 0) {
    for (int s = tid; s < k_max; s += NT) out[s] = -1;
    if (tid == 0) {
      sel_cnt[size_t(bh) * nb + I] = 0;
      if (sel_margin) sel_margin[size_t(bh) * nb + I] = 1.f;
    }
    return;
  }
  const float* row = scores + (size_t(bh) * nb + I) * nb;
  float mx = -INFINITY;
  int nl = 0;
  for (int J = tid; J < nb; J += NT) {
    const bool live = bv[J] > 0;
    const float l = live ? row[J] : -INFINITY;
    sP[J] = l;
    mx = fmaxf(mx, l);
    nl += live;
  }
  mx = block_max<NT>(mx, redf);
  const int nlive = block_sum_i<NT>(nl, redi);
  float se = 0.f;
  for (int J = tid; J < nb; J += NT) {
    const float l = sP[J];
    const float e = l == -INFINITY ? -1.f : expf(l - mx);
    sP[J] = e;
    if (e >= 0.f) se += e;
  }
  se = block_sum<NT>(se, redf);
  float tot = 0.f;
  for (int J = tid; J < nb; J += NT) {
    const float e = sP[J];
    if (e >= 0.f) {
      const float p = e / se;
      sP[J] = p;
      tot += p;
    }
  }
  const float p = prm.top_p;
  tot = block_sum<NT>(tot, redf);  // also orders the writes above before the passes below

  // ---- Top-p: largest key v with sum(P >= v) > p
  int n_p = nlive, need_p = 0;
  uint32_t vstar = 0;
  float sum_gt_p = 0.f;
  if (tot > p) {
    uint32_t Tk = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = Tk | (1u << bit);
      float s = 0.f;
      for (int J = tid; J < nb; J += NT) {
        const float q = sP[J];
        if (q >= 0.f && key_of(q) >= cand) s += q;
      }
      s = block_sum<NT>(s, redf);
      if (s > p) Tk = cand;
    }
    vstar = Tk;
    float sg = 0.f;
    int cg = 0, ce = 0;
    for (int J = tid; J < nb; J += NT) {
      const float q = sP[J];
      if (q < 0.f) continue;
      const uint32_t kq = key_of(q);
      if (kq > Tk) { sg += q; ++cg; }
      else if (kq == Tk) ++ce;
    }
    sg = block_sum<NT>(sg, redf);
    cg = block_sum_i<NT>(cg, redi);
    ce = block_sum_i<NT>(ce, redi);
    const float v = __uint_as_float(Tk);
    int m = 1;
    while (m < ce && !(sg + float(m) * v > p)) ++m;
    n_p = cg + m;
    need_p = m;
    sum_gt_p = sg;
  }
  const int n = min(min(max(n_p, prm.k_min), prm.k_max), nlive);

  // ---- cut threshold for exactly n kept blocks
  uint32_t Tcut;
  int need_eq;
  if (n == n_p && tot > p) {
    Tcut = vstar;
    need_eq = need_p;
  } else {
    uint32_t Tk = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = Tk | (1u << bit);
      int c = 0;
      for (int J = tid; J < nb; J += NT) {
        const float q = sP[J];
        c += (q >= 0.f && key_of(q) >= cand);
      }
      c = block_sum_i<NT>(c, redi);
      if (c >= n) Tk = cand;
    }
    Tcut = Tk;
    int cg = 0;
    for (int J = tid; J < nb; J += NT) {
      const float q = sP[J];
      cg += (q >= 0.f && key_of(q) > Tk);
    }
    cg = block_sum_i<NT>(cg, redi);
    need_eq = n - cg;
  }

  // ---- emit ascending: each thread owns a contiguous range of key blocks
  const int R = (nb + NT - 1) / NT;
  const int J0 = min(nb, tid * R), J1 = min(nb, J0 + R);
  int my_eq = 0;
  for (int J = J0; J < J1; ++J) {
    const float q = sP[J];
    my_eq += (q >= 0.f && key_of(q) == Tcut);
  }
  int tot_eq;
  int eq_rank = block_excl_scan<NT>(my_eq, redi, &tot_eq);
  int my_sel = 0;
  for (int J = J0, r = eq_rank; J < J1; ++J) {
    const float q = sP[J];
    if (q < 0.f) continue;
    const uint32_t kq = key_of(q);
    if (kq > Tcut) ++my_sel;
    else if (kq == Tcut) { my_sel += (r < need_eq); ++r; }
  }
  int tot_sel;
  int pos = block_excl_scan<NT>(my_sel, redi, &tot_sel);
  float pmin_sel = INFINITY, pmax_uns = -INFINITY;
  uint32_t* bm = bitmap + size_t(bh) * nb * words32(nb);
  for (int J = J0, r = eq_rank; J < J1; ++J) {
    const float q = sP[J];
    if (q < 0.f) continue;
    const uint32_t kq = key_of(q);
    bool take = kq > Tcut;
    if (kq == Tcut) { take = r < need_eq; ++r; }
    if (take) {
      out[pos++] = J;
      atomicOr(bm + size_t(J) * words32(nb) + (I >> 5), 1u << (I & 31));
      pmin_sel = fminf(pmin_sel, q);
    } else {
      pmax_uns = fmaxf(pmax_uns, q);
    }
  }
  for (int s = tot_sel + tid; s < k_max; s += NT) out[s] = -1;
  if (sel_margin) {
    pmin_sel = -block_max<NT>(-pmin_sel, redf);
    pmax_uns = block_max<NT>(pmax_uns, redf);
  }
  if (tid == 0) {
    sel_cnt[size_t(bh) * nb + I] = tot_sel;
    if (sel_margin) {
      float mg = n < nlive ? (pmin_sel - pmax_uns) / pmin_sel : 1.f;
      if (tot > p && n == n_p) {
        const float v = __uint_as_float(vstar);
        const float c_np = sum_gt_p + float(need_p) * v, c_prev = c_np - v;
        mg = fminf(mg, fabsf(c_np - p));
        if (n_p > 1) mg = fminf(mg, fabsf(c_prev - p));
      }
      sel_margin[size_t(bh) * nb + I] = mg;
    }
  }
}

__global__ void k_rev_count(const uint32_t* __restrict__ bitmap, int nb, int total_rows,
                            int32_t* __restrict__ rcnt) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= total_rows) return;
  const int W = words32(nb);
  const uint32_t* row = bitmap + size_t(r) * W;
  int c = 0;
  for (int w = 0; w < W; ++w) c += __popc(row[w]);
  rcnt[r] = c;
}

__global__ __launch_bounds__(1024) void k_rev_scan(const int32_t* __restrict__ rcnt, int nb,
                                                   int32_t* __restrict__ rev_ptr) {
  __shared__ int red[20];
  const int bh = blockIdx.x;
  const int R = (nb + 1023) / 1024;
  const int J0 = min(nb, int(threadIdx.x) * R), J1 = min(nb, J0 + R);
  const int32_t* c = rcnt + size_t(bh) * nb;
  int s = 0;
  for (int J = J0; J < J1; ++J) s += c[J];
  int tot;
  int off = block_excl_scan<1024>(s, red, &tot);
  int32_t* rp = rev_ptr + size_t(bh) * (nb + 1);
  for (int J = J0; J < J1; ++J) {
    rp[J] = off;
    off += c[J];
  }
  if (threadIdx.x == 0) rp[nb] = tot;
}

// One wavefront per (key block, head): lists the set bits of the key block's bitmap row.
__global__ __launch_bounds__(64) void k_rev_fill(const uint32_t* __restrict__ bitmap, const int32_t* __restrict__ rev_ptr,
                                                 int nb, int k_max, int32_t* __restrict__ rev_idx) {
  const int J = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const int W = words32(nb);
  const uint32_t* row = bitmap + (size_t(bh) * nb + J) * W;
  int base = rev_ptr[size_t(bh) * (nb + 1) + J];
  int32_t* out = rev_idx + size_t(bh) * nb * k_max;
  for (int w0 = 0; w0 < W; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t word = w < W ? row[w] : 0u;
    const int pc = __popc(word);
    int incl = pc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int nn = __shfl_up(incl, o, 64);
      if (lane >= o) incl += nn;
    }
    int pos = base + incl - pc;
    uint32_t bits = word;
    while (bits) {
      const int b = __ffs(bits) - 1;
      out[pos++] = w * 32 + b;
      bits &= bits - 1;
    }
    base += __shfl(incl, 63, 64);
  }
}

}  // namespace

size_t select_ws_bytes(int BH, int nb, int d) {
  return 2 * align256(size_t(BH) * nb * d * 4) + align256(size_t(BH) * nb * nb * 4) +
         align256(size_t(BH) * nb * words32(nb) * 4) + align256(size_t(BH) * nb * 4);
}

hipError_t launch_select(const void* qp, const void* kp, prism_dtype dt, const int32_t* bvalid,
                         int BH, int nb, int vol, int d, float scale, const prism_select_params& p,
                         int32_t* sel_idx, int32_t* sel_cnt, int32_t* rev_ptr, int32_t* rev_idx,
                         float* sel_margin, void* ws, hipStream_t s) {
  SelWs w = carve(ws, BH, nb, d);
  const size_t nbits = size_t(BH) * nb * words32(nb);
  hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, s, w.bitmap, nbits, 0u);
  hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(rev_idx),
                     size_t(BH) * nb * p.k_max, 0xffffffffu);
  // d is one of 32, 64, 128, 256 (checked by the caller)
  if (dt == PRISM_BF16)
    launch_pool<bf16_t>(qp, kp, bvalid, BH, nb, vol, d, w.qbar, w.kbar, s);
  else
    launch_pool<float>(qp, kp, bvalid, BH, nb, vol, d, w.qbar, w.kbar, s);
  const int tiles = (nb + 63) / 64;
  hipLaunchKernelGGL(k_scores, dim3(tiles, tiles, BH), dim3(256), 0, s, w.qbar, w.kbar, nb, d, scale, w.scores);
  hipLaunchKernelGGL(k_select, dim3(nb, BH), dim3(NT), size_t(nb) * 4, s, w.scores, bvalid, nb, p, p.k_max,
                     sel_idx, sel_cnt, sel_margin, w.bitmap);
  const int rows = BH * nb;
  hipLaunchKernelGGL(k_rev_count, dim3((rows + 255) / 256), dim3(256), 0, s, w.bitmap, nb, rows, w.rcnt);
  hipLaunchKernelGGL(k_rev_scan, dim3(BH), dim3(1024), 0, s, w.rcnt, nb, rev_ptr);
  hipLaunchKernelGGL(k_rev_fill, dim3(nb, BH), dim3(64), 0, s, w.bitmap, rev_ptr, nb, p.k_max, rev_idx);
  return hipGetLastError();
}

}  // namespace prism
