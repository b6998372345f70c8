// Block pooling and hybrid Top-k/Top-p block selection (Prism abstract: block-level
// features and a hybrid selection that fixes each query block's sparsity; Figure 2
// caption; Table 7 caption: Top-p keeps the smallest set of key blocks whose cumulative
// attention weight exceeds the threshold).
//
//   k_pool    mean of each block's valid rows (float32)           HBM-bound
//   k_scores  scale * Qbar Kbar^T per head, 128x128 tiles, 8x8 per thread   fp32 ALU
//   k_select_reg  per query block, the row of scores in registers: softmax over live
//             key blocks, then the hybrid count found by bitwise search on the float bits
//             of the probabilities (no sort): the Top-p threshold is the largest
//             probability v whose "sum of probabilities >= v" still exceeds p; the Top-k
//             clamp is a count search.  The kept set is emitted in ascending block order
//             and marked in a bitmap for the reverse index.
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

// Workspace layout: [pooled Q, pooled K,] scores, bitmap, reverse counts.  The pooled
// means are absent when the caller passes them in (prism_select_blocks_pooled).
SelWs carve(void* ws, int BH, int nb, int d, bool with_pooled) {
  char* p = static_cast<char*>(ws);
  SelWs w{};
  if (with_pooled) {
    w.qbar = reinterpret_cast<float*>(p);
    p += align256(size_t(BH) * nb * d * 4);
    w.kbar = reinterpret_cast<float*>(p);
    p += align256(size_t(BH) * nb * d * 4);
  }
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
// Dead key blocks (no valid token) get the score -inf.
// 128x128 tile per workgroup, 8x8 per thread (rows ty + 16i, columns tx + 16j), c in
// chunks of 16 staged in LDS: four FMAs per LDS value read.  Each score sums its d
// products in order of c, one fused multiply-add at a time.
constexpr int kScT = 128;
__global__ __launch_bounds__(256) void k_scores(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                const int32_t* __restrict__ bvalid, int nb, int d, float scale,
                                                float* __restrict__ scores) {
  __shared__ float As[16][kScT];
  __shared__ float Bs[16][kScT];
  const int bh = blockIdx.z;
  const int I0 = blockIdx.y * kScT, J0 = blockIdx.x * kScT;
  const float* Q = qbar + size_t(bh) * nb * d;
  const float* K = kbar + size_t(bh) * nb * d;
  const int t = threadIdx.x, ty = t / 16, tx = t % 16;
  const int lr = t / 4, lc = (t % 4) * 4;  // staging: rows lr and lr + 64, columns lc..lc+3
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < d; k0 += 16) {
    float4 a[2], b[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 64 * h;
      a[h] = I0 + r < nb ? *reinterpret_cast<const float4*>(Q + size_t(I0 + r) * d + k0 + lc) : make_float4(0.f, 0.f, 0.f, 0.f);
      b[h] = J0 + r < nb ? *reinterpret_cast<const float4*>(K + size_t(J0 + r) * d + k0 + lc) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lr + 64 * h;
      As[lc + 0][r] = a[h].x; As[lc + 1][r] = a[h].y; As[lc + 2][r] = a[h].z; As[lc + 3][r] = a[h].w;
      Bs[lc + 0][r] = b[h].x; Bs[lc + 1][r] = b[h].y; Bs[lc + 2][r] = b[h].z; Bs[lc + 3][r] = b[h].w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float ar[8], br[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ar[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 8; ++j) br[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
    }
  }
  const int32_t* bv = bvalid + size_t(bh) * nb;
  bool live[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int J = J0 + tx + 16 * j;
    live[j] = J < nb && bv[J] > 0;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int I = I0 + ty + 16 * i;
    if (I >= nb) continue;
    float* row = scores + (size_t(bh) * nb + I) * nb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int J = J0 + tx + 16 * j;
      if (J < nb) row[J] = live[j] ? acc[i][j] * scale : -INFINITY;
    }
  }
}


// One workgroup per query block, the row held in registers: thread t of a TPB-thread
// workgroup keeps key blocks t, t + TPB, t + 2 TPB, ... (VPT of them), so that the 31-step
// searches are register passes.  Sums run over each thread's blocks in that order, then
// across the workgroup, so results are deterministic.  Ascending emission uses wave
// ballots per round of TPB blocks.  Used for nb <= TPB * VPT (at most 1024 * 32).
__device__ __forceinline__ int below(uint64_t mask) {  // set bits of mask below this lane
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}
template <int TPB, int VPT>
__global__ __launch_bounds__(TPB) void k_select_reg(const float* __restrict__ scores, const int32_t* __restrict__ bvalid,
                                                   int nb, prism_select_params prm, int k_max,
                                                   int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
                                                   float* __restrict__ sel_margin, uint32_t* __restrict__ bitmap) {
  constexpr int NW = TPB / 64;
  __shared__ float redf[NW];
  __shared__ int redi[NW];
  __shared__ float pf[2][NW];  // the search passes alternate between two slots, so one
  __shared__ int pi[2][NW];    // barrier per pass orders each write after the last reads
  int par = 0;
  auto pass_sum = [&](float v) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) pf[par][threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) t += pf[par][w2];
    par ^= 1;
    return t;
  };
  auto pass_sum_i = [&](int v) {
    v = wave_sum_i(v);
    if ((threadIdx.x & 63) == 0) pi[par][threadIdx.x >> 6] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) t += pi[par][w2];
    par ^= 1;
    return t;
  };
  __shared__ int wcnt[2][NW][VPT];  // per wave and round: equal-key count, taken count
  const int I = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t* bv = bvalid + size_t(bh) * nb;
  int32_t* out = sel_idx + (size_t(bh) * nb + I) * k_max;
  if (bv[I] == 0) {
    for (int s = tid; s < k_max; s += TPB) out[s] = -1;
    if (tid == 0) {
      sel_cnt[size_t(bh) * nb + I] = 0;
      if (sel_margin) sel_margin[size_t(bh) * nb + I] = 1.f;
    }
    return;
  }
  const float* row = scores + (size_t(bh) * nb + I) * nb;
  float q[VPT];  // logit, then exp, then probability; -1 for dead (or absent) key blocks
  float mx = -INFINITY;
  int nl = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int J = tid + TPB * i;
    const float l = J < nb ? row[J] : -INFINITY;  // -inf: dead key block (k_scores)
    q[i] = l;
    mx = fmaxf(mx, l);
    nl += l != -INFINITY;
  }
  mx = block_max<TPB>(mx, redf);
  const int nlive = block_sum_i<TPB>(nl, redi);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const float e = q[i] == -INFINITY ? -1.f : expf(q[i] - mx);
    q[i] = e;
    if (e >= 0.f) se += e;
  }
  se = block_sum<TPB>(se, redf);
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    if (q[i] >= 0.f) {
      q[i] = q[i] / se;
      tot += q[i];
    }
  const float p = prm.top_p;
  tot = block_sum<TPB>(tot, redf);
  // Top-p at p >= 1 keeps every live block: no proper prefix of weights summing to 1
  // exceeds 1, and a float32 total that rounds above 1 must not cut the tail.
  const bool cut_p = p < 1.f && tot > p;
  // The searches run over keys kk = bits(P) + 1 for live blocks and 0 for dead ones, so
  // they find key + 1.  Probabilities are never -0 and the bit patterns of non-negative
  // floats are ordered like their values, so for a live block kk >= c is P >= at(c - 1)
  // and kk == c is P == at(c - 1) (at(u): the float with bits u); a dead block's -1 fails
  // every such comparison, as its kk = 0 does (c >= 1 throughout).  The searches never
  // accept a key above that of 1.0, so every threshold compared is finite.  The
  // comparisons therefore run on q itself and no keys are kept.
  auto at = [](uint32_t u) { return __uint_as_float(u); };

  // ---- Top-p: largest key v with sum(P >= v) > p
  int n_p = nlive, need_p = 0;
  uint32_t vstar = 0;
  float sum_gt_p = 0.f;
  if (cut_p) {
    uint32_t Tk = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = Tk | (1u << bit);
      const float c = at(cand - 1u);
      float sm = 0.f;
#pragma unroll
      for (int i = 0; i < VPT; ++i) sm += q[i] >= c ? q[i] : 0.f;
      sm = pass_sum(sm);
      if (sm > p) Tk = cand;
    }
    vstar = Tk - 1u;  // Tk >= 1: all live blocks have kk >= 1 and sum to tot > p
    float sg = 0.f;
    int cg = 0, ce = 0;
    const float above = at(Tk), equal = at(Tk - 1u);  // kk > Tk, kk == Tk
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      sg += q[i] >= above ? q[i] : 0.f;
      cg += q[i] >= above;
      ce += q[i] == equal;
    }
    sg = block_sum<TPB>(sg, redf);
    cg = block_sum_i<TPB>(cg, redi);
    ce = block_sum_i<TPB>(ce, redi);
    const float v = __uint_as_float(vstar);
    int m = 1;
    while (m < ce && !(sg + float(m) * v > p)) ++m;
    n_p = cg + m;
    need_p = m;
    sum_gt_p = sg;
  }
  const int n = min(min(max(n_p, prm.k_min), prm.k_max), nlive);

  // ---- cut threshold (as kk) for exactly n kept blocks
  uint32_t Tcut;
  int need_eq;
  if (n == n_p && cut_p) {
    Tcut = vstar + 1u;
    need_eq = need_p;
  } else {
    uint32_t Tk = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = Tk | (1u << bit);
      const float cf = at(cand - 1u);
      int c = 0;
#pragma unroll
      for (int i = 0; i < VPT; ++i) c += q[i] >= cf;
      c = pass_sum_i(c);
      if (c >= n) Tk = cand;
    }
    Tcut = Tk;
    int cg = 0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) cg += q[i] >= at(Tk);
    cg = block_sum_i<TPB>(cg, redi);
    need_eq = n - cg;
  }

  // ---- emit ascending.  Block order is (round i, wave, lane).  Each wave counts its
  // equal-key blocks per round (ballots); lane i of every wave then holds the number of
  // such blocks that precede round i of this wave (a scan over rounds plus the earlier
  // waves of round i), which the lanes of round i read back with readlane.  The same is
  // done for the taken blocks.
  auto offsets = [&](int k2) {  // lane i < VPT: blocks of kind k2 before (round i, this wave)
    int tot_i = 0, before_i = 0;
    if (lane < VPT) {
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        const int c = wcnt[k2][w2][lane];
        tot_i += c;
        before_i += w2 < wv ? c : 0;
      }
    }
    int incl = tot_i;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int nn = __shfl_up(incl, o, 64);
      if (lane >= o) incl += nn;
    }
    return incl - tot_i + before_i;
  };
  const float cut_eq = at(Tcut - 1u), cut_above = at(Tcut);  // kk == Tcut, kk > Tcut
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const uint64_t eq = __builtin_amdgcn_ballot_w64(q[i] == cut_eq);
    if (lane == 0) wcnt[0][wv][i] = __builtin_popcountll(eq);
  }
  __syncthreads();
  const int eqo = offsets(0);
  // taken: above the cut, or at it and among the first need_eq such blocks in block order
  auto take_at = [&](int i) {
    const bool isq = q[i] == cut_eq;
    const int rank = __builtin_amdgcn_readlane(eqo, i) + below(__builtin_amdgcn_ballot_w64(isq));
    return q[i] >= cut_above || (isq && rank < need_eq);
  };
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const uint64_t tk = __builtin_amdgcn_ballot_w64(take_at(i));
    if (lane == 0) wcnt[1][wv][i] = __builtin_popcountll(tk);
  }
  __syncthreads();
  const int tko = offsets(1);
  int tot_sel = 0;
  if (lane < VPT) {
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) tot_sel += wcnt[1][w2][lane];
  }
  tot_sel = wave_sum_i(tot_sel);
  float pmin_sel = INFINITY, pmax_uns = -INFINITY;
  uint32_t* bm = bitmap + size_t(bh) * nb * words32(nb);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const bool tk = take_at(i);
    const int pos = __builtin_amdgcn_readlane(tko, i) + below(__builtin_amdgcn_ballot_w64(tk));
    const int J = tid + TPB * i;
    if (tk) {
      out[pos] = J;
      atomicOr(bm + size_t(J) * words32(nb) + (I >> 5), 1u << (I & 31));
      pmin_sel = fminf(pmin_sel, q[i]);
    } else if (q[i] >= 0.f) {  // live
      pmax_uns = fmaxf(pmax_uns, q[i]);
    }
  }
  for (int s = tot_sel + tid; s < k_max; s += TPB) out[s] = -1;
  if (sel_margin) {
    pmin_sel = -block_max<TPB>(-pmin_sel, redf);
    pmax_uns = block_max<TPB>(pmax_uns, redf);
  }
  if (tid == 0) {
    sel_cnt[size_t(bh) * nb + I] = tot_sel;
    if (sel_margin) {
      float mg = n < nlive ? (pmin_sel - pmax_uns) / pmin_sel : 1.f;
      if (cut_p && n == n_p) {
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

size_t select_ws_bytes(int BH, int nb, int d, bool with_pooled) {
  return (with_pooled ? 2 * align256(size_t(BH) * nb * d * 4) : 0) + align256(size_t(BH) * nb * nb * 4) +
         align256(size_t(BH) * nb * words32(nb) * 4) + align256(size_t(BH) * nb * 4);
}

// Scores, hybrid cut and reverse index from pooled means qbar, kbar [BH][nb][d] float32.
static void launch_select_core(const float* qbar, const float* kbar, const int32_t* bvalid, int BH, int nb, int d,
                               float scale, const prism_select_params& p, int32_t* sel_idx, int32_t* sel_cnt,
                               int32_t* rev_ptr, int32_t* rev_idx, float* sel_margin, const SelWs& w, hipStream_t s) {
  const size_t nbits = size_t(BH) * nb * words32(nb);
  hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, s, w.bitmap, nbits, 0u);
  hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(rev_idx),
                     size_t(BH) * nb * p.k_max, 0xffffffffu);
  const int tiles = (nb + kScT - 1) / kScT;
  hipLaunchKernelGGL(k_scores, dim3(tiles, tiles, BH), dim3(256), 0, s, qbar, kbar, bvalid, nb, d, scale, w.scores);
  // Workgroup shapes as measured fastest: 256 lanes up to 32 blocks each, then 512 lanes of
  // 32 (at 64 per lane the register file allows one wave per SIMD), then 1024 lanes of 32
  // (at most 128 registers per lane, which the kernel fits).  nb <= 1024 * 32 is checked
  // by the caller.
  const dim3 sg(nb, BH);
  if (nb <= 256 * 8)
    hipLaunchKernelGGL((k_select_reg<256, 8>), sg, dim3(256), 0, s, w.scores, bvalid, nb, p, p.k_max, sel_idx,
                       sel_cnt, sel_margin, w.bitmap);
  else if (nb <= 256 * 16)
    hipLaunchKernelGGL((k_select_reg<256, 16>), sg, dim3(256), 0, s, w.scores, bvalid, nb, p, p.k_max, sel_idx,
                       sel_cnt, sel_margin, w.bitmap);
  else if (nb <= 256 * 32)
    hipLaunchKernelGGL((k_select_reg<256, 32>), sg, dim3(256), 0, s, w.scores, bvalid, nb, p, p.k_max, sel_idx,
                       sel_cnt, sel_margin, w.bitmap);
  else if (nb <= 512 * 32)
    hipLaunchKernelGGL((k_select_reg<512, 32>), sg, dim3(512), 0, s, w.scores, bvalid, nb, p, p.k_max, sel_idx,
                       sel_cnt, sel_margin, w.bitmap);
  else
    hipLaunchKernelGGL((k_select_reg<1024, 32>), sg, dim3(1024), 0, s, w.scores, bvalid, nb, p, p.k_max, sel_idx,
                       sel_cnt, sel_margin, w.bitmap);
  const int rows = BH * nb;
  hipLaunchKernelGGL(k_rev_count, dim3((rows + 255) / 256), dim3(256), 0, s, w.bitmap, nb, rows, w.rcnt);
  hipLaunchKernelGGL(k_rev_scan, dim3(BH), dim3(1024), 0, s, w.rcnt, nb, rev_ptr);
  hipLaunchKernelGGL(k_rev_fill, dim3(nb, BH), dim3(64), 0, s, w.bitmap, rev_ptr, nb, p.k_max, rev_idx);
}

hipError_t launch_select(const void* qp, const void* kp, prism_dtype dt, const int32_t* bvalid,
                         int BH, int nb, int vol, int d, float scale, const prism_select_params& p,
                         int32_t* sel_idx, int32_t* sel_cnt, int32_t* rev_ptr, int32_t* rev_idx,
                         float* sel_margin, void* ws, hipStream_t s) {
  const SelWs w = carve(ws, BH, nb, d, true);
  // d is one of 32, 64, 128, 256 (checked by the caller)
  if (dt == PRISM_BF16)
    launch_pool<bf16_t>(qp, kp, bvalid, BH, nb, vol, d, w.qbar, w.kbar, s);
  else
    launch_pool<float>(qp, kp, bvalid, BH, nb, vol, d, w.qbar, w.kbar, s);
  launch_select_core(w.qbar, w.kbar, bvalid, BH, nb, d, scale, p, sel_idx, sel_cnt, rev_ptr, rev_idx, sel_margin, w,
                     s);
  return hipGetLastError();
}

hipError_t launch_select_pooled(const float* qbar, const float* kbar, const int32_t* bvalid, int BH, int nb, int d,
                                float scale, const prism_select_params& p, int32_t* sel_idx, int32_t* sel_cnt,
                                int32_t* rev_ptr, int32_t* rev_idx, float* sel_margin, void* ws, hipStream_t s) {
  const SelWs w = carve(ws, BH, nb, d, false);
  launch_select_core(qbar, kbar, bvalid, BH, nb, d, scale, p, sel_idx, sel_cnt, rev_ptr, rev_idx, sel_margin, w, s);
  return hipGetLastError();
}

}  // namespace prism
