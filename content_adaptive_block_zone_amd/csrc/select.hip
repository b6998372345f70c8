// Block pooling and hybrid Top-k/Top-p block selection (Prism abstract: block-level
// features and a hybrid selection that fixes each query block's sparsity; Figure 2
// caption; Table 7 caption: Top-p keeps the smallest set of key blocks whose cumulative
// attention weight exceeds the threshold).
//
//   k_pool     mean of each block's valid rows (float32)                 HBM-bound
//   k_scores   scale * Qbar Kbar^T for one chunk of query blocks, on the bf16 matrix
//              cores with float32 accuracy (three-way bf16 split), 64x64 tiles
//   k_select   per query block, the row of scores in registers: softmax over live key
//              blocks, then the hybrid count found by bitwise search on the float bits
//              of the probabilities (no sort): the Top-p threshold is the largest
//              probability v whose "sum of probabilities >= v" still exceeds p; the Top-k
//              clamp is a count search.  Once few values remain in the searched range
//              they move to LDS and one wavefront finishes the search.  The kept set is
//              emitted in ascending block order, with a row of selection bits.
//   k_col_*    reverse index from those rows of bits, chunk by chunk: counts, then (after
//              k_rev_scan) ascending lists; no atomics, every output has one writer.
// Only one chunk of scores exists at a time (at most 256 MB), so no nb x nb matrix is
// ever formed.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int NT = 256;

struct SelWs {
  float* qbar;
  float* kbar;
  float* scores;
  uint32_t* rowbits;
  int32_t* rcnt;
  int32_t* cursor;
};

__host__ __device__ inline int words32(int nb) { return (nb + 31) / 32; }

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

// Scores of one chunk of query rows: out[bh][I - I0][J] = scale * sum_c qbar[bh][I][c]
// kbar[bh][J][c] for I0 <= I < I0 + rows; dead key blocks (no valid token) get -inf.
// 64x64 tile per workgroup; wave (wi, wj) forms rows 32wi.., columns 32wj.. on the bf16
// matrix cores (v_mfma_f32_32x32x16_bf16) with float32 accuracy: each float32 operand x
// is split into three bf16 pieces, x0 = bf16(x), x1 = bf16(x - x0), x2 = bf16(x - x0 -
// x1) (24 significant bits between them), and a product takes the six piece products
// x_i y_j with i + j <= 2, each exact in float32 and summed in float32; the terms left
// out are below 2^-24 of the product.  c runs in chunks of 32, split once while staged in
// LDS (three planes per operand, rows padded to 80 bytes: the 16-byte reads of the 32
// rows of one product fall on distinct banks).
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
constexpr int kScT = 64, kScK = 32, kScRow = kScK + 8;
__global__ __launch_bounds__(256) void k_scores(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                const int32_t* __restrict__ bvalid, int nb, int d, float scale,
                                                int I0, int rows, int CH, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) __bf16 As[3][kScT][kScRow];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[3][kScT][kScRow];
  const int bh = blockIdx.z;
  const int r0 = blockIdx.y * kScT;   // first row of the tile, relative to I0
  const int j0 = blockIdx.x * kScT;
  const float* Q = qbar + (size_t(bh) * nb + I0) * d;
  const float* K = kbar + size_t(bh) * nb * d;
  const int t = threadIdx.x, l = t & 63, w = t >> 6, wi = w & 1, wj = w >> 1;
  const int sr = t >> 3, sc = (t & 7) * 4;  // staging: rows sr, sr + 32, columns sc..sc+3
  auto split = [](float x, __bf16 (&pc)[3]) {
    pc[0] = (__bf16)x;
    const float r1 = x - (float)pc[0];
    pc[1] = (__bf16)r1;
    pc[2] = (__bf16)(r1 - (float)pc[1]);
  };
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  for (int k0 = 0; k0 < d; k0 += kScK) {
    // d is a multiple of 16: the second half of a 32-column stage may be past d
    const bool cin = k0 + sc < d;
    float4 a[2], b[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = sr + 32 * h;
      a[h] = cin && r0 + r < rows ? *reinterpret_cast<const float4*>(Q + size_t(r0 + r) * d + k0 + sc)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
      b[h] = cin && j0 + r < nb ? *reinterpret_cast<const float4*>(K + size_t(j0 + r) * d + k0 + sc)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = sr + 32 * h;
      const float av[4] = {a[h].x, a[h].y, a[h].z, a[h].w}, bv[4] = {b[h].x, b[h].y, b[h].z, b[h].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        __bf16 pa[3], pb[3];
        split(av[c], pa);
        split(bv[c], pb);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          As[i][r][sc + c] = pa[i];
          Bs[i][r][sc + c] = pb[i];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s16 = 0; s16 < kScK; s16 += 16) {
      const int col = s16 + 8 * (l >> 5);
      bf16x8s x[3], y[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        x[i] = *reinterpret_cast<const bf16x8s*>(&As[i][32 * wi + (l & 31)][col]);
        y[i] = *reinterpret_cast<const bf16x8s*>(&Bs[i][32 * wj + (l & 31)][col]);
      }
      // smallest terms first
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[2], y[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[1], y[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[0], y[2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[1], y[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[0], y[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[0], y[0], acc, 0, 0, 0);
    }
  }
  // lane l, register e: row 8(e/4) + 4(l/32) + e%4, column l%32 of the wave's 32x32 tile
  const int J = j0 + 32 * wj + (l & 31);
  if (J >= nb) return;
  const bool live = bvalid[size_t(bh) * nb + J] > 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int r = r0 + 32 * wi + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
    if (r < rows) out[(size_t(bh) * CH + r) * nb + J] = live ? acc[e] * scale : -INFINITY;
  }
}

// One workgroup per query block of the chunk, the row held in registers: thread t of a
// TPB-thread workgroup keeps key blocks t, t + TPB, t + 2 TPB, ... (VPT of them).
// Probabilities are searched as keys kk = bits(P) + 1 (live) or 0 (dead), bit by bit from
// the top.  A pass tests one candidate key over the whole row and also counts the values
// left in the range that the next bits can still split.  Once that range holds at most
// 4 TPB values they are compacted to LDS (in thread and register order) and the passes
// continue over them, four per thread, with the fixed sum and count of the values above
// the range added; once it holds at most kCand, they are compacted again and one
// wavefront finishes the remaining bits with wave sums.  Every sum runs in a fixed order,
// so results are deterministic.
// Ascending emission uses wave ballots per round of TPB blocks.  nb <= TPB * VPT.
constexpr int kCand = 64;  // one per lane of the finishing wavefront
__device__ __forceinline__ int below(uint64_t mask) {  // set bits of mask below this lane
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}
template <int TPB, int VPT>
__global__ __launch_bounds__(TPB) void k_select(const float* __restrict__ scores, const int32_t* __restrict__ bvalid,
                                               int nb, int I0, int CH, prism_select_params prm, int k_max,
                                               int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
                                               float* __restrict__ sel_margin, uint32_t* __restrict__ rowbits) {
  constexpr int NW = TPB / 64;
  __shared__ int redi[NW + 1];
  __shared__ float pv[2][NW][3];  // the passes alternate between two slots, so one barrier
  int par = 0;                    // per pass orders each write after the last reads
  __shared__ float cand[kCand];
  constexpr int NBV = 4, kMid = NBV * TPB;  // middle stage: NBV values per thread
  __shared__ float mid[kMid];
  __shared__ float found[4];
  const int I = I0 + blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t* bv = bvalid + size_t(bh) * nb;
  int32_t* out = sel_idx + (size_t(bh) * nb + I) * k_max;
  if (bv[I] == 0) {  // a dead query block selects nothing: its list and its row of bits
    for (int s = tid; s < k_max; s += TPB) out[s] = -1;
    uint32_t* rb = rowbits + (size_t(bh) * CH + blockIdx.x) * words32(nb);
    for (int s = tid; s < words32(nb); s += TPB) rb[s] = 0u;
    if (tid == 0) {
      sel_cnt[size_t(bh) * nb + I] = 0;
      if (sel_margin) sel_margin[size_t(bh) * nb + I] = 1.f;
    }
    return;
  }
  // three reductions over the workgroup behind one barrier (op 0: sum, 1: max, 2: min);
  // sums run over the waves in a fixed order
  auto wred = [&](float v, int op) { return op == 0 ? wave_sum(v) : op == 1 ? wave_max(v) : -wave_max(-v); };
  auto comb = [](float acc, float v, int op) { return op == 0 ? acc + v : op == 1 ? fmaxf(acc, v) : fminf(acc, v); };
  auto red3 = [&](float& a, float& b, float& c, int oa, int ob, int oc) {
    a = wred(a, oa);
    b = wred(b, ob);
    c = wred(c, oc);
    if (lane == 0) {
      pv[par][wv][0] = a;
      pv[par][wv][1] = b;
      pv[par][wv][2] = c;
    }
    __syncthreads();
    auto init = [](int op) { return op == 0 ? 0.f : op == 1 ? -INFINITY : INFINITY; };
    a = init(oa);
    b = init(ob);
    c = init(oc);
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      a = comb(a, pv[par][w2][0], oa);
      b = comb(b, pv[par][w2][1], ob);
      c = comb(c, pv[par][w2][2], oc);
    }
    par ^= 1;
  };
  auto pass3 = [&](float& a, float& b, float& c) { red3(a, b, c, 0, 0, 0); };
  const float* row = scores + (size_t(bh) * CH + blockIdx.x) * nb;
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
  float nlf = float(nl), unused0 = 0.f;  // counts up to 32768: exact in float
  red3(mx, nlf, unused0, 1, 0, 0);
  const int nlive = int(nlf);
  // exp on the hardware base-2 unit and one reciprocal: a few ulps from the correctly
  // rounded softmax, far inside the 1e-4 relative margin below which a decision counts as
  // a near-tie
  constexpr float kLog2e = 1.4426950408889634f;
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const float e = q[i] == -INFINITY ? -1.f : __builtin_amdgcn_exp2f((q[i] - mx) * kLog2e);
    q[i] = e;
    if (e >= 0.f) se += e;
  }
  {
    float u1 = 0.f, u2 = 0.f;
    pass3(se, u1, u2);
  }
  const float rse = __builtin_amdgcn_rcpf(se);
  float tot = 0.f, pmin = INFINITY, pmax = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    if (q[i] >= 0.f) {
      q[i] = q[i] * rse;
      tot += q[i];
      pmin = fminf(pmin, q[i]);
      pmax = fmaxf(pmax, q[i]);
    }
  const float p = prm.top_p;
  red3(tot, pmin, pmax, 0, 2, 1);
  // Top-p at p >= 1 keeps every live block: no proper prefix of weights summing to 1
  // exceeds 1, and a float32 total that rounds above 1 must not cut the tail.
  const bool cut_p = p < 1.f && tot > p;
  // For a live block kk >= c is P >= at(c - 1) and kk == c is P == at(c - 1) (at(u): the
  // float with bits u; probabilities are never -0 and the bit patterns of non-negative
  // floats are ordered like their values); a dead block's -1 fails every such test, as
  // its kk = 0 does (c >= 1 throughout).  The searches never accept a key above that of
  // 1.0 (when the target is at least one block), so every threshold compared is finite.
  auto at = [](uint32_t u) { return __uint_as_float(u); };

  // The largest key T with metric(T) > target (sum of P over kk >= T; top-p) or
  // metric(T) >= target (count of kk >= T; a count cut), and over kk > T the sum (sg) and
  // count (cg) and at kk == T the count (ce).  Counts come from wave ballots (exact, and
  // scalar work); the number of live keys in the open range [Tk, hi) follows from the
  // counts at its two ends.
  auto wcount = [&](bool pred) { return int(__builtin_popcountll(__builtin_amdgcn_ballot_w64(pred))); };
  auto search = [&](bool use_sum, float target, uint32_t& T_out, float& sg, float& cg, float& ce) {
    auto pass_ok = [&](float m) { return use_sum ? m > target : m >= target; };
    uint32_t Tk = 0, hi = 0x80000000u;  // the answer lies in [Tk, hi)
    float c_lo = float(nlive), c_hi = 0.f;  // live keys at or above Tk, at or above hi
    int bit = 30;
    // When the target is met at key 1 (a Top-p cut, or a count of at least one block) the
    // answer is the key of one of the row's probabilities, so it lies in [key(pmin),
    // key(pmax)]: the bits these two keys share are the answer's, and the search starts
    // below them.  Every live key is then at or above Tk and none reaches hi.
    if (nlive > 0 && (use_sum || target >= 1.f)) {
      const uint32_t klo = __float_as_uint(pmin) + 1u, khi = __float_as_uint(pmax) + 1u;
      const int b0 = 31 - __builtin_clz((klo ^ khi) | 1u);  // highest differing bit
      const uint32_t span = b0 >= 31 ? 0u : (1u << (b0 + 1));
      if (b0 < 30) {
        Tk = klo & ~(span - 1u);
        hi = Tk + span;
        bit = b0;
      }
    }
    // One pass: the metric at candidate key cnd over the values of `vals` (plus the fixed
    // sum fs0 and count ch0 of the values above them), then the range update.
    auto step = [&](const auto& vals, float fs0, float ch0) {
      constexpr int N = sizeof(vals) / sizeof(vals[0]);
      const uint32_t cnd = Tk | (1u << bit);
      const float c = at(cnd - 1u);
      float m = 0.f, unused = 0.f;
      int cwi = 0;  // wave-uniform: scalar work
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bool ge = vals[i] >= c;
        if (use_sum) m += ge ? vals[i] : 0.f;
        cwi += wcount(ge);
      }
      float cw = lane == 0 ? float(cwi) : 0.f;
      pass3(m, cw, unused);
      m += fs0;
      cw += ch0;
      if (pass_ok(use_sum ? m : cw)) {
        Tk = cnd;
        c_lo = cw;
      } else {
        hi = cnd;
        c_hi = cw;
      }
    };
    // every bit decided: the sums and counts at the answer
    auto conclude = [&](const auto& vals, float fs0, float ch0) {
      constexpr int N = sizeof(vals) / sizeof(vals[0]);
      const float above = at(Tk), equal = at(Tk - 1u);
      float s1 = 0.f;
      int c1i = 0, e1i = 0;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        s1 += vals[i] >= above ? vals[i] : 0.f;
        c1i += wcount(vals[i] >= above);
        e1i += wcount(vals[i] == equal);
      }
      float c1 = lane == 0 ? float(c1i) : 0.f, e1 = lane == 0 ? float(e1i) : 0.f;
      pass3(s1, c1, e1);
      T_out = Tk;
      sg = s1 + fs0;
      cg = c1 + ch0;
      ce = e1;
    };
    // the values of `vals` in [Tk, hi) to dst[0 .. cap) in thread and register order; the
    // sum of those at or above hi is added to fs.  Returns how many were written.
    auto compact = [&](const auto& vals, float* dst, int cap, float& fs) {
      constexpr int N = sizeof(vals) / sizeof(vals[0]);
      const float lo_v = Tk ? at(Tk - 1u) : 0.f;
      const bool hi_all = hi > 0x3F800001u;  // every live key is below hi
      const float hi_v = hi_all ? 0.f : at(hi - 1u);
      auto in_range = [&](float v) { return v >= 0.f && v >= lo_v && (hi_all || v < hi_v); };
      int mine = 0;
      float up = 0.f, u1 = 0.f, u2 = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        mine += in_range(vals[i]);
        up += !hi_all && vals[i] >= hi_v ? vals[i] : 0.f;
      }
      int total;
      int off = block_excl_scan<TPB>(mine, redi, &total);
      total = min(total, cap);  // at most c_lo - c_hi <= cap; NaN scores only lower it
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (in_range(vals[i]) && off < cap) dst[off++] = vals[i];
      pass3(up, u1, u2);  // its barrier also publishes dst
      fs += up;
      return total;
    };
    // at most kCand values left in range, in cand[]: one wavefront decides the remaining
    // bits with wave sums, adding the fixed sum fs and count c_hi of the values above
    auto finish = [&](int total, float fs) {
      if (wv == 0) {
        const float v = lane < total ? cand[lane] : -1.f;
        uint32_t T = Tk;
        for (int b = bit; b >= 0; --b) {
          const uint32_t cnd = T | (1u << b);
          const float c = at(cnd - 1u);
          const float m = wave_sum(v >= c ? (use_sum ? v : 1.f) : 0.f) + (use_sum ? fs : c_hi);
          if (pass_ok(m)) T = cnd;
        }
        const float above = at(T), equal = at(T - 1u);
        float s1 = v >= above ? v : 0.f, c1 = v >= above ? 1.f : 0.f, e1 = v == equal ? 1.f : 0.f;
        s1 = wave_sum(s1) + fs;
        c1 = wave_sum(c1) + c_hi;
        e1 = wave_sum(e1);
        if (lane == 0) {
          found[0] = __uint_as_float(T);
          found[1] = s1;
          found[2] = c1;
          found[3] = e1;
        }
      }
      __syncthreads();
      T_out = __float_as_uint(found[0]);
      sg = found[1];
      cg = found[2];
      ce = found[3];
      __syncthreads();  // found[] and cand[] are free again
    };

    // Passes over the whole row until at most kMid values remain in range
    bool done = true;
    for (; bit >= 0; --bit) {
      step(q, 0.f, 0.f);
      if (bit > 0 && c_lo - c_hi <= float(kMid)) {
        done = false;
        --bit;
        break;
      }
    }
    if (done) {
      conclude(q, 0.f, 0.f);
      return;
    }
    float fs = 0.f;
    if (c_lo - c_hi <= float(kCand)) {
      const int ncand = compact(q, cand, kCand, fs);
      finish(ncand, fs);
      return;
    }
    // then over those values, NBV per thread, the ones above them a fixed sum and count
    const int nmid = compact(q, mid, kMid, fs);
    float vb[NBV];
#pragma unroll
    for (int k = 0; k < NBV; ++k) {
      const int j = tid + TPB * k;
      vb[k] = j < nmid ? mid[j] : -1.f;
    }
    const float fs0 = fs, ch0 = c_hi;
    bool small = false;
    for (; bit >= 0; --bit) {
      step(vb, fs0, ch0);
      if (bit > 0 && c_lo - c_hi <= float(kCand)) {
        small = true;
        --bit;
        break;
      }
    }
    if (!small) {
      conclude(vb, fs0, ch0);
      return;
    }
    const int ncand = compact(vb, cand, kCand, fs);
    finish(ncand, fs);
  };

  // ---- Top-p: largest key v with sum(P >= v) > p
  int n_p = nlive, need_p = 0, ce_p = 0;
  uint32_t vstar = 0;
  float sum_gt_p = 0.f;
  if (cut_p) {
    uint32_t Tk;
    float sg, cgf, cef;
    search(true, p, Tk, sg, cgf, cef);
    vstar = Tk - 1u;  // Tk >= 1: all live blocks have kk >= 1 and sum to tot > p
    const int cg = int(cgf), ce = int(cef);
    ce_p = ce;
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
  int need_eq, ce_cut;  // blocks to keep at the cut's key, and how many have it
  if (n == n_p && cut_p) {
    Tcut = vstar + 1u;
    need_eq = need_p;
    ce_cut = ce_p;
  } else {
    float sg, cgf, cef;
    search(false, float(n), Tcut, sg, cgf, cef);
    need_eq = n - int(cgf);
    ce_cut = int(cef);
  }

  // ---- emit ascending.  Block order is (round i, wave, lane).  Each wave counts its
  // equal-key blocks per round (ballots); lane i of every wave then holds the number of
  // such blocks that precede round i of this wave (a scan over rounds plus the earlier
  // waves of round i), which the lanes of round i read back with readlane.  The same is
  // done for the taken blocks.
  __shared__ int wcnt[2][NW][VPT];  // per wave and round: equal-key count, taken count
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
  // When every block at the cut's key is kept (all but exact ties split by the cut), the
  // taken set is P >= cut_eq and the ranks of the equal keys are not needed.
  const bool all_eq = need_eq >= ce_cut;
  int eqo = 0;
  if (!all_eq) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const uint64_t eq = __builtin_amdgcn_ballot_w64(q[i] == cut_eq);
      if (lane == 0) wcnt[0][wv][i] = __builtin_popcountll(eq);
    }
    __syncthreads();
    eqo = offsets(0);
  }
  // taken: above the cut, or at it and among the first need_eq such blocks in block order
  auto take_at = [&](int i) {
    if (all_eq) return q[i] >= cut_eq;
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
  // this query block's row of the chunk's bit matrix: bit J of words32(nb) words, written
  // whole by the wave whose 64 lanes hold key blocks J0 .. J0 + 63 (J0 a multiple of 64)
  const int WN = words32(nb);
  uint32_t* rbits = rowbits + (size_t(bh) * CH + blockIdx.x) * WN;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const bool tk = take_at(i);
    const uint64_t tkm = __builtin_amdgcn_ballot_w64(tk);
    const int pos = __builtin_amdgcn_readlane(tko, i) + below(tkm);
    const int J = tid + TPB * i;
    const int wd = (J - lane) / 32 + (lane >> 5);  // lane 0: low word, lane 32: high word
    if ((lane & 31) == 0 && wd < WN) rbits[wd] = lane ? uint32_t(tkm >> 32) : uint32_t(tkm);
    if (tk) {
      out[pos] = J;
      pmin_sel = fminf(pmin_sel, q[i]);
    } else if (q[i] >= 0.f) {  // live
      pmax_uns = fmaxf(pmax_uns, q[i]);
    }
  }
  for (int s = tot_sel + tid; s < k_max; s += TPB) out[s] = -1;
  if (sel_margin) {
    float u = 0.f;
    red3(pmin_sel, pmax_uns, u, 2, 1, 0);
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

// Reverse index, built chunk by chunk.  The selection kernel leaves each query block's
// selected key blocks as a row of bits (rowbits [BH][CH][words32(nb)]).  One wavefront
// per (head, 32 key blocks) reads the matching word of every row of the chunk, 64 rows
// at a time, and turns them into columns with one ballot per key block: lane j then
// holds the 64 bits of key block 32 gj + j for those rows.  Pass one counts them into the
// key block's total; pass two (after the scan) lists them.  Every output has one writer.
__global__ __launch_bounds__(256) void k_col_count(const uint32_t* __restrict__ rowbits, int nb, int CH, int rows,
                                                   int32_t* __restrict__ rcnt) {
  const int WN = words32(nb), lane = threadIdx.x & 63;
  const int gj = blockIdx.x * 4 + (threadIdx.x >> 6), bh = blockIdx.y;
  if (gj >= WN) return;
  const uint32_t* rb = rowbits + size_t(bh) * CH * WN + gj;
  int cnt = 0;
  for (int r0 = 0; r0 < rows; r0 += 64) {
    const uint32_t w = r0 + lane < rows ? rb[size_t(r0 + lane) * WN] : 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int c = __builtin_popcountll(__builtin_amdgcn_ballot_w64((w >> j) & 1u));
      if (lane == j) cnt += c;
    }
  }
  const int J = 32 * gj + lane;
  if (lane < 32 && J < nb) rcnt[size_t(bh) * nb + J] += cnt;
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

// Pass two: a query block's row of bits again, from its selection list, built in LDS.
template <int MAXW>
__global__ __launch_bounds__(256) void k_rowbits(const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
                                                int nb, int k_max, int I0, int CH, uint32_t* __restrict__ rowbits) {
  __shared__ uint32_t sb[MAXW];
  const int r = blockIdx.x, bh = blockIdx.y, I = I0 + r;
  const int WN = words32(nb);
  for (int w = threadIdx.x; w < WN; w += 256) sb[w] = 0u;
  __syncthreads();
  const int n = clampi(sel_cnt[size_t(bh) * nb + I], 0, k_max);
  const int32_t* lst = sel_idx + (size_t(bh) * nb + I) * k_max;
  for (int s2 = threadIdx.x; s2 < n; s2 += 256) {
    const int J = lst[s2];
    if (J >= 0 && J < nb) atomicOr(&sb[J >> 5], 1u << (J & 31));
  }
  __syncthreads();
  uint32_t* out = rowbits + (size_t(bh) * CH + r) * WN;
  for (int w = threadIdx.x; w < WN; w += 256) out[w] = sb[w];
}

// As k_col_count, then lane j appends the chunk's query blocks of key block 32 gj + j
// (ascending) at its cursor.  Chunks run in ascending order of I0, so every reverse list
// comes out ascending.
__global__ __launch_bounds__(256) void k_col_fill(const uint32_t* __restrict__ rowbits, const int32_t* __restrict__ rev_ptr,
                                                  int32_t* __restrict__ cursor, int nb, int k_max, int I0, int CH,
                                                  int rows, int32_t* __restrict__ rev_idx) {
  const int WN = words32(nb), lane = threadIdx.x & 63;
  const int gj = blockIdx.x * 4 + (threadIdx.x >> 6), bh = blockIdx.y;
  if (gj >= WN) return;
  const int J = 32 * gj + lane;
  const bool owner = lane < 32 && J < nb;
  const uint32_t* rb = rowbits + size_t(bh) * CH * WN + gj;
  int32_t* out = rev_idx + size_t(bh) * nb * k_max;
  const int cur = owner ? cursor[size_t(bh) * nb + J] : 0;
  int pos = owner ? rev_ptr[size_t(bh) * (nb + 1) + J] + cur : 0;
  int added = 0;
  for (int r0 = 0; r0 < rows; r0 += 64) {
    const uint32_t w = r0 + lane < rows ? rb[size_t(r0 + lane) * WN] : 0u;
    uint64_t col = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint64_t m = __builtin_amdgcn_ballot_w64((w >> j) & 1u);
      if (lane == j) col = m;
    }
    if (owner) {
      while (col) {
        const int b = __builtin_ctzll(col);
        out[pos++] = I0 + r0 + b;
        ++added;
        col &= col - 1;
      }
    }
  }
  if (owner) cursor[size_t(bh) * nb + J] = cur + added;
}

}  // namespace

// Query blocks per chunk of the selection (every head at once): as many as keep the
// chunk's scores, [BH][CH][nb] float32, within 256 MB (the size of the last-level cache,
// where they stay between the score and the selection kernels), in multiples of 64 and
// never fewer than 512.  The workspace is therefore bounded by max(256 MB, 2 KB * BH *
// nb) plus terms linear in nb: it grows linearly with nb, never as nb^2.
constexpr size_t kSelChunkBytes = size_t(256) << 20;
constexpr int kSelChunkMin = 512;
static int sel_chunk(int BH, int nb) {
  const size_t fit = kSelChunkBytes / (size_t(BH) * nb * 4) / 64 * 64;
  const int ch = int(fit > size_t(kSelChunkMin) ? (fit < size_t(nb) ? fit : size_t(nb)) : size_t(kSelChunkMin));
  return ch < nb ? ch : nb;
}

// Workspace layout: [pooled Q, pooled K,] chunk scores, chunk row bits, reverse counts,
// reverse cursors.  The pooled means are absent when the caller
// passes them in (prism_select_blocks_pooled).
static SelWs carve(void* ws, int BH, int nb, int d, bool with_pooled) {
  char* p = static_cast<char*>(ws);
  const int CH = sel_chunk(BH, nb);
  SelWs w{};
  if (with_pooled) {
    w.qbar = reinterpret_cast<float*>(p);
    p += align256(size_t(BH) * nb * d * 4);
    w.kbar = reinterpret_cast<float*>(p);
    p += align256(size_t(BH) * nb * d * 4);
  }
  w.scores = reinterpret_cast<float*>(p);
  p += align256(size_t(BH) * CH * nb * 4);
  w.rowbits = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(BH) * CH * words32(nb) * 4);
  w.rcnt = reinterpret_cast<int32_t*>(p);
  p += align256(size_t(BH) * nb * 4);
  w.cursor = reinterpret_cast<int32_t*>(p);
  return w;
}

size_t select_ws_bytes(int BH, int nb, int d, bool with_pooled) {
  const int CH = sel_chunk(BH, nb);
  return (with_pooled ? 2 * align256(size_t(BH) * nb * d * 4) : 0) + align256(size_t(BH) * CH * nb * 4) +
         align256(size_t(BH) * CH * words32(nb) * 4) + 2 * align256(size_t(BH) * nb * 4);
}

template <int TPB, int VPT>
static void launch_select_chunk(const SelWs& w, const int32_t* bvalid, int BH, int nb, int I0, int rows, int CH,
                                const prism_select_params& p, int32_t* sel_idx, int32_t* sel_cnt, float* sel_margin,
                                hipStream_t s) {
  hipLaunchKernelGGL((k_select<TPB, VPT>), dim3(rows, BH), dim3(TPB), 0, s, w.scores, bvalid, nb, I0, CH, p, p.k_max,
                     sel_idx, sel_cnt, sel_margin, w.rowbits);
}

// Scores, hybrid cut and reverse index from pooled means qbar, kbar [BH][nb][d] float32,
// one chunk of query blocks at a time.
static void launch_select_core(const float* qbar, const float* kbar, const int32_t* bvalid, int BH, int nb, int d,
                               float scale, const prism_select_params& p, int32_t* sel_idx, int32_t* sel_cnt,
                               int32_t* rev_ptr, int32_t* rev_idx, float* sel_margin, const SelWs& w, hipStream_t s) {
  const int CH = sel_chunk(BH, nb), WN = words32(nb), rows_all = BH * nb;
  const dim3 cols((WN + 3) / 4, BH);  // one wavefront per 32 key blocks
  hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(w.rcnt), size_t(rows_all), 0u);
  hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(w.cursor), size_t(rows_all),
                     0u);
  hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint32_t*>(rev_idx),
                     size_t(BH) * nb * p.k_max, 0xffffffffu);
  for (int I0 = 0; I0 < nb; I0 += CH) {
    const int rows = min(CH, nb - I0);
    hipLaunchKernelGGL(k_scores, dim3((nb + kScT - 1) / kScT, (rows + kScT - 1) / kScT, BH), dim3(256), 0, s, qbar,
                       kbar, bvalid, nb, d, scale, I0, rows, CH, w.scores);
    // Workgroup shapes as measured fastest: 256 lanes up to 32 blocks each, then 512 lanes
    // of 32 (at 64 per lane the register file allows one wave per SIMD), then 1024 lanes of
    // 32.  nb <= 1024 * 32 is checked by the caller.
    if (nb <= 256 * 8)
      launch_select_chunk<256, 8>(w, bvalid, BH, nb, I0, rows, CH, p, sel_idx, sel_cnt, sel_margin, s);
    else if (nb <= 256 * 16)
      launch_select_chunk<256, 16>(w, bvalid, BH, nb, I0, rows, CH, p, sel_idx, sel_cnt, sel_margin, s);
    else if (nb <= 256 * 32)
      launch_select_chunk<256, 32>(w, bvalid, BH, nb, I0, rows, CH, p, sel_idx, sel_cnt, sel_margin, s);
    else if (nb <= 512 * 32)
      launch_select_chunk<512, 32>(w, bvalid, BH, nb, I0, rows, CH, p, sel_idx, sel_cnt, sel_margin, s);
    else
      launch_select_chunk<1024, 32>(w, bvalid, BH, nb, I0, rows, CH, p, sel_idx, sel_cnt, sel_margin, s);
    hipLaunchKernelGGL(k_col_count, cols, dim3(256), 0, s, w.rowbits, nb, CH, rows, w.rcnt);
  }
  hipLaunchKernelGGL(k_rev_scan, dim3(BH), dim3(1024), 0, s, w.rcnt, nb, rev_ptr);
  for (int I0 = 0; I0 < nb; I0 += CH) {
    const int rows = min(CH, nb - I0);
    hipLaunchKernelGGL(k_rowbits<kMaxSelectNb / 32>, dim3(rows, BH), dim3(256), 0, s, sel_idx, sel_cnt, nb, p.k_max,
                       I0, CH, w.rowbits);
    hipLaunchKernelGGL(k_col_fill, cols, dim3(256), 0, s, w.rowbits, rev_ptr, w.cursor, nb, p.k_max, I0, CH, rows,
                       rev_idx);
  }
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
