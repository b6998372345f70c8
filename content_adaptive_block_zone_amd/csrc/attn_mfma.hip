// Block-sparse attention on the bf16 matrix cores of gfx950 (Prism Figure 2 caption: exact
// softmax attention over the selected blocks), for 64-token blocks and d = 128.
//
// Design.  One wavefront owns one 64-row block for the whole kernel (query block in the
// forward and dQ kernels, key block in the dK/dV kernel) and keeps its accumulators in
// registers; there is no cross-wave sharing to pay for, because the key lists of
// neighbouring query blocks barely overlap.  All products use v_mfma_f32_32x32x16_bf16.
// Scores are formed transposed where that keeps the softmax reductions inside a lane:
// S^T = K Q^T puts one query per lane column, so a row max / row sum is 32 in-lane values
// plus one swap with lane^32.  The accumulator of a 32x32 tile holds, in lane l and
// register e, row 8*(e/4) + 4*(l/32) + e%4 of column l%32; read eight registers at a time
// it is directly the B operand of the next product whose contraction runs over those
// rows, provided the other operand lists the rows in the same order.  That order
// ("kappa": rows 0-3, 8-11 for lane half 0 and 4-7, 12-15 for lane half 1 in each group
// of 16) is produced by k_transpose, which writes each 64x128 block as [128][64] with
// position p holding row kappa(p) (bits 2 and 3 of p swapped).  So every operand load is a
// 16-byte row segment: K, Q, V, dO row-major for the first products, and the transposed
// copies V^T (forward), K^T (dQ), Q^T and dO^T (dK/dV) for the second ones.
#include "prism_internal.h"

namespace prism {

int attn_mfma_supported(const AttnArgs& a, prism_dtype dt);
hipError_t launch_attn_fwd_mfma(const AttnArgs& a, void* ws, hipStream_t s);
hipError_t launch_attn_bwd_mfma(const AttnArgs& a, void* ws, hipEvent_t* marks, hipStream_t s);
size_t attn_mfma_ws_bytes(int BH, int nb, int copies);

namespace {

constexpr int D = 128;
constexpr int TR = 64;  // rows per block tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }
__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 ld8h(const uint16_t* p) {
  return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}
// Registers 8*h .. 8*h+7 of an accumulator as a bf16 operand (rows in kappa order).
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int h) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)c[8 * h + e];
  return r;
}
// The same as an fp16 operand (probabilities in [0, 1] keep 11 significant bits).
__device__ __forceinline__ f16x8 pack8h(const f32x16& c, int h) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)c[8 * h + e];
  return r;
}
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}
// Store registers 4j..4j+3 (four consecutive rows of a column) as 4 bf16 at p.
__device__ __forceinline__ void st4(bf16_t* p, const f32x16& c, int j, float s) {
  u32x2 v = {pk2(c[4 * j] * s, c[4 * j + 1] * s), pk2(c[4 * j + 2] * s, c[4 * j + 3] * s)};
  *reinterpret_cast<u32x2*>(p) = v;
}
__device__ __forceinline__ int acc_row(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }
__device__ __forceinline__ int kappa(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

__device__ __forceinline__ int nrows_of(const AttnArgs& a, int bh, int I) {
  return a.dense ? min(TR, a.nrows - I * TR) : a.bvalid[size_t(bh) * a.nb + I];
}
__device__ __forceinline__ size_t row0_of(const AttnArgs& a, int bh, int I) {
  return size_t(bh) * a.nrows + size_t(I) * TR;
}

// X [bh][rows][128] -> XT [bh][nb][128][64], XT[..][c][p] = X[block row kappa(p)][c]
// (zeros for rows past the block's valid count in the unpermuted layout).
// With to_f16 set the copy is written as fp16 (exact for bf16 values inside fp16's range).
__global__ __launch_bounds__(256) void k_transpose(const bf16_t* __restrict__ X, uint16_t* __restrict__ XT, int nb,
                                                   int nrows, int dense, int to_f16) {
  __shared__ uint16_t tile[TR][D + 2];
  const int I = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int n = dense ? min(TR, nrows - I * TR) : TR;
  const bf16_t* src = X + (size_t(bh) * nrows + size_t(I) * TR) * D;
  for (int e = tid; e < TR * D / 8; e += 256) {
    const int r = e / (D / 8), c8 = (e % (D / 8)) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < n) v = *reinterpret_cast<const u32x4*>(src + size_t(r) * D + c8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint16_t lo = uint16_t(v[k] & 0xffffu), hi = uint16_t(v[k] >> 16);
      if (to_f16) {
        lo = __builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(uint32_t(lo) << 16));
        hi = __builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(uint32_t(hi) << 16));
      }
      tile[r][c8 + 2 * k] = lo;
      tile[r][c8 + 2 * k + 1] = hi;
    }
  }
  __syncthreads();
  uint16_t* dst = XT + (size_t(bh) * nb + I) * D * TR;
  for (int e = tid; e < D * TR / 8; e += 256) {
    const int c = e / (TR / 8), p8 = (e % (TR / 8)) * 8;
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = uint32_t(tile[kappa(p8 + 2 * k)][c]) | (uint32_t(tile[kappa(p8 + 2 * k + 1)][c]) << 16);
    *reinterpret_cast<u32x4*>(dst + size_t(c) * TR + p8) = v;
  }
}

// ------------------------------------------------------------------ forward
__global__ __launch_bounds__(64) void k_fwd_mfma(AttnArgs a, const uint16_t* __restrict__ vt) {
  const int I = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
  const int nI = nrows_of(a, bh, I);
  const size_t q0 = row0_of(a, bh, I);
  const bf16_t* Q = static_cast<const bf16_t*>(a.q);
  const bf16_t* K = static_cast<const bf16_t*>(a.k);
  bf16_t* O = static_cast<bf16_t*>(a.out);
  const int cnt = a.dense ? a.nb : (nI > 0 ? a.sel_cnt[size_t(bh) * a.nb + I] : 0);
  const int32_t* lst = a.dense ? nullptr : a.sel_idx + (size_t(bh) * a.nb + I) * a.k_max;

  bf16x8 qf[2][8];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 32 * r + l32;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[r][s] = row < nI ? ld8(Q + (q0 + row) * D + 16 * s + 8 * g) : zero8();
  }
  f32x16 o[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int t = 0; t < 4; ++t) o[r][t] = zero16();
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};
  const float sl2 = a.scale * 1.4426950408889634f;

  bf16x8 kf[2][8];
  int J = cnt > 0 ? (a.dense ? 0 : lst[0]) : 0;
  int nJ = cnt > 0 ? nrows_of(a, bh, J) : 0;
  if (cnt > 0) {
    const size_t k0 = row0_of(a, bh, J);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        kf[c][s] = 32 * c + l32 < nJ ? ld8(K + (k0 + 32 * c + l32) * D + 16 * s + 8 * g) : zero8();
  }
  for (int it = 0; it < cnt; ++it) {
    const uint16_t* vb = vt + (size_t(bh) * a.nb + J) * D * TR;
    f16x8 vf[4][2][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) vf[t][c][h] = ld8h(vb + (32 * t + l32) * TR + 32 * c + 16 * h + 8 * g);
    f32x16 st[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 2; ++r) st[c][r] = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 2; ++r) st[c][r] = mma(kf[c][s], qf[r][s], st[c][r]);
    const int nJc = nJ;
    if (it + 1 < cnt) {
      J = a.dense ? it + 1 : lst[it + 1];
      nJ = nrows_of(a, bh, J);
      const size_t k0 = row0_of(a, bh, J);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int s = 0; s < 8; ++s)
          kf[c][s] = 32 * c + l32 < nJ ? ld8(K + (k0 + 32 * c + l32) * D + 16 * s + 8 * g) : zero8();
    }
    f16x8 pf[2][2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float v = (32 * c + acc_row(e, g) < nJc) ? st[c][r][e] * sl2 : -INFINITY;
          st[c][r][e] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(mrow[r], mx);
      const float alpha = exp2f(mrow[r] - mn);
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2f(st[c][r][e] - mn);
          st[c][r][e] = p;
          rs += p;
        }
      rs += __shfl_xor(rs, 32, 64);
      lrow[r] = lrow[r] * alpha + rs;
      mrow[r] = mn;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[r][t] *= alpha;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) pf[r][c][h] = pack8h(st[c][r], h);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 2; ++r) o[r][t] = mma(vf[t][c][h], pf[r][c][h], o[r][t]);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 32 * r + l32;
    if (row < nI) {
      const float inv = 1.f / lrow[r];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) st4(O + (q0 + row) * D + 32 * t + 8 * j + 4 * g, o[r][t], j, inv);
      if (g == 0) a.lse_out[q0 + row] = (mrow[r] + log2f(lrow[r])) * 0.6931471805599453f;
    } else if (!a.dense) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) st4(O + (q0 + row) * D + 32 * t + 8 * j + 4 * g, o[r][t], j, 0.f);
      if (g == 0) a.lse_out[q0 + row] = 0.f;
    }
  }
}

// ------------------------------------------------------------------ dK / dV
// One wavefront per key block J; loops over the query blocks that selected J (reverse
// index) in two halves of 32 query rows.  K and V of block J sit in LDS; dK^T and dV^T
// accumulate in registers.
__global__ __launch_bounds__(64) void k_dkdv_mfma(AttnArgs a, const uint16_t* __restrict__ qt,
                                                  const uint16_t* __restrict__ dot) {
  constexpr int P = D + 8;  // padded LDS row
  __shared__ __attribute__((aligned(16))) bf16_t sK[TR * P];
  __shared__ __attribute__((aligned(16))) bf16_t sV[TR * P];
  const int J = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
  const int nJ = nrows_of(a, bh, J);
  const size_t k0 = row0_of(a, bh, J);
  const bf16_t* Q = static_cast<const bf16_t*>(a.q);
  const bf16_t* K = static_cast<const bf16_t*>(a.k);
  const bf16_t* V = static_cast<const bf16_t*>(a.v);
  const bf16_t* G = static_cast<const bf16_t*>(a.dout);
  bf16_t* dK = static_cast<bf16_t*>(a.dk);
  bf16_t* dV = static_cast<bf16_t*>(a.dv);

  int cnt = 0;
  const int32_t* lst = nullptr;
  if (a.dense) {
    cnt = a.nb;
  } else if (nJ > 0) {
    const int32_t* rp = a.rev_ptr + size_t(bh) * (a.nb + 1);
    cnt = rp[J + 1] - rp[J];
    lst = a.rev_idx + size_t(bh) * a.nb * a.k_max + rp[J];
  }
  for (int e = lane; e < TR * D / 8; e += 64) {
    const int r = e / (D / 8), c8 = (e % (D / 8)) * 8;
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = kv;
    if (r < nJ) {
      kv = *reinterpret_cast<const u32x4*>(K + (k0 + r) * D + c8);
      vv = *reinterpret_cast<const u32x4*>(V + (k0 + r) * D + c8);
    }
    *reinterpret_cast<u32x4*>(&sK[r * P + c8]) = kv;
    *reinterpret_cast<u32x4*>(&sV[r * P + c8]) = vv;
  }
  __syncthreads();

  f32x16 dkT[4][2], dvT[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      dkT[t][c] = zero16();
      dvT[t][c] = zero16();
    }
  const float sl2 = a.scale * 1.4426950408889634f;
  for (int it = 0; it < cnt; ++it) {
    const int I = a.dense ? it : lst[it];
    const int nI = nrows_of(a, bh, I);
    const size_t q0 = row0_of(a, bh, I);
    const bf16_t* qtb = reinterpret_cast<const bf16_t*>(qt) + (size_t(bh) * a.nb + I) * D * TR;
    const bf16_t* dtb = reinterpret_cast<const bf16_t*>(dot) + (size_t(bh) * a.nb + I) * D * TR;
#pragma unroll 1
    for (int hq = 0; hq < 2; ++hq) {
      const int qrow = 32 * hq + l32;
      f32x16 s_[2], dp[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        s_[c] = zero16();
        dp[c] = zero16();
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 aq = qrow < nI ? ld8(Q + (q0 + qrow) * D + 16 * s + 8 * g) : zero8();
        const bf16x8 ag = qrow < nI ? ld8(G + (q0 + qrow) * D + 16 * s + 8 * g) : zero8();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&sK[(32 * c + l32) * P + 16 * s + 8 * g]);
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&sV[(32 * c + l32) * P + 16 * s + 8 * g]);
          s_[c] = mma(aq, bk, s_[c]);
          dp[c] = mma(ag, bv, dp[c]);
        }
      }
      // rows of s_/dp are query rows 32*hq + acc_row(e, g); LSE and D of those rows
      float lse2[16], Dr[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = 32 * hq + 8 * j + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = r0 + i < nI;
          lse2[4 * j + i] = ok ? a.lse_in[q0 + r0 + i] * 1.4426950408889634f : INFINITY;
          Dr[4 * j + i] = ok ? a.Dbuf[q0 + r0 + i] : 0.f;
        }
      }
      bf16x8 pb[2][2], sb[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2f(s_[c][e] * sl2 - lse2[e]);
          s_[c][e] = p;
          dp[c][e] = p * (dp[c][e] - Dr[e]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          pb[c][h] = pack8(s_[c], h);
          sb[c][h] = pack8(dp[c], h);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 ag = ld8(dtb + (32 * t + l32) * TR + 32 * hq + 16 * h + 8 * g);
          const bf16x8 aq = ld8(qtb + (32 * t + l32) * TR + 32 * hq + 16 * h + 8 * g);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            dvT[t][c] = mma(ag, pb[c][h], dvT[t][c]);
            dkT[t][c] = mma(aq, sb[c][h], dkT[t][c]);
          }
        }
    }
  }
  // dK^T / dV^T tile (t, c): column = key 32c + l32, rows = d 32t + acc_row(e, g)
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int key = 32 * c + l32;
    if (key >= nJ && (a.dense || key >= TR)) continue;
    const float sk = key < nJ ? a.scale : 0.f, sv = key < nJ ? 1.f : 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        st4(dK + (k0 + key) * D + 32 * t + 8 * j + 4 * g, dkT[t][c], j, sk);
        st4(dV + (k0 + key) * D + 32 * t + 8 * j + 4 * g, dvT[t][c], j, sv);
      }
  }
}

// ------------------------------------------------------------------ dQ
// One wavefront per query block I; loops over its selected key blocks in two halves of
// 32 keys.  Q and dO of block I stay in registers as B operands; dQ^T accumulates.
__global__ __launch_bounds__(64) void k_dq_mfma(AttnArgs a, const uint16_t* __restrict__ kt_) {
  const bf16_t* kt = reinterpret_cast<const bf16_t*>(kt_);
  const int I = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x, l32 = lane & 31, g = lane >> 5;
  const int nI = nrows_of(a, bh, I);
  const size_t q0 = row0_of(a, bh, I);
  const bf16_t* Q = static_cast<const bf16_t*>(a.q);
  const bf16_t* K = static_cast<const bf16_t*>(a.k);
  const bf16_t* V = static_cast<const bf16_t*>(a.v);
  const bf16_t* G = static_cast<const bf16_t*>(a.dout);
  bf16_t* dQ = static_cast<bf16_t*>(a.dq);
  const int cnt = a.dense ? a.nb : (nI > 0 ? a.sel_cnt[size_t(bh) * a.nb + I] : 0);
  const int32_t* lst = a.dense ? nullptr : a.sel_idx + (size_t(bh) * a.nb + I) * a.k_max;

  bf16x8 qb[2][8], gb[2][8];
  float lse2[2], Dq[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 32 * r + l32;
    const bool ok = row < nI;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qb[r][s] = ok ? ld8(Q + (q0 + row) * D + 16 * s + 8 * g) : zero8();
      gb[r][s] = ok ? ld8(G + (q0 + row) * D + 16 * s + 8 * g) : zero8();
    }
    lse2[r] = ok ? a.lse_in[q0 + row] * 1.4426950408889634f : INFINITY;
    Dq[r] = ok ? a.Dbuf[q0 + row] : 0.f;
  }
  f32x16 dqT[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 2; ++r) dqT[t][r] = zero16();
  const float sl2 = a.scale * 1.4426950408889634f;
  for (int it = 0; it < cnt; ++it) {
    const int J = a.dense ? it : lst[it];
    const int nJ = nrows_of(a, bh, J);
    const size_t k0 = row0_of(a, bh, J);
    const bf16_t* ktb = kt + (size_t(bh) * a.nb + J) * D * TR;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int key = 32 * c + l32;
      f32x16 st[2], dpt[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        st[r] = zero16();
        dpt[r] = zero16();
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 ak = key < nJ ? ld8(K + (k0 + key) * D + 16 * s + 8 * g) : zero8();
        const bf16x8 av = key < nJ ? ld8(V + (k0 + key) * D + 16 * s + 8 * g) : zero8();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          st[r] = mma(ak, qb[r][s], st[r]);
          dpt[r] = mma(av, gb[r][s], dpt[r]);
        }
      }
      // rows of st/dpt are keys 32c + acc_row(e, g), column = query 32r + l32
      bf16x8 sbf[2][2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool ok = 32 * c + acc_row(e, g) < nJ;
          const float p = ok ? exp2f(st[r][e] * sl2 - lse2[r]) : 0.f;
          dpt[r][e] = p * (dpt[r][e] - Dq[r]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) sbf[r][h] = pack8(dpt[r], h);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 ak = ld8(ktb + (32 * t + l32) * TR + 32 * c + 16 * h + 8 * g);
#pragma unroll
          for (int r = 0; r < 2; ++r) dqT[t][r] = mma(ak, sbf[r][h], dqT[t][r]);
        }
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 32 * r + l32;
    if (row >= nI && (a.dense || row >= TR)) continue;
    const float sc = row < nI ? a.scale : 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) st4(dQ + (q0 + row) * D + 32 * t + 8 * j + 4 * g, dqT[t][r], j, sc);
  }
}

__global__ __launch_bounds__(256) void k_bwd_pre_bf16(AttnArgs a, size_t total_rows) {
  const size_t row = size_t(blockIdx.x) * 16 + threadIdx.x / 16;
  const int cg = threadIdx.x % 16;
  float s = 0.f;
  if (row < total_rows) {
    float x[8], y[8];
    load8(static_cast<const bf16_t*>(a.dout) + row * D + cg * 8, x);
    load8(static_cast<const bf16_t*>(a.o) + row * D + cg * 8, y);
#pragma unroll
    for (int k = 0; k < 8; ++k) s = fmaf(x[k], y[k], s);
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (row < total_rows && cg == 0) a.Dbuf[row] = s;
}

}  // namespace

int attn_mfma_supported(const AttnArgs& a, prism_dtype dt) {
  return dt == PRISM_BF16 && a.d == D && (a.dense || a.vol == TR);
}

size_t attn_mfma_ws_bytes(int BH, int nb, int copies) {
  return size_t(copies) * align256(size_t(BH) * nb * D * TR * 2);
}

hipError_t launch_attn_fwd_mfma(const AttnArgs& a, void* ws, hipStream_t s) {
  uint16_t* vt = static_cast<uint16_t*>(ws);
  hipLaunchKernelGGL(k_transpose, dim3(a.nb, a.BH), dim3(256), 0, s, static_cast<const bf16_t*>(a.v), vt, a.nb,
                     a.nrows, a.dense, 1);
  hipLaunchKernelGGL(k_fwd_mfma, dim3(a.nb, a.BH), dim3(64), 0, s, a, vt);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_mfma(const AttnArgs& a, void* ws, hipEvent_t* marks, hipStream_t s) {
  const size_t one = align256(size_t(a.BH) * a.nb * D * TR * 2);
  char* p = static_cast<char*>(ws);
  uint16_t* qt = reinterpret_cast<uint16_t*>(p);
  uint16_t* kt = reinterpret_cast<uint16_t*>(p + one);
  uint16_t* gt = reinterpret_cast<uint16_t*>(p + 2 * one);
  if (marks) (void)hipEventRecord(marks[0], s);
  const size_t rows = size_t(a.BH) * a.nrows;
  hipLaunchKernelGGL(k_bwd_pre_bf16, dim3(unsigned((rows + 15) / 16)), dim3(256), 0, s, a, rows);
  hipLaunchKernelGGL(k_transpose, dim3(a.nb, a.BH), dim3(256), 0, s, static_cast<const bf16_t*>(a.q), qt, a.nb,
                     a.nrows, a.dense, 0);
  hipLaunchKernelGGL(k_transpose, dim3(a.nb, a.BH), dim3(256), 0, s, static_cast<const bf16_t*>(a.k), kt, a.nb,
                     a.nrows, a.dense, 0);
  hipLaunchKernelGGL(k_transpose, dim3(a.nb, a.BH), dim3(256), 0, s, static_cast<const bf16_t*>(a.dout), gt, a.nb,
                     a.nrows, a.dense, 0);
  if (marks) (void)hipEventRecord(marks[1], s);
  hipLaunchKernelGGL(k_dkdv_mfma, dim3(a.nb, a.BH), dim3(64), 0, s, a, qt, gt);
  if (marks) (void)hipEventRecord(marks[2], s);
  hipLaunchKernelGGL(k_dq_mfma, dim3(a.nb, a.BH), dim3(64), 0, s, a, kt);
  if (marks) (void)hipEventRecord(marks[3], s);
  return hipGetLastError();
}

}  // namespace prism
