// Block-sparse attention, scalar form (Prism Figure 2 caption: exact softmax attention
// restricted to the selected key blocks).  These kernels serve float32 inputs and any
// block volume up to 64; the bf16 path with 64-token blocks and d = 128 runs on the MFMA
// kernels of attn_mfma.hip.
//
// Layout of a workgroup: 256 threads = 64 rows x 4 channel quarters.  A row's dot
// products are split over its 4 lanes and combined with two lane swaps; key/value (or
// query/gradient) tiles of the current block pair are staged in LDS.
#include "prism_internal.h"

namespace prism {

__device__ __forceinline__ int tile_rows(const AttnArgs& a) { return a.dense ? kTileRows : a.vol; }
__device__ __forceinline__ int block_rows(const AttnArgs& a, int bh, int I) {
  return a.dense ? min(kTileRows, a.nrows - I * kTileRows) : clampi(a.bvalid[size_t(bh) * a.nb + I], 0, a.vol);
}
__device__ __forceinline__ size_t block_row0(const AttnArgs& a, int bh, int I) {
  return size_t(bh) * a.nrows + size_t(I) * tile_rows(a);
}

namespace {

constexpr int NT = 256;

template <typename T>
__device__ __forceinline__ void stage_rows(T* dst, const T* src, int rows, int d) {
  const int chunks = rows * d * int(sizeof(T)) / 16;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* o = reinterpret_cast<uint4*>(dst);
  for (int e = threadIdx.x; e < chunks; e += NT) o[e] = s[e];
}

template <typename T, int D>
__global__ __launch_bounds__(NT) void k_fwd_generic(AttnArgs a) {
  constexpr int CP = D / 4;
  __shared__ T sK[kTileRows * D];
  __shared__ T sV[kTileRows * D];
  const int I = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int nI = block_rows(a, bh, I);
  const size_t r0 = block_row0(a, bh, I);
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  T* O = static_cast<T*>(a.out);
  float q[CP], acc[CP];
#pragma unroll
  for (int c = 0; c < CP; ++c) {
    q[c] = r < nI ? to_f32(Q[(r0 + r) * D + part * CP + c]) : 0.f;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int cnt = a.dense ? a.nb : (nI > 0 ? clampi(a.sel_cnt[size_t(bh) * a.nb + I], 0, a.k_max) : 0);
  const int32_t* lst = a.dense ? nullptr : a.sel_idx + (size_t(bh) * a.nb + I) * a.k_max;
  for (int s = 0; s < cnt; ++s) {
    const int J = a.dense ? s : clampi(lst[s], 0, a.nb - 1);
    const int nJ = block_rows(a, bh, J);
    const size_t k0 = block_row0(a, bh, J);
    __syncthreads();
    stage_rows(sK, K + k0 * D, nJ, D);
    stage_rows(sV, V + k0 * D, nJ, D);
    __syncthreads();
    for (int j = 0; j < nJ; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < CP; ++c) dot = fmaf(q[c], to_f32(sK[j * D + part * CP + c]), dot);
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      const float sc = dot * a.scale;
      const float mn = fmaxf(m, sc);
      const float corr = expf(m - mn), pe = expf(sc - mn);
      l = l * corr + pe;
#pragma unroll
      for (int c = 0; c < CP; ++c) acc[c] = fmaf(pe, to_f32(sV[j * D + part * CP + c]), acc[c] * corr);
      m = mn;
    }
  }
  const int tr = tile_rows(a);
  if (r < nI) {
    // nothing to attend (l = 0): O = 0 and LSE = 0, as at padding rows
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < CP; ++c) O[(r0 + r) * D + part * CP + c] = from_f32<T>(acc[c] * inv);
    if (part == 0) a.lse_out[r0 + r] = l > 0.f ? m + logf(l) : 0.f;
  } else if (!a.dense && r < tr) {
#pragma unroll
    for (int c = 0; c < CP; ++c) O[(r0 + r) * D + part * CP + c] = from_f32<T>(0.f);
    if (part == 0) a.lse_out[r0 + r] = 0.f;
  }
}

// D_i = dO_i . O_i for every row (padding rows hold zeros in both, so D = 0 there).
template <typename T, int D>
__global__ __launch_bounds__(NT) void k_bwd_pre(AttnArgs a, size_t total_rows) {
  constexpr int G = D / 8;
  const size_t row = size_t(blockIdx.x) * (NT / G) + threadIdx.x / G;
  const int cg = threadIdx.x % G;
  float s = 0.f;
  if (row < total_rows) {
    float x[8], y[8];
    load8(static_cast<const T*>(a.dout) + row * D + cg * 8, x);
    load8(static_cast<const T*>(a.o) + row * D + cg * 8, y);
#pragma unroll
    for (int k = 0; k < 8; ++k) s = fmaf(x[k], y[k], s);
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (row < total_rows && cg == 0) a.Dbuf[row] = s;
}

template <typename T, int D>
__global__ __launch_bounds__(NT) void k_dkdv_generic(AttnArgs a) {
  constexpr int CP = D / 4;
  __shared__ T sQ[kTileRows * D];
  __shared__ T sG[kTileRows * D];
  __shared__ float sL[kTileRows], sD[kTileRows];
  const int J = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int nJ = block_rows(a, bh, J);
  const size_t r0 = block_row0(a, bh, J);
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  const T* G = static_cast<const T*>(a.dout);
  float kk[CP], vv[CP], dk[CP], dv[CP];
#pragma unroll
  for (int c = 0; c < CP; ++c) {
    kk[c] = r < nJ ? to_f32(K[(r0 + r) * D + part * CP + c]) : 0.f;
    vv[c] = r < nJ ? to_f32(V[(r0 + r) * D + part * CP + c]) : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  int cnt = 0;
  const int32_t* lst = nullptr;
  if (a.dense) {
    cnt = a.nb;
  } else if (nJ > 0) {
    const RevRange rr = rev_range(a.rev_ptr + size_t(bh) * (a.nb + 1), J, a.nb, a.k_max);
    cnt = rr.cnt;
    lst = a.rev_idx + size_t(bh) * a.nb * a.k_max + rr.start;
  }
  for (int s = 0; s < cnt; ++s) {
    const int I = a.dense ? s : clampi(lst[s], 0, a.nb - 1);
    const int nI = block_rows(a, bh, I);
    const size_t q0 = block_row0(a, bh, I);
    __syncthreads();
    stage_rows(sQ, Q + q0 * D, nI, D);
    stage_rows(sG, G + q0 * D, nI, D);
    if (tid < nI) {
      sL[tid] = a.lse_in[q0 + tid];
      sD[tid] = a.Dbuf[q0 + tid];
    }
    __syncthreads();
    for (int i = 0; i < nI; ++i) {
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < CP; ++c) {
        dot = fmaf(to_f32(sQ[i * D + part * CP + c]), kk[c], dot);
        dp = fmaf(to_f32(sG[i * D + part * CP + c]), vv[c], dp);
      }
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      dp += __shfl_xor(dp, 1, 64);
      dp += __shfl_xor(dp, 2, 64);
      const float pr = expf(dot * a.scale - sL[i]);
      const float ds = pr * (dp - sD[i]);
#pragma unroll
      for (int c = 0; c < CP; ++c) {
        dv[c] = fmaf(pr, to_f32(sG[i * D + part * CP + c]), dv[c]);
        dk[c] = fmaf(ds, to_f32(sQ[i * D + part * CP + c]), dk[c]);
      }
    }
  }
  T* dK = static_cast<T*>(a.dk);
  T* dV = static_cast<T*>(a.dv);
  const int tr = tile_rows(a);
  if (r < nJ) {
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      dK[(r0 + r) * D + part * CP + c] = from_f32<T>(dk[c] * a.scale);
      dV[(r0 + r) * D + part * CP + c] = from_f32<T>(dv[c]);
    }
  } else if (!a.dense && r < tr) {
#pragma unroll
    for (int c = 0; c < CP; ++c) {
      dK[(r0 + r) * D + part * CP + c] = from_f32<T>(0.f);
      dV[(r0 + r) * D + part * CP + c] = from_f32<T>(0.f);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(NT) void k_dq_generic(AttnArgs a) {
  constexpr int CP = D / 4;
  __shared__ T sK[kTileRows * D];
  __shared__ T sV[kTileRows * D];
  const int I = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int nI = block_rows(a, bh, I);
  const size_t r0 = block_row0(a, bh, I);
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  const T* G = static_cast<const T*>(a.dout);
  float q[CP], g[CP], dq[CP];
#pragma unroll
  for (int c = 0; c < CP; ++c) {
    q[c] = r < nI ? to_f32(Q[(r0 + r) * D + part * CP + c]) : 0.f;
    g[c] = r < nI ? to_f32(G[(r0 + r) * D + part * CP + c]) : 0.f;
    dq[c] = 0.f;
  }
  const float li = r < nI ? a.lse_in[r0 + r] : 0.f;
  const float Di = r < nI ? a.Dbuf[r0 + r] : 0.f;
  const int cnt = a.dense ? a.nb : (nI > 0 ? clampi(a.sel_cnt[size_t(bh) * a.nb + I], 0, a.k_max) : 0);
  const int32_t* lst = a.dense ? nullptr : a.sel_idx + (size_t(bh) * a.nb + I) * a.k_max;
  for (int s = 0; s < cnt; ++s) {
    const int J = a.dense ? s : clampi(lst[s], 0, a.nb - 1);
    const int nJ = block_rows(a, bh, J);
    const size_t k0 = block_row0(a, bh, J);
    __syncthreads();
    stage_rows(sK, K + k0 * D, nJ, D);
    stage_rows(sV, V + k0 * D, nJ, D);
    __syncthreads();
    for (int j = 0; j < nJ; ++j) {
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < CP; ++c) {
        dot = fmaf(q[c], to_f32(sK[j * D + part * CP + c]), dot);
        dp = fmaf(g[c], to_f32(sV[j * D + part * CP + c]), dp);
      }
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      dp += __shfl_xor(dp, 1, 64);
      dp += __shfl_xor(dp, 2, 64);
      const float pr = expf(dot * a.scale - li);
      const float ds = pr * (dp - Di);
#pragma unroll
      for (int c = 0; c < CP; ++c) dq[c] = fmaf(ds, to_f32(sK[j * D + part * CP + c]), dq[c]);
    }
  }
  T* dQ = static_cast<T*>(a.dq);
  const int tr = tile_rows(a);
  if (r < nI) {
#pragma unroll
    for (int c = 0; c < CP; ++c) dQ[(r0 + r) * D + part * CP + c] = from_f32<T>(dq[c] * a.scale);
  } else if (!a.dense && r < tr) {
#pragma unroll
    for (int c = 0; c < CP; ++c) dQ[(r0 + r) * D + part * CP + c] = from_f32<T>(0.f);
  }
}

template <typename T, int D>
hipError_t fwd_t(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_fwd_generic<T, D>), dim3(a.nb, a.BH), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_t(const AttnArgs& a, hipEvent_t* marks, hipStream_t s) {
  if (marks) (void)hipEventRecord(marks[0], s);
  const size_t rows = size_t(a.BH) * a.nrows;
  constexpr int rpb = NT / (D / 8);
  hipLaunchKernelGGL((k_bwd_pre<T, D>), dim3(unsigned((rows + rpb - 1) / rpb)), dim3(NT), 0, s, a, rows);
  if (marks) (void)hipEventRecord(marks[1], s);
  hipLaunchKernelGGL((k_dkdv_generic<T, D>), dim3(a.nb, a.BH), dim3(NT), 0, s, a);
  if (marks) (void)hipEventRecord(marks[2], s);
  hipLaunchKernelGGL((k_dq_generic<T, D>), dim3(a.nb, a.BH), dim3(NT), 0, s, a);
  if (marks) (void)hipEventRecord(marks[3], s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_generic(const AttnArgs& a, prism_dtype dt, hipStream_t s) {
  if (dt == PRISM_BF16) return a.d == 64 ? fwd_t<bf16_t, 64>(a, s) : fwd_t<bf16_t, 128>(a, s);
  return a.d == 64 ? fwd_t<float, 64>(a, s) : fwd_t<float, 128>(a, s);
}

hipError_t launch_attn_bwd_generic(const AttnArgs& a, prism_dtype dt, hipEvent_t* marks, hipStream_t s) {
  if (dt == PRISM_BF16) return a.d == 64 ? bwd_t<bf16_t, 64>(a, marks, s) : bwd_t<bf16_t, 128>(a, marks, s);
  return a.d == 64 ? bwd_t<float, 64>(a, marks, s) : bwd_t<float, 128>(a, marks, s);
}

int attn_mfma_supported(const AttnArgs& a, prism_dtype dt);
size_t attn_mfma_sched_bytes(const AttnArgs& a);
hipError_t launch_attn_fwd_mfma(const AttnArgs& a, void* ws, hipStream_t s);
hipError_t launch_attn_bwd_mfma(const AttnArgs& a, int32_t* sched, hipEvent_t* marks, hipStream_t s);

// Forward workspace: on the matrix-core path the workgroup schedule (sparse mode) and the
// fp16 copy of V with its per-head scales; none on the scalar path.
size_t attn_fwd_ws_bytes(const AttnArgs& a, prism_dtype dt) {
  return attn_mfma_supported(a, dt) ? attn_mfma_fwd_ws_bytes(a) : 0;
}

// Backward workspace: D = rowsum(dO * O) per row, then (matrix-core path, sparse mode)
// the query-major and key-major workgroup schedules.
size_t attn_bwd_ws_bytes(const AttnArgs& a, prism_dtype dt) {
  const size_t dbuf = align256(size_t(a.BH) * a.nrows * 4);
  return dbuf + (attn_mfma_supported(a, dt) ? 2 * attn_mfma_sched_bytes(a) : 0);
}

hipError_t launch_attn_fwd(const AttnArgs& a, prism_dtype dt, void* ws, hipStream_t s) {
  if (attn_mfma_supported(a, dt)) return launch_attn_fwd_mfma(a, ws, s);
  return launch_attn_fwd_generic(a, dt, s);
}

hipError_t launch_attn_bwd(const AttnArgs& a_in, prism_dtype dt, void* ws, hipEvent_t* marks, hipStream_t s) {
  AttnArgs a = a_in;
  a.Dbuf = static_cast<float*>(ws);
  if (attn_mfma_supported(a, dt)) {
    int32_t* sched = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align256(size_t(a.BH) * a.nrows * 4));
    return launch_attn_bwd_mfma(a, sched, marks, s);
  }
  return launch_attn_bwd_generic(a, dt, marks, s);
}

}  // namespace prism
