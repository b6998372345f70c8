// Token permutation into blocks (Prism abstract: every block's tokens are kept together;
// Figure 2 caption).  One workgroup per (block, batch*head).  The slot -> token map is
// pure arithmetic on the zone's shape id: zones in raster order, blocks in raster order
// inside the zone, and inside a block its valid sub-box (the part inside the real grid)
// in raster order followed by the padding slots.  Rows move as 16-byte chunks.
//
// The forward direction can also pool (abstract: block-level features): the workgroup
// already holds every valid row of its block, so it sums them per channel in float32 and
// writes the block mean, which saves the selection a second pass over Q' and K'.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int NT = 256;

// 8 (bf16) or 4 (float32) elements of a 16-byte chunk, widened to float32
template <typename T>
__device__ __forceinline__ void widen(const uint4& u, float (&v)[8]);
template <>
__device__ __forceinline__ void widen<bf16_t>(const uint4& u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void widen<float>(const uint4& u, float (&v)[8]) {
  v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
  v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  v[4] = v[5] = v[6] = v[7] = 0.f;
}

// T: element type, only used when pooled != nullptr (forward direction, every candidate
// of the table holding exactly one unit).  Thread t always handles chunk t % chunks
// (chunks divides NT), so its partial sums cover one set of channels; they are combined
// across the workgroup in a fixed order through LDS.
template <typename T>
__global__ __launch_bounds__(NT) void k_permute(const uint4* __restrict__ x, uint4* __restrict__ y, Geo g,
                                                ShapeTab tab, const int32_t* __restrict__ shape_id,
                                                int chunks, int nb, int inverse,
                                                int32_t* __restrict__ block_valid, float* __restrict__ pooled) {
  constexpr int EPC = 16 / sizeof(T);  // elements per chunk
  __shared__ float s_part[NT][EPC];
  const int I = blockIdx.x;
  const int bh = blockIdx.y;
  const int vol = tab.vol;          // slots handled by this workgroup (the unit)
  const int slot0 = I * vol;
  const int z = slot0 / g.Vz;
  const int c = shape_id[size_t(bh) * g.nZ + z];
  // A shape id that is not a feasible candidate (caller error) maps no token: the unit is
  // written as padding (forward), left alone (inverse) and reported with 0 valid rows.
  const bool c_ok = c >= 0 && c < tab.n && tab.feasible[c];
  const int cc = c_ok ? c : 0;
  const int bt = tab.bt[cc], bhh = tab.bh[cc], bw = tab.bw[cc];
  // the zone's blocks hold S = cvol tokens, a multiple of the unit: this unit is the part
  // j0 .. j0 + vol - 1 of block blk
  const int S = tab.cvol[cc];
  const int blk = (slot0 % g.Vz) / S, j0 = (slot0 % g.Vz) % S;
  const int nbh = g.zh / bhh, nbw = g.zw / bw;
  const int iw = z % g.nzw, ih = (z / g.nzw) % g.nzh, it = z / (g.nzw * g.nzh);
  const int t0 = it * g.zt + (blk / (nbh * nbw)) * bt;
  const int h0 = ih * g.zh + ((blk / nbw) % nbh) * bhh;
  const int w0 = iw * g.zw + (blk % nbw) * bw;
  const int et = max(0, min(bt, g.T - t0)), eh = max(0, min(bhh, g.H - h0)), ew = max(0, min(bw, g.W - w0));
  const int nval = c_ok ? et * eh * ew : 0;
  const size_t slot_base = (size_t(bh) * nb + I) * vol;
  const size_t tok_base = size_t(bh) * g.N;
  const int total = vol * chunks;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int e = threadIdx.x; e < total; e += NT) {
    const int r = e / chunks, ch = e - r * chunks;
    const int j = j0 + r;           // position inside the block
    const size_t srow = (slot_base + r) * chunks + ch;
    if (j < nval) {
      const int tok = ((t0 + j / (eh * ew)) * g.H + h0 + (j / ew) % eh) * g.W + w0 + j % ew;
      const size_t trow = (tok_base + tok) * chunks + ch;
      if (inverse) {
        // the token-order result goes back to the caller, not to a later step of the path:
        // streamed past the caches (non-temporal), so that it leaves no dirty lines there
        typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
        const u32x4_nt u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(x + srow));
        __builtin_nontemporal_store(u, reinterpret_cast<u32x4_nt*>(y + trow));
      } else {
        const uint4 u = x[trow];
        y[srow] = u;
        if (pooled) {
          float v[8];
          widen<T>(u, v);
#pragma unroll
          for (int k = 0; k < EPC; ++k) acc[k] += v[k];
        }
      }
    } else if (!inverse) {
      y[srow] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const int nv = max(0, min(vol, nval - j0));
  if (threadIdx.x == 0 && block_valid) block_valid[size_t(bh) * nb + I] = nv;
  if (pooled) {
#pragma unroll
    for (int k = 0; k < EPC; ++k) s_part[threadIdx.x][k] = acc[k];
    __syncthreads();
    // channel ch*EPC + k sums the partials of threads ch, ch + chunks, ch + 2 chunks, ...
    const int d = chunks * EPC;
    float* out = pooled + (size_t(bh) * nb + I) * d;
    for (int col = threadIdx.x; col < d; col += NT) {
      const int ch = col / EPC, k = col % EPC;
      float s = 0.f;
      for (int t = ch; t < NT; t += chunks) s += s_part[t][k];
      out[col] = nv > 0 ? s / float(nv) : 0.f;
    }
  }
}

}  // namespace

hipError_t launch_permute(const void* x, void* y, prism_dtype dt, int BH, int d, const Geo& g,
                          const ShapeTab& tab, const int32_t* shape_id, int inverse,
                          int32_t* block_valid, float* pooled, hipStream_t s) {
  const int esize = dt == PRISM_BF16 ? 2 : 4;
  const int chunks = d * esize / 16;
  const int nb = g.nZ * (g.Vz / tab.vol);
  const auto* xs = static_cast<const uint4*>(x);
  auto* ys = static_cast<uint4*>(y);
  if (dt == PRISM_BF16)
    hipLaunchKernelGGL(k_permute<bf16_t>, dim3(nb, BH), dim3(NT), 0, s, xs, ys, g, tab, shape_id, chunks, nb, inverse,
                       block_valid, pooled);
  else
    hipLaunchKernelGGL(k_permute<float>, dim3(nb, BH), dim3(NT), 0, s, xs, ys, g, tab, shape_id, chunks, nb, inverse,
                       block_valid, pooled);
  return hipGetLastError();
}

}  // namespace prism
