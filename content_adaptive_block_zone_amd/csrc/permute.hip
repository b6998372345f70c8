// Token permutation into blocks (Prism abstract: every block's tokens are kept together;
// Figure 2 caption).  One workgroup per (block, batch*head).  The slot -> token map is
// pure arithmetic on the zone's shape id: zones in raster order, blocks in raster order
// inside the zone, and inside a block its valid sub-box (the part inside the real grid)
// in raster order followed by the padding slots.  Rows move as 16-byte chunks.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void k_permute(const uint4* __restrict__ x, uint4* __restrict__ y, Geo g,
                                                ShapeTab tab, const int32_t* __restrict__ shape_id,
                                                int chunks, int nb, int inverse,
                                                int32_t* __restrict__ block_valid) {
  const int I = blockIdx.x;
  const int bh = blockIdx.y;
  const int vol = tab.vol;          // slots handled by this workgroup (the unit)
  const int slot0 = I * vol;
  const int z = slot0 / g.Vz;
  const int c = shape_id[size_t(bh) * g.nZ + z];
  const int bt = tab.bt[c], bhh = tab.bh[c], bw = tab.bw[c];
  // the zone's blocks hold S = cvol tokens, a multiple of the unit: this unit is the part
  // j0 .. j0 + vol - 1 of block blk
  const int S = tab.cvol[c];
  const int blk = (slot0 % g.Vz) / S, j0 = (slot0 % g.Vz) % S;
  const int nbh = g.zh / bhh, nbw = g.zw / bw;
  const int iw = z % g.nzw, ih = (z / g.nzw) % g.nzh, it = z / (g.nzw * g.nzh);
  const int t0 = it * g.zt + (blk / (nbh * nbw)) * bt;
  const int h0 = ih * g.zh + ((blk / nbw) % nbh) * bhh;
  const int w0 = iw * g.zw + (blk % nbw) * bw;
  const int et = max(0, min(bt, g.T - t0)), eh = max(0, min(bhh, g.H - h0)), ew = max(0, min(bw, g.W - w0));
  const int nval = et * eh * ew;
  const size_t slot_base = (size_t(bh) * nb + I) * vol;
  const size_t tok_base = size_t(bh) * g.N;
  const int total = vol * chunks;
  for (int e = threadIdx.x; e < total; e += NT) {
    const int r = e / chunks, ch = e - r * chunks;
    const int j = j0 + r;           // position inside the block
    const size_t srow = (slot_base + r) * chunks + ch;
    if (j < nval) {
      const int tok = ((t0 + j / (eh * ew)) * g.H + h0 + (j / ew) % eh) * g.W + w0 + j % ew;
      const size_t trow = (tok_base + tok) * chunks + ch;
      if (inverse)
        y[trow] = x[srow];
      else
        y[srow] = x[trow];
    } else if (!inverse) {
      y[srow] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (threadIdx.x == 0 && block_valid) block_valid[size_t(bh) * nb + I] = max(0, min(vol, nval - j0));
}

}  // namespace

hipError_t launch_permute(const void* x, void* y, prism_dtype dt, int BH, int d, const Geo& g,
                          const ShapeTab& tab, const int32_t* shape_id, int inverse,
                          int32_t* block_valid, hipStream_t s) {
  const int esize = dt == PRISM_BF16 ? 2 : 4;
  const int chunks = d * esize / 16;
  const int nb = g.nZ * (g.Vz / tab.vol);
  hipLaunchKernelGGL(k_permute, dim3(nb, BH), dim3(NT), 0, s, static_cast<const uint4*>(x),
                     static_cast<uint4*>(y), g, tab, shape_id, chunks, nb, inverse, block_valid);
  return hipGetLastError();
}

}  // namespace prism
