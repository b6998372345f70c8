// Blocks of 128 or 256 tokens (the C_128 / C_256 candidate sets of Tables 9 and 11) run
// through the 64-row attention kernels as runs of 2 or 4 consecutive 64-row tiles.  The
// selection stays at block level (pooling, scores and the Top-k/Top-p cut are per block);
// these kernels expand it, and its reverse index, to tile level:
//   query tile (I, u) lists every live tile of every block J that block I selected;
//   key tile (J, v) lists every live tile of every block I that selected block J.
// A block's valid rows come first (then its padding), so its live tiles are the first
// ceil(n/64); fully padded tiles appear in no list.  Lists stay ascending because the
// block lists are ascending.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int NT = 256;
constexpr int TT = 64;  // rows per tile

// live tiles of a block with n valid rows, at most maxu (the most tiles a block owns;
// counts out of range are clamped, see prism_internal.h)
__device__ __forceinline__ int live_tiles(int n, int maxu) { return clampi((max(n, 0) + TT - 1) / TT, 0, maxu); }

__global__ void k_tile_valid(const int32_t* __restrict__ bvalid, size_t total_tiles, int g,
                             int32_t* __restrict__ tvalid) {
  const size_t t = blockIdx.x * size_t(blockDim.x) + threadIdx.x;
  if (t >= total_tiles) return;
  const int n = bvalid[t / g] - TT * int(t % g);
  tvalid[t] = n < 0 ? 0 : (n > TT ? TT : n);
}

// Tile numbering.  Fixed volume: block J owns tiles J*g .. J*g+g-1 (stride g, nt = nb*g).
// Mixed volumes: blocks are identified by their first 64-row unit, so block J owns tiles
// J, J+1, ... (stride 1, nt = nb) and units that start no block carry a zero count; there
// the lists and reverse counts are pre-filled (empty) and only live tiles are written.

// One workgroup per (block, head): the expanded list of `cnt` blocks taken from `lst`,
// written to every live tile of the block; with `rows_owned` > own_live also the empty
// lists of the block's dead tiles.  Offsets come from an exclusive scan of the listed
// blocks' live-tile counts, taken in chunks of NT with a running carry.
__device__ void expand_rows(const int32_t* __restrict__ lst, int cnt, const int32_t* __restrict__ bv_head, int nb,
                            int maxu, int own_live, int rows_owned, int stride, int cap, int32_t* __restrict__ out_rows,
                            int32_t* __restrict__ out_cnt, int* red) {
  int carry = 0;
  for (int k0 = 0; k0 < cnt; k0 += NT) {
    const int k = k0 + int(threadIdx.x);
    const int J = k < cnt ? clampi(lst[k], 0, nb - 1) : 0;
    const int c = k < cnt ? live_tiles(bv_head[J], maxu) : 0;
    int tot;
    const int off = carry + block_excl_scan<NT>(c, red, &tot);
    for (int u = 0; u < own_live; ++u)
      for (int v = 0; v < c; ++v) out_rows[size_t(u) * cap + off + v] = J * stride + v;
    carry += tot;
    __syncthreads();
  }
  for (int u = 0; u < rows_owned; ++u) {
    const int used = u < own_live ? carry : 0;
    for (int s = used + int(threadIdx.x); s < cap; s += NT) out_rows[size_t(u) * cap + s] = -1;
    if (threadIdx.x == 0) out_cnt[u] = used;
  }
}

__global__ __launch_bounds__(NT) void k_tile_lists(const int32_t* __restrict__ bvalid,
                                                   const int32_t* __restrict__ sel_idx,
                                                   const int32_t* __restrict__ sel_cnt, int nb, int stride,
                                                   int k_max, int cap, int mixed, int32_t* __restrict__ tile_idx,
                                                   int32_t* __restrict__ tile_cnt) {
  __shared__ int red[8];
  const int I = blockIdx.x, bh = blockIdx.y;
  const int32_t* bv = bvalid + size_t(bh) * nb;
  const int maxu = cap / k_max;  // tiles per block: g (fixed volume) or the largest block's units (mixed)
  // a mixed block's tiles are the units from its first one on, inside the head
  const int own_live = min(live_tiles(bv[I], maxu), mixed ? nb - I : stride);
  if (mixed && own_live == 0) return;  // no block starts here (or a dead one): pre-filled
  const int cnt = own_live > 0 ? clampi(sel_cnt[size_t(bh) * nb + I], 0, k_max) : 0;
  const size_t t0 = size_t(bh) * nb * stride + size_t(I) * stride;
  expand_rows(sel_idx + (size_t(bh) * nb + I) * k_max, cnt, bv, nb, maxu, own_live, mixed ? own_live : stride,
              stride, cap, tile_idx + t0 * cap, tile_cnt + t0, red);
}

// Reverse counts: key tile (J, v) is listed by every live tile of every block that selected J.
__global__ __launch_bounds__(64) void k_tile_rev_count(const int32_t* __restrict__ bvalid,
                                                       const int32_t* __restrict__ rev_ptr,
                                                       const int32_t* __restrict__ rev_idx, int nb, int stride,
                                                       int k_max, int maxu, int mixed, int32_t* __restrict__ rcnt) {
  const int J = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const int32_t* bv = bvalid + size_t(bh) * nb;
  const RevRange rr = rev_range(rev_ptr + size_t(bh) * (nb + 1), J, nb, k_max);
  const int32_t* ri = rev_idx + size_t(bh) * nb * k_max + rr.start;
  int c = 0;
  for (int k = lane; k < rr.cnt; k += 64) c += live_tiles(bv[clampi(ri[k], 0, nb - 1)], maxu);
  c = wave_sum_i(c);
  const int live = min(live_tiles(bv[J], maxu), mixed ? nb - J : stride);
  if (lane < (mixed ? live : stride)) rcnt[(size_t(bh) * nb + J) * stride + lane] = lane < live ? c : 0;
}

__global__ void k_fill_i32(int32_t* __restrict__ p, size_t n, int32_t val) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x) p[i] = val;
}

__global__ __launch_bounds__(1024) void k_tile_rev_scan(const int32_t* __restrict__ rcnt, int nt,
                                                        int32_t* __restrict__ tile_rev_ptr) {
  __shared__ int red[20];
  const int bh = blockIdx.x;
  const int R = (nt + 1023) / 1024;
  const int t0 = min(nt, int(threadIdx.x) * R), t1 = min(nt, t0 + R);
  const int32_t* c = rcnt + size_t(bh) * nt;
  int s = 0;
  for (int t = t0; t < t1; ++t) s += c[t];
  int tot;
  int off = block_excl_scan<1024>(s, red, &tot);
  int32_t* rp = tile_rev_ptr + size_t(bh) * (nt + 1);
  for (int t = t0; t < t1; ++t) {
    rp[t] = off;
    off += c[t];
  }
  if (threadIdx.x == 0) rp[nt] = tot;
}

__global__ __launch_bounds__(NT) void k_tile_rev_fill(const int32_t* __restrict__ bvalid,
                                                      const int32_t* __restrict__ rev_ptr,
                                                      const int32_t* __restrict__ rev_idx, int nb, int stride,
                                                      int k_max, int maxu, int mixed, int cap,
                                                      const int32_t* __restrict__ tile_rev_ptr,
                                                      int32_t* __restrict__ tile_rev_idx) {
  __shared__ int red[8];
  const int J = blockIdx.x, bh = blockIdx.y;
  const int32_t* bv = bvalid + size_t(bh) * nb;
  const RevRange rr = rev_range(rev_ptr + size_t(bh) * (nb + 1), J, nb, k_max);
  const int32_t* ri = rev_idx + size_t(bh) * nb * k_max + rr.start;
  const int nt = nb * stride;
  const int32_t* trp = tile_rev_ptr + size_t(bh) * (nt + 1);
  int32_t* out = tile_rev_idx + size_t(bh) * nt * size_t(cap);
  // the same clamps as k_tile_rev_count, so that the fill stays inside the counted ranges
  const int live = min(live_tiles(bv[J], maxu), mixed ? nb - J : stride);
  const int cnt = rr.cnt;
  int carry = 0;
  for (int k0 = 0; k0 < cnt; k0 += NT) {
    const int k = k0 + int(threadIdx.x);
    const int I = k < cnt ? clampi(ri[k], 0, nb - 1) : 0;
    const int c = k < cnt ? live_tiles(bv[I], maxu) : 0;
    int tot;
    const int off = carry + block_excl_scan<NT>(c, red, &tot);
    for (int v = 0; v < live; ++v) {
      const int base = trp[J * stride + v];
      for (int u = 0; u < c; ++u) out[base + off + u] = I * stride + u;
    }
    carry += tot;
    __syncthreads();
  }
}

}  // namespace

size_t tiles_ws_bytes(int BH, int nb, int vol) { return align256(size_t(BH) * nb * (vol / TT) * 4); }

hipError_t launch_blocks_to_tiles(const int32_t* bvalid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                  const int32_t* rev_ptr, const int32_t* rev_idx, int BH, int nb, int vol, int k_max,
                                  int32_t* tile_valid, int32_t* tile_idx, int32_t* tile_cnt, int32_t* tile_rev_ptr,
                                  int32_t* tile_rev_idx, void* ws, hipStream_t s) {
  const int g = vol / TT;
  const int nt = nb * g, cap = k_max * g;
  const size_t total = size_t(BH) * nt;
  int32_t* rcnt = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_tile_valid, dim3(unsigned((total + 255) / 256)), dim3(256), 0, s, bvalid, total, g, tile_valid);
  hipLaunchKernelGGL(k_tile_lists, dim3(nb, BH), dim3(NT), 0, s, bvalid, sel_idx, sel_cnt, nb, g, k_max, cap, 0,
                     tile_idx, tile_cnt);
  hipLaunchKernelGGL(k_tile_rev_count, dim3(nb, BH), dim3(64), 0, s, bvalid, rev_ptr, rev_idx, nb, g, k_max, g, 0,
                     rcnt);
  hipLaunchKernelGGL(k_tile_rev_scan, dim3(BH), dim3(1024), 0, s, rcnt, nt, tile_rev_ptr);
  hipLaunchKernelGGL(k_tile_rev_fill, dim3(nb, BH), dim3(NT), 0, s, bvalid, rev_ptr, rev_idx, nb, g, k_max, g, 0, cap,
                     tile_rev_ptr, tile_rev_idx);
  return hipGetLastError();
}

size_t tiles_mixed_ws_bytes(int BH, int nb) { return align256(size_t(BH) * nb * 4); }

hipError_t launch_blocks_to_tiles_mixed(const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                        const int32_t* rev_ptr, const int32_t* rev_idx, int BH, int nb, int k_max,
                                        int max_units, int32_t* tile_idx, int32_t* tile_cnt, int32_t* tile_rev_ptr,
                                        int32_t* tile_rev_idx, void* ws, hipStream_t s) {
  const int cap = k_max * max_units;
  const size_t total = size_t(BH) * nb;
  int32_t* rcnt = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_fill_i32, dim3(2048), dim3(256), 0, s, tile_idx, total * size_t(cap), -1);
  hipLaunchKernelGGL(k_fill_i32, dim3(256), dim3(256), 0, s, tile_cnt, total, 0);
  hipLaunchKernelGGL(k_fill_i32, dim3(256), dim3(256), 0, s, rcnt, total, 0);
  hipLaunchKernelGGL(k_tile_lists, dim3(nb, BH), dim3(NT), 0, s, block_valid, sel_idx, sel_cnt, nb, 1, k_max, cap, 1,
                     tile_idx, tile_cnt);
  hipLaunchKernelGGL(k_tile_rev_count, dim3(nb, BH), dim3(64), 0, s, block_valid, rev_ptr, rev_idx, nb, 1, k_max,
                     max_units, 1, rcnt);
  hipLaunchKernelGGL(k_tile_rev_scan, dim3(BH), dim3(1024), 0, s, rcnt, nb, tile_rev_ptr);
  hipLaunchKernelGGL(k_tile_rev_fill, dim3(nb, BH), dim3(NT), 0, s, block_valid, rev_ptr, rev_idx, nb, 1, k_max,
                     max_units, 1, cap, tile_rev_ptr, tile_rev_idx);
  return hipGetLastError();
}

}  // namespace prism
