// Block-sparse attention on the matrix cores of gfx950 (Prism Figure 2 caption: exact
// softmax attention over the selected blocks), for bf16, 64-token blocks and d = 128.
//
// Shape of the work.  Every (query block, key block) pair costs 2 MFLOP per product but
// needs a whole 64x128 tile pair from memory, and the key lists of neighbouring query
// blocks barely overlap, so these kernels are bound by how fast tiles arrive, not by the
// matrix cores.  Each streamed tile is read from memory exactly once per pair:
//   * a workgroup of 4 wavefronts owns one 64-row block (the query block in the forward
//     and dQ kernels, the key block in the dK/dV kernel), whose own operands stay in
//     registers for the whole list;
//   * the streamed block (K/V, or Q/dO) is copied straight from memory into LDS
//     (global_load_lds, no registers involved) and shared by the four waves; there are two
//     LDS stages, and the next pair's copy is in flight while the current one is computed.
// All three kernels split the 64x64 pair 2x2 over the waves and use
// v_mfma_f32_32x32x16_bf16 (A = 32 rows x 16 k, lane l: row l%32, k = 8(l/32)..+7; B
// likewise with columns; C = 16 registers, lane l register e at row 8(e/4) + 4(l/32) + e%4,
// column l%32).  The forward and dQ waves each cover one key half and merge the halves
// once at the end; the dK/dV waves swap P and dS halves through LDS each pair.
// Products whose contraction runs over the streamed block's rows (P V, Q^T dS, dO^T P,
// K^T dS) take accumulator registers directly as the B operand, whose k index then runs
// over the rows in the accumulator's order, "kappa32": within each 16-row group, position
// p holds row p with bits 2 and 3 swapped.  The matching A operand is the streamed tile
// transposed with its rows in that order, read from the row-major tile with gfx950's
// transposing LDS read (ds_read_b64_tr_b16), two 8-byte reads per operand.
// All accumulation is fp32.  The forward's P V product runs in fp16: P (below 2^8 under
// the lazy rescaling) is rounded to fp16, and V comes from an fp16 copy made once per
// launch and scaled per head by a power of two, in which every bf16 value is exact.
// In sparse mode the workgroups take their owner blocks longest list first within each
// head (k_schedule), which balances the launch and lets workgroups resident together
// share tiles in L2.

#include "prism_internal.h"

namespace prism {

int attn_mfma_supported(const AttnArgs& a, prism_dtype dt);
size_t attn_mfma_sched_bytes(const AttnArgs& a);
hipError_t launch_attn_fwd_mfma(const AttnArgs& a, void* ws, hipStream_t s);
hipError_t launch_attn_bwd_mfma(const AttnArgs& a, int32_t* sched, hipEvent_t* marks, hipStream_t s);
hipError_t launch_gather_fwd_mfma(const AttnArgs& a, int32_t* sched, hipStream_t s);

namespace {

constexpr int D = 128;        // head dimension
constexpr int TR = 64;        // rows per block
constexpr int NT = 256;       // 4 wavefronts
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 2^x by the hardware instruction; results below 2^-126 (probabilities too small to register
// in a bf16 or fp32 sum of terms up to 1) flush to zero
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }

template <typename V>
__device__ __forceinline__ V lds8(const uint16_t* p) {
  return __builtin_bit_cast(V, *reinterpret_cast<const u32x4*>(p));
}
// 8 bf16 from global memory, or zeros when the row does not exist
__device__ __forceinline__ bf16x8 gld8(const bf16_t* p, bool ok) {
  return __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const u32x4*>(p) : zero_u4());
}
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return uint32_t(__builtin_bit_cast(uint16_t, (__bf16)a)) | (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)b)) << 16);
}
__device__ __forceinline__ int nrows_of(const AttnArgs& a, int bh, int I) {
  return a.dense ? min(TR, a.nrows - I * TR) : clampi(a.bvalid[size_t(bh) * a.nb + I], 0, TR);
}
__device__ __forceinline__ size_t row0_of(const AttnArgs& a, int bh, int I) {
  return size_t(bh) * a.nrows + size_t(I) * TR;
}
// first row of key block J (keys may be a different sequence in a dense cross-attention)
__device__ __forceinline__ size_t krow0_of(const AttnArgs& a, int bh, int J) {
  return size_t(bh) * a.nkrows + size_t(J) * TR;
}

// Owner block of a workgroup.  Heads are taken in order, so that a head's K/V (or Q/dO)
// pass through the 256 MB last-level cache one at a time.
// Sparse mode: the launcher's schedule (k_schedule: longest list first within each head).
// Dense mode (every list the same length): workgroups are dealt to the eight XCDs
// round-robin by id, and the ids are remapped so that each XCD receives runs of G
// consecutive blocks (runs dealt round-robin, so the work stays balanced); G = 16 for the
// query-major kernels and 64 for the key-major one.  Ids past the last whole group of 8G
// keep their place.
template <int G>
__device__ __forceinline__ void owner_of(const AttnArgs& a, const int32_t* order, int& I, int& bh) {
  int id = blockIdx.x;
  if (order) {
    id = __builtin_amdgcn_readfirstlane(order[id]);
  } else {
    const int full = (a.nb * a.BH / (8 * G)) * (8 * G);
    if (id < full) {
      const int x = id % 8, l = id / 8;
      id = (l / G) * (8 * G) + x * G + (l % G);
    }
  }
  I = id % a.nb;
  bh = id / a.nb;
}

// ------------------------------------------------------------------ workgroup schedule
// The order in which the workgroups of one sparse launch take their owner blocks: within
// each head (heads stay in order), longest list first, in bins of `width` lengths.  Two
// effects, both measured on the 2K-like workload (about 7 % over the three kernels):
//   * the longest lists start first, so a launch does not end on a few long workgroups;
//   * workgroups resident together have lists of about the same length, so, walking their
//     ascending lists, they move through the streamed blocks at about the same pace and
//     ask for the same tiles close together in time, which then hit in L2.
// The order changes only which workgroup runs when: every block's result is computed by
// one workgroup alone, so the outputs do not depend on it.  Within a bin the order is
// that of LDS atomics and may differ from call to call.
// Grid: BH workgroups for the query-major order (from the list counts), then, when
// order_k is given, BH more for the key-major order (from the reverse-list lengths).
constexpr int kSchedBins = 2048;
constexpr int kSchedThreads = 1024;
__global__ __launch_bounds__(kSchedThreads) void k_schedule(AttnArgs a, int32_t* order_q, int32_t* order_k) {
  __shared__ int bins[kSchedBins];
  __shared__ int wsum[kSchedThreads / 64];
  const int key_major = blockIdx.x >= a.BH;
  const int bh = blockIdx.x - (key_major ? a.BH : 0);
  int32_t* out = (key_major ? order_k : order_q) + size_t(bh) * a.nb;
  const int bound = key_major ? a.nb : a.k_max;  // longest possible list
  const int width = bound / kSchedBins + 1;
  auto bin_of = [&](int I) {
    int len;
    if (key_major) {
      const int32_t* rp = a.rev_ptr + size_t(bh) * (a.nb + 1) + I;
      len = rp[1] - rp[0];
    } else {
      len = a.bvalid[size_t(bh) * a.nb + I] > 0 ? a.sel_cnt[size_t(bh) * a.nb + I] : 0;
    }
    return kSchedBins - 1 - min(max(len, 0), bound) / width;  // longest first
  };
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int i = t; i < kSchedBins; i += kSchedThreads) bins[i] = 0;
  __syncthreads();
  for (int I = t; I < a.nb; I += kSchedThreads) atomicAdd(&bins[bin_of(I)], 1);
  __syncthreads();
  // exclusive prefix sum of the bins, two per thread
  static_assert(kSchedBins == 2 * kSchedThreads, "two bins per thread");
  const int h0 = bins[2 * t], h1 = bins[2 * t + 1];
  int x = h0 + h1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int start = x - h0 - h1;
  for (int i = 0; i < w; ++i) start += wsum[i];
  bins[2 * t] = start;  // each thread rewrites only the two bins it read
  bins[2 * t + 1] = start + h0;
  __syncthreads();
  for (int I = t; I < a.nb; I += kSchedThreads) out[atomicAdd(&bins[bin_of(I)], 1)] = bh * a.nb + I;
}

// The streamed block list of a workgroup, with each block's valid-row count, is copied to
// LDS once (packed as J | n << 16), so that finding the next block to prefetch costs an
// LDS read instead of two dependent global loads.  Lists longer than the kernel's capacity
// (or block indices past 16 bits) fall back to reading global memory per step.
constexpr int kMetaCap = 2048;
struct BlockList {
  const int32_t* lst;  // nullptr in dense mode (block k is k)
  int cnt;
  bool in_lds;
};
template <int CAP = kMetaCap, int NTH = NT>
__device__ __forceinline__ BlockList load_list(const AttnArgs& a, int bh, const int32_t* lst, int cnt, int* meta) {
  BlockList L{lst, cnt, !a.dense && cnt <= CAP && a.nb < 65536};
  if (L.in_lds)
    for (int k = threadIdx.x; k < cnt; k += NTH) {
      const int J = clampi(lst[k], 0, a.nb - 1);
      meta[k] = J | (nrows_of(a, bh, J) << 16);
    }
  __syncthreads();
  return L;
}
// srows: rows per head of the streamed tensor (dense mode's ragged last block)
__device__ __forceinline__ void list_at(const AttnArgs& a, int bh, const BlockList& L, const int* meta, int k, int& J,
                                        int& n, int srows) {
  if (a.dense) {
    J = k;
    n = min(TR, srows - k * TR);
  } else if (L.in_lds) {
    const int m = __builtin_amdgcn_readfirstlane(meta[k]);  // the same for every lane
    J = m & 0xffff;
    n = m >> 16;
  } else {
    J = __builtin_amdgcn_readfirstlane(clampi(L.lst[k], 0, a.nb - 1));
    n = __builtin_amdgcn_readfirstlane(nrows_of(a, bh, J));
  }
}
// The kernels walk their list in order.  In LDS mode the entry after the one being used is
// read one step ahead (`pre`), so that its LDS latency overlaps a whole iteration instead of
// delaying the next copy.
__device__ __forceinline__ int list_first(const BlockList& L, const int* meta) {
  return L.in_lds && L.cnt > 0 ? meta[0] : 0;
}
__device__ __forceinline__ void list_next(const AttnArgs& a, int bh, const BlockList& L, const int* meta, int k,
                                          int& pre, int& J, int& n, int srows) {
  if (L.in_lds) {
    const int m = __builtin_amdgcn_readfirstlane(pre);
    J = m & 0xffff;
    n = m >> 16;
    pre = meta[min(k + 1, L.cnt - 1)];
  } else {
    list_at(a, bh, L, meta, k, J, n, srows);
  }
}

// ---- 32x32x16 products.  A = 32 rows x 16 k (lane l: row l%32,
// k = 8(l/32)..+7), B likewise with columns, C = 16 registers: lane l register e at row
// 8(e/4) + 4(l/32) + e%4, column l%32.  Registers 8s..8s+7 of an accumulator are the B
// operand of a product contracting over its rows when the A operand lists those rows in
// "kappa32" order: position p of each 16-row group holds row p with bits 2 and 3 swapped.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// value of lane l ^ 32 (v_permlane32_swap: a VALU exchange of the two 32-lane halves)
__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}
__device__ __forceinline__ int acc_row32(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }
// accumulator registers 8s..8s+7 rounded to fp16 (round to nearest even)
__device__ __forceinline__ f16x8 pack8h(const f32x16& c, int s) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)c[8 * s + e];
  return r;
}
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)c[8 * s + e];
  return r;
}
// ---- direct-to-LDS staging.  A streamed 64x128 bf16 tile is copied by
// global_load_lds (16 bytes per lane, written to LDS in lane order, no registers involved)
// into an unpadded tile of 256-byte rows whose 16-byte chunks are permuted by an XOR with
// sw(r) = 4(r%4) + (r/4)%4.  Reads of one chunk from 16 consecutive rows (the row operands)
// and transposing reads of an aligned 64-byte span from 4 consecutive rows both land on 16
// distinct chunk positions, i.e. on all 64 banks once.
constexpr int TB = TR * D * 2;  // bytes of a tile
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;
__device__ __forceinline__ int sw(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// element offset of (row r, column c) in a tile
__device__ __forceinline__ int tofs(int r, int c) { return r * D + ((((c >> 3) ^ sw(r)) & 15) << 3) + (c & 7); }
// One 16-byte-per-lane copy, global memory -> LDS.  It is written as inline assembly so that the compiler, which would otherwise make
// the next LDS read of any stage wait for it, leaves its completion to the kernel: the
// kernels wait for their own copies (wait_loads) before the barrier that opens a stage,
// and no LDS location is read while a copy into it can be in flight.  M0 holds the LDS
// destination; one wait state separates its write from the copy.  The source is a
// wave-uniform base (SGPRs) plus a 32-bit byte offset per lane.
__device__ __forceinline__ void copy16_to_lds(const void* base, uint32_t off, const void* lds_dst) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds_dst);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m));
}
// tile <- rows 0..63 of src (wave-uniform); rows past n repeat row n-1 (finite; their
// products are masked).  Wave w (0..3 of the waves sharing the tile) writes rows
// 16w..16w+15, 4 rows (1 KB) per instruction.
// (Copying only the valid rows, with the other lanes inactive, measured 2-3 % slower.)
__device__ __forceinline__ void load_tile(const bf16_t* src, int n, uint16_t* tile, int w = threadIdx.x >> 6) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * i + (l >> 4);
    const uint32_t off = uint32_t(max(min(r, n - 1), 0)) * (D * 2) + uint32_t(((l & 15) ^ sw(r)) << 4);
    copy16_to_lds(src, off, tile + (16 * w + 4 * i) * D);
  }
}
// A operand of a 32x32x16 product whose rows are tile columns 32t.. (d) and whose 16 k are
// tile rows 16j.. in kappa32 order, by two transposing reads (ds_read_b64_tr_b16).  Within
// each 16 lanes such a read returns to lane i element i%4 of the 4-element pieces that lanes
// 4k + i/4 address (k = 0..3); so lane 16b + 4q + c of half g addresses row
// 16j + 8h + 4g + q, columns 32t + 16b + 4c.., and receives column 32t + 16b + 4q + c of
// rows 16j + 8h + 4g + 0..3, which are kappa32 positions 8g + 4h + 0..3.
__device__ __forceinline__ bf16x8 ldtr(const uint16_t* tile, int t, int j, int l = threadIdx.x & 63) {
  const int c = 32 * t + 16 * ((l >> 4) & 1) + 4 * (l & 3);
  const int r = 16 * j + 4 * (l >> 5) + ((l & 15) >> 2);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + tofs(r, c)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + tofs(r + 8, c)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// vmcnt(0): the direct-to-LDS copies this wave issued have landed
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// rows 8j+4g .. +3 of column `col` of a 32x32 accumulator tile, times s, as 4 bf16
__device__ __forceinline__ void store4_32(bf16_t* p, const f32x16& c, int j, float s) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pk2(c[4 * j] * s, c[4 * j + 1] * s), pk2(c[4 * j + 2] * s, c[4 * j + 3] * s)};
}

// ------------------------------------------------------------------ forward (32x32x16)
// Owner: query block I.  Wave w = (qh = w&1, kh = w>>1) takes queries 32qh.. against keys
// 32kh.. of every streamed key block and keeps its own online softmax (running max m, sum
// l and O^T) over its key half; the two halves are merged once at the end through LDS.
// K and V tiles stream through two LDS stages as in the backward kernels.
// P V precision.  The probabilities must be carried to well below the output's own bf16
// rounding: rounded to bf16 (8 bits) they cost up to half a bf16 ulp of a large output.
//   H = true: P rounded to fp16 (11 bits) against the fp16 copy of V (per-head scale
//     2^s, exact for bf16 values; undone in the epilogue): one product per 16 keys.
//   H = false: P split into a bf16 head and a bf16 remainder (about 16 bits) against the
//     bf16 V: two products.  Used by the audio-to-video cross-attention, whose call takes
//     no workspace for the fp16 copy.
// P split into bf16 head and remainder, accumulator registers 8s..8s+7
__device__ __forceinline__ void split8(const f32x16& c, int s, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)c[8 * s + e];
    hi[e] = h;
    lo[e] = (__bf16)(c[8 * s + e] - (float)h);
  }
}
constexpr float kLazy = 8.f;  // log2 units
template <bool H>
__global__ __launch_bounds__(NT, 2) void k_fwd(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TB];
  __shared__ int sMeta[kMetaCap];
  int I, bh;
  owner_of<16>(a, a.order_q, I, bh);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int qh = w & 1, kh = w >> 1;
  const int nI = nrows_of(a, bh, I);
  const size_t q0 = row0_of(a, bh, I);
  const bf16_t* Q = static_cast<const bf16_t*>(a.q);
  const bf16_t* K = static_cast<const bf16_t*>(a.k);
  // the V tile's 16-bit elements: fp16 (H) or bf16; the copy moves them as bits
  const bf16_t* V = static_cast<const bf16_t*>(H ? a.v16 : a.v);
  bf16_t* O = static_cast<bf16_t*>(a.out);
  const int cnt = a.dense ? a.nkb : (nI > 0 ? clampi(a.sel_cnt[size_t(bh) * a.nb + I], 0, a.k_max) : 0);
  const BlockList bl = load_list(a, bh, a.dense ? nullptr : a.sel_idx + (size_t(bh) * a.nb + I) * a.k_max, cnt, sMeta);
  const float vscale = H ? a.vinv[bh] : 1.f;   // undoes the fp16 copy's per-head scale
  const int qrow = 32 * qh + l32;
  const bool qok = qrow < nI;
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = gld8(Q + (q0 + qrow) * D + 16 * s + 8 * g, qok);
  f32x16 o[4];  // O^T: rows d = 32t + acc_row32(e, g), column = query qrow
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = zero16();
  float m = -INFINITY, l = 0.f;  // over this wave's key half, log2 units
  const float sl2 = a.scale * LOG2E;

  // stage st: K tile at 2st, V tile at 2st+1
  int pre = list_first(bl, sMeta);
  auto issue = [&](int k, int st) {
    int J, n;
    list_next(a, bh, bl, sMeta, k, pre, J, n, a.nkrows);
    const size_t r0 = krow0_of(a, bh, J);
    load_tile(K + r0 * D, n, reinterpret_cast<uint16_t*>(smem + 2 * st * TB));
    load_tile(V + r0 * D, n, reinterpret_cast<uint16_t*>(smem + (2 * st + 1) * TB));
    return n;
  };
  int n_next = cnt > 0 ? issue(0, 0) : 0;
  for (int it = 0; it < cnt; ++it) {
    const int st = it & 1, nJ = n_next;
    wait_loads();
    __syncthreads();
    if (it + 1 < cnt) n_next = issue(it + 1, st ^ 1);
    const uint16_t* sK = reinterpret_cast<const uint16_t*>(smem + 2 * st * TB);
    const uint16_t* sV = reinterpret_cast<const uint16_t*>(smem + (2 * st + 1) * TB);
    // S^T: rows = keys 32kh + acc_row32(e, g), column = query qrow
    f32x16 sc = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s) sc = mma32(lds8<bf16x8>(sK + tofs(32 * kh + l32, 16 * s + 8 * g)), qf[s], sc);
    // V^T operands of this wave's key half, read while the softmax runs
    bf16x8 vt[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      vt[t][0] = ldtr(sV, t, 2 * kh);
      vt[t][1] = ldtr(sV, t, 2 * kh + 1);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float v = 32 * kh + acc_row32(e, g) < nJ ? sc[e] * sl2 : -INFINITY;
      sc[e] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, xor32(mx));  // lane l^32 holds the other rows of the column
    // The reference m moves only when some query's max exceeds it by more than kLazy (or
    // on its first valid key): the probabilities exp2(s - m) then stay below 2^kLazy, which
    // fp32 sums and the split bf16 P carry without loss, and O^T is rescaled (which waits
    // for the previous products) only on those rare steps.
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {
      const float mn = fmaxf(m, mx);
      const float alpha = mn == -INFINITY ? 1.f : exp2_fast(m - mn);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] *= alpha;
      m = mn;
    }
    const float mref = m == -INFINITY ? 0.f : m;  // no valid key yet in this half
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = exp2_fast(sc[e] - mref);
      sc[e] = p;
      rs += p;
    }
    rs += xor32(rs);
    l += rs;
    if constexpr (H) {
      const f16x8 p0 = pack8h(sc, 0), p1 = pack8h(sc, 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        o[t] = mma32h(__builtin_bit_cast(f16x8, vt[t][0]), p0, o[t]);
        o[t] = mma32h(__builtin_bit_cast(f16x8, vt[t][1]), p1, o[t]);
      }
    } else {
      bf16x8 h0, r0_, h1, r1_;
      split8(sc, 0, h0, r0_);
      split8(sc, 1, h1, r1_);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        o[t] = mma32(vt[t][0], h0, o[t]);
        o[t] = mma32(vt[t][0], r0_, o[t]);
        o[t] = mma32(vt[t][1], h1, o[t]);
        o[t] = mma32(vt[t][1], r1_, o[t]);
      }
    }
  }
  // merge the key halves: waves with kh = 1 hand (m, l, O^T) to kh = 0 through LDS
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem) + qh * (4 * 16 * 64 + 2 * 64);
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(t * 16 + e) * 64 + lane] = o[t][e];
    red[4 * 16 * 64 + lane] = m;
    red[4 * 16 * 64 + 64 + lane] = l;
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float m1 = red[4 * 16 * 64 + lane], l1 = red[4 * 16 * 64 + 64 + lane];
    const float mm = fmaxf(m, m1);
    const float mref = mm == -INFINITY ? 0.f : mm;
    const float a0 = exp2_fast(m - mref), a1 = exp2_fast(m1 - mref);
    l = l * a0 + l1 * a1;
    m = mm;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] = o[t][e] * a0 + red[(t * 16 + e) * 64 + lane] * a1;
  }
  // O, LSE and the row norm are each optional (the norm serves the audio-to-video
  // cross-attention's per-token norm).  A row with nothing to attend (an empty list, or
  // lists of blocks without valid rows: l = 0) gets O = 0 and LSE = 0, as padding rows do.
  if (qok) {
    const float inv = l > 0.f ? vscale / l : 0.f;
    if (O) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) store4_32(O + (q0 + qrow) * D + 32 * t + 8 * j + 4 * g, o[t], j, inv);
    }
    if (a.lse_out && g == 0) a.lse_out[q0 + qrow] = l > 0.f ? (m + log2f(l)) * 0.6931471805599453f : 0.f;
    if (a.norm_out) {
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) ss = fmaf(o[t][e] * inv, o[t][e] * inv, ss);
      ss += xor32(ss);  // both lanes of the query are in this branch
      if (g == 0) a.norm_out[q0 + qrow] = sqrtf(ss);
    }
  } else if (!a.dense && qrow < TR) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) store4_32(O + (q0 + qrow) * D + 32 * t + 8 * j + 4 * g, o[t], j, 0.f);
    if (g == 0) a.lse_out[q0 + qrow] = 0.f;
  }
}

// ------------------------------------------------------------------ dQ (32x32x16)
// Owner: query block I.  Wave w = (qh = w&1, kh = w>>1) handles queries 32qh.. against
// keys 32kh.. of every streamed key block and accumulates a partial dQ^T over its key
// half; the two halves are summed through LDS at the end.  K and V tiles stream through
// two LDS stages: the copy of the next pair is issued right after the barrier that opens
// the current one.
__global__ __launch_bounds__(NT, 2) void k_dq32(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TB];
  __shared__ int sMeta[kMetaCap];
  int I, bh;
  owner_of<16>(a, a.order_q, I, bh);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int qh = w & 1, kh = w >> 1;
  const int nI = nrows_of(a, bh, I);
  const size_t q0 = row0_of(a, bh, I);
  const bf16_t* Q = static_cast<const bf16_t*>(a.q);
  const bf16_t* K = static_cast<const bf16_t*>(a.k);
  const bf16_t* V = static_cast<const bf16_t*>(a.v);
  const bf16_t* Gd = static_cast<const bf16_t*>(a.dout);
  bf16_t* dQ = static_cast<bf16_t*>(a.dq);
  const int cnt = a.dense ? a.nb : (nI > 0 ? clampi(a.sel_cnt[size_t(bh) * a.nb + I], 0, a.k_max) : 0);
  const BlockList bl = load_list(a, bh, a.dense ? nullptr : a.sel_idx + (size_t(bh) * a.nb + I) * a.k_max, cnt, sMeta);
  const int qrow = 32 * qh + l32;
  const bool qok = qrow < nI;
  bf16x8 qf[8], gf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qf[s] = gld8(Q + (q0 + qrow) * D + 16 * s + 8 * g, qok);
    gf[s] = gld8(Gd + (q0 + qrow) * D + 16 * s + 8 * g, qok);
  }
  const float lse2 = qok ? a.lse_in[q0 + qrow] * LOG2E : INFINITY;
  const float Dq = qok ? a.Dbuf[q0 + qrow] : 0.f;
  f32x16 dq[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) dq[t] = zero16();
  const float sl2 = a.scale * LOG2E;

  // stage st: K tile at 2st, V tile at 2st+1
  int pre = list_first(bl, sMeta);
  auto issue = [&](int k, int st) {
    int J, n;
    list_next(a, bh, bl, sMeta, k, pre, J, n, a.nkrows);
    const size_t r0 = row0_of(a, bh, J);
    load_tile(K + r0 * D, n, reinterpret_cast<uint16_t*>(smem + 2 * st * TB));
    load_tile(V + r0 * D, n, reinterpret_cast<uint16_t*>(smem + (2 * st + 1) * TB));
    return n;
  };
  int n_next = cnt > 0 ? issue(0, 0) : 0;
  for (int it = 0; it < cnt; ++it) {
    const int st = it & 1, nJ = n_next;
    wait_loads();
    __syncthreads();
    if (it + 1 < cnt) n_next = issue(it + 1, st ^ 1);
    const uint16_t* sK = reinterpret_cast<const uint16_t*>(smem + 2 * st * TB);
    const uint16_t* sV = reinterpret_cast<const uint16_t*>(smem + (2 * st + 1) * TB);
    // S^T, dP^T: rows = keys 32kh + acc_row32(e, g), column = query qrow
    f32x16 st_ = zero16(), dp = zero16();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      st_ = mma32(lds8<bf16x8>(sK + tofs(32 * kh + l32, 16 * s + 8 * g)), qf[s], st_);
      dp = mma32(lds8<bf16x8>(sV + tofs(32 * kh + l32, 16 * s + 8 * g)), gf[s], dp);
    }
    // the first K^T operands of the dQ product, read before the softmax step
    const auto preK0 = ldtr(sK, 0, 2 * kh), preK1 = ldtr(sK, 0, 2 * kh + 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool ok = 32 * kh + acc_row32(e, g) < nJ;
      const float p = ok ? exp2_fast(st_[e] * sl2 - lse2) : 0.f;
      dp[e] = p * (dp[e] - Dq);
    }
    const bf16x8 s0 = pack8(dp, 0), s1 = pack8(dp, 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dq[t] = mma32(t == 0 ? preK0 : ldtr(sK, t, 2 * kh), s0, dq[t]);
      dq[t] = mma32(t == 0 ? preK1 : ldtr(sK, t, 2 * kh + 1), s1, dq[t]);
    }
  }
  // sum the two key halves: waves with kh = 1 hand their partials to kh = 0 through LDS
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem) + qh * (4 * 16 * 64);
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(t * 16 + e) * 64 + lane] = dq[t][e];
  }
  __syncthreads();
  if (kh == 0 && (qok || (!a.dense && qrow < TR))) {
    const float sc = qok ? a.scale : 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) dq[t][e] += red[(t * 16 + e) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) store4_32(dQ + (q0 + qrow) * D + 32 * t + 8 * j + 4 * g, dq[t], j, sc);
    }
  }
}

// ------------------------------------------------------------------ dK / dV (32x32x16)
// Owner: key block J.  Wave w = (kh = w&1, x = w>>1): keys 32kh.. of the owner block,
// queries 32x.. of each streamed query block for S and dP.  Wave (kh, 0) accumulates dV^T
// and wave (kh, 1) dK^T of those 32 keys over all 64 queries: after the softmax step the
// pair swaps halves through LDS (x = 0 hands over its dS, x = 1 its P), so neither keeps a
// partial sum of the other's output and no reduction is left for the end.  Each wave adds
// its own query half first, then its partner's.  Q, dO, LSE and D stream through two LDS
// stages, copied without passing through registers.  The role x is a compile-time
// parameter of the pair loop (one copy per role), so choosing between P and dS, or Q and
// dO, costs no instructions; query rows past a block's valid rows get LSE = +inf, so
// their P and dS come out as exact zeros from the exponential itself.
constexpr int kMetaCapKV = 1280;  // keeps two workgroups per CU within 160 KB of LDS
template <int X>
struct Role {
  static constexpr int x = X;
};
__global__ __launch_bounds__(NT, 2) void k_dkdv32(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TB + 4 * 2048];
  __shared__ __attribute__((aligned(16))) float sLD[2][4][TR];  // [stage][LSE*log2(e), D, .., ..][row]
  __shared__ int sMeta[kMetaCapKV];
  bf16x8* xbuf = reinterpret_cast<bf16x8*>(smem + 4 * TB);  // 2 KB per wave
  int J, bh;
  owner_of<64>(a, a.order_k, J, bh);
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            g = lane >> 5;
  const int kh = w & 1;
  const int nJ = nrows_of(a, bh, J);
  const size_t k0 = row0_of(a, bh, J);
  const bf16_t* Q = static_cast<const bf16_t*>(a.q);
  const bf16_t* K = static_cast<const bf16_t*>(a.k);
  const bf16_t* V = static_cast<const bf16_t*>(a.v);
  const bf16_t* Gd = static_cast<const bf16_t*>(a.dout);
  int cnt = 0;
  const int32_t* lst = nullptr;
  if (a.dense) {
    cnt = a.nb;
  } else if (nJ > 0) {
    const RevRange rr = rev_range(a.rev_ptr + size_t(bh) * (a.nb + 1), J, a.nb, a.k_max);
    cnt = rr.cnt;
    lst = a.rev_idx + size_t(bh) * a.nb * a.k_max + rr.start;
  }
  const BlockList bl = load_list<kMetaCapKV>(a, bh, lst, cnt, sMeta);
  const int key = 32 * kh + l32;
  const bool kok = key < nJ;
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    kf[s] = gld8(K + (k0 + key) * D + 16 * s + 8 * g, kok);
    vf[s] = gld8(V + (k0 + key) * D + 16 * s + 8 * g, kok);
  }
  const float sl2 = a.scale * LOG2E;

  auto run = [&](auto role) {
    constexpr int x = decltype(role)::x;
    f32x16 acc[4];  // x = 0: dV^T, x = 1: dK^T (rows d = 32t + acc_row32, column key)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = zero16();
    // stage st: Q tile at 2st, dO tile at 2st+1 (copied to LDS directly); the LSE or D
    // value of row `lane` comes through a register (odd waves D, even waves LSE) and is
    // written to sLD[st][w] before the barrier that opens the stage.
    float ld = 0.f;
    int pre = list_first(bl, sMeta);
    auto issue = [&](int k, int st) {
      int Ib, n;
      list_next(a, bh, bl, sMeta, k, pre, Ib, n, a.nrows);
      const size_t r0 = row0_of(a, bh, Ib);
      load_tile(Q + r0 * D, n, reinterpret_cast<uint16_t*>(smem + 2 * st * TB));
      load_tile(Gd + r0 * D, n, reinterpret_cast<uint16_t*>(smem + (2 * st + 1) * TB));
      ld = ((w & 1) ? a.Dbuf : a.lse_in)[r0 + max(min(lane, n - 1), 0)];
      return n;
    };
    int n_next = cnt > 0 ? issue(0, 0) : 0;
    for (int it = 0; it < cnt; ++it) {
      const int st = it & 1, nIn = n_next;
      wait_loads();
      // rows past the valid ones repeat the last valid row (finite); LSE = +inf gives them P = 0
      sLD[st][w][lane] = (w & 1) ? ld : (lane < nIn ? ld * LOG2E : INFINITY);
      __syncthreads();
      if (it + 1 < cnt) n_next = issue(it + 1, st ^ 1);
      const uint16_t* sQ = reinterpret_cast<const uint16_t*>(smem + 2 * st * TB);
      const uint16_t* sG = reinterpret_cast<const uint16_t*>(smem + (2 * st + 1) * TB);
      // LSE and D of this lane's 16 rows (4 runs of 4), read before the products
      f32x4 lr[4], dr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lr[q] = *reinterpret_cast<const f32x4*>(&sLD[st][0][32 * x + 8 * q + 4 * g]);
        dr[q] = *reinterpret_cast<const f32x4*>(&sLD[st][1][32 * x + 8 * q + 4 * g]);
      }
      // S, dP: rows = queries 32x + acc_row32(e, g), column = key
      f32x16 s_ = zero16(), dp = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        s_ = mma32(lds8<bf16x8>(sQ + tofs(32 * x + l32, 16 * s + 8 * g)), kf[s], s_);
        dp = mma32(lds8<bf16x8>(sG + tofs(32 * x + l32, 16 * s + 8 * g)), vf[s], dp);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2_fast(s_[e] * sl2 - lr[e >> 2][e & 3]);
        s_[e] = p;
        dp[e] = p * (dp[e] - dr[e >> 2][e & 3]);
      }
      // own: the operand this wave keeps (P for dV, dS for dK); give: the one its partner needs
      const f32x16& ownf = x == 0 ? s_ : dp;
      const f32x16& givef = x == 0 ? dp : s_;
      const bf16x8 own0 = pack8(ownf, 0), own1 = pack8(ownf, 1);
      const bf16x8 give0 = pack8(givef, 0), give1 = pack8(givef, 1);
      // the transposed operands: dO^T for dV, Q^T for dK; rows of the own query half are
      // the 16-row groups 2x, 2x+1, the partner's 2(1-x), 2(1-x)+1.  The products with the
      // own half do not depend on the swap: they run before its barrier, so the matrix
      // cores work through the wait; the partner's half follows it.
      const uint16_t* At = x == 0 ? sG : sQ;
      constexpr int jo = 2 * x, jp = 2 * (1 - x);
      xbuf[w * 128 + lane] = give0;
      xbuf[w * 128 + 64 + lane] = give1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[t] = mma32(ldtr(At, t, jo), own0, acc[t]);
        acc[t] = mma32(ldtr(At, t, jo + 1), own1, acc[t]);
      }
      const auto pre2 = ldtr(At, 0, jp), pre3 = ldtr(At, 0, jp + 1);
      __syncthreads();
      const bf16x8 got0 = xbuf[(w ^ 2) * 128 + lane], got1 = xbuf[(w ^ 2) * 128 + 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[t] = mma32(t == 0 ? pre2 : ldtr(At, t, jp), got0, acc[t]);
        acc[t] = mma32(t == 0 ? pre3 : ldtr(At, t, jp + 1), got1, acc[t]);
      }
    }
    if (kok || (!a.dense && key < TR)) {
      const float sc = kok ? (x == 1 ? a.scale : 1.f) : 0.f;
      bf16_t* out = static_cast<bf16_t*>(x == 1 ? a.dk : a.dv);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) store4_32(out + (k0 + key) * D + 32 * t + 8 * j + 4 * g, acc[t], j, sc);
    }
  };
  // the role is uniform over each wave; both copies pass the same barriers in the same order
  if ((w >> 1) == 0)
    run(Role<0>{});
  else
    run(Role<1>{});
}

// ------------------------------------------------------------------ fp16 copy of V
// The forward's P V product runs in fp16 on a copy of V scaled per head by 2^s, with s
// chosen so that the head's largest |V| lands in [2^14, 2^15): every bf16 value of the
// head within a factor 2^29 of that maximum is then exact in fp16 (8 significant bits fit
// the 11 of fp16) and nothing overflows.  The epilogue multiplies by 2^-s.  A head whose
// maximum is 0 or not finite keeps s = 0 (NaN and infinity pass through as they would).
// One pass finds the maxima (atomicMax on the bits of non-negative floats: the result
// does not depend on the order), one writes the copy.
__global__ void k_zero_u32(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}
__global__ __launch_bounds__(256) void k_vmax(const u32x4* __restrict__ v, size_t chunks_per_head,
                                              uint32_t* __restrict__ vmax) {
  const int bh = blockIdx.y;
  const u32x4* src = v + size_t(bh) * chunks_per_head;
  float m = 0.f;
  auto take = [&](const u32x4& u) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, fabsf(__uint_as_float(u[j] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(u[j] & 0xffff0000u)));
    }
  };
  // four independent loads in flight per thread, then the remainder one at a time
  const size_t stride = size_t(gridDim.x) * 256;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < chunks_per_head; i += 4 * stride) {
    u32x4 u[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < 4; ++k) take(u[k]);
  }
  for (; i < chunks_per_head; i += stride) take(src[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomicMax(vmax + bh, __float_as_uint(m));
}
__device__ __forceinline__ float v16_scale(uint32_t mbits) {
  const float m = __uint_as_float(mbits);
  if (!(m > 0.f) || !isfinite(m)) return 1.f;
  int ex;
  (void)frexpf(m, &ex);                       // m = f 2^ex, f in [0.5, 1)
  return ldexpf(1.f, min(max(15 - ex, -100), 100));
}
__global__ __launch_bounds__(256) void k_v16(const u32x4* __restrict__ v, u32x4* __restrict__ v16,
                                             size_t chunks_per_head, const uint32_t* __restrict__ vmax,
                                             float* __restrict__ vinv) {
  const int bh = blockIdx.y;
  const float sc = v16_scale(vmax[bh]);
  if (blockIdx.x == 0 && threadIdx.x == 0) vinv[bh] = 1.f / sc;  // a power of two: exact
  const u32x4* src = v + size_t(bh) * chunks_per_head;
  u32x4* dst = v16 + size_t(bh) * chunks_per_head;
  auto conv = [&](const u32x4& u) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)(__uint_as_float(u[j] << 16) * sc);
      const _Float16 hi = (_Float16)(__uint_as_float(u[j] & 0xffff0000u) * sc);
      r[j] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    return r;
  };
  const size_t stride = size_t(gridDim.x) * 256;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < chunks_per_head; i += 4 * stride) {
    u32x4 u[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[i + k * stride] = conv(u[k]);
  }
  for (; i < chunks_per_head; i += stride) dst[i] = conv(src[i]);
}

// ------------------------------------------------------------------ tile-gather ceiling
// A measurement kernel, not part of the path: the forward's launch (its schedule, grid,
// workgroup size, LDS footprint and two LDS stages) moving the same bytes with no
// arithmetic.  Every listed K and V tile is copied into LDS by the forward's own copy
// routine, and each owner block's valid Q rows are copied to O, so the kernel reads and
// writes the forward's algorithmic bytes; its time is what the forward's memory traffic
// alone costs with this launch.
__global__ __launch_bounds__(NT, 2) void k_gather_fwd(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TB];
  __shared__ int sMeta[kMetaCap];
  int I, bh;
  owner_of<16>(a, a.order_q, I, bh);
  const int nI = nrows_of(a, bh, I);
  const size_t q0 = row0_of(a, bh, I);
  const bf16_t* K = static_cast<const bf16_t*>(a.k);
  const bf16_t* V = static_cast<const bf16_t*>(a.v);
  const int cnt = nI > 0 ? clampi(a.sel_cnt[size_t(bh) * a.nb + I], 0, a.k_max) : 0;
  const BlockList bl = load_list(a, bh, a.sel_idx + (size_t(bh) * a.nb + I) * a.k_max, cnt, sMeta);
  // the owner block: Q rows in, O rows out (16 bytes per lane, 4 rows per wave step)
  const u32x4* Q = reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.q) + q0 * D);
  u32x4* O = reinterpret_cast<u32x4*>(static_cast<bf16_t*>(a.out) + q0 * D);
  for (int e = threadIdx.x; e < nI * (D / 8); e += NT) O[e] = Q[e];
  int pre = list_first(bl, sMeta);
  auto issue = [&](int k, int st) {
    int J, n;
    list_next(a, bh, bl, sMeta, k, pre, J, n, a.nkrows);
    const size_t r0 = krow0_of(a, bh, J);
    load_tile(K + r0 * D, n, reinterpret_cast<uint16_t*>(smem + 2 * st * TB));
    load_tile(V + r0 * D, n, reinterpret_cast<uint16_t*>(smem + (2 * st + 1) * TB));
  };
  if (cnt > 0) issue(0, 0);
  for (int it = 0; it < cnt; ++it) {
    wait_loads();
    __syncthreads();
    if (it + 1 < cnt) issue(it + 1, (it & 1) ^ 1);
  }
  wait_loads();
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

// Bytes of one workgroup schedule (sparse mode; dense mode needs none).
size_t attn_mfma_sched_bytes(const AttnArgs& a) { return a.dense ? 0 : align256(size_t(a.BH) * a.nb * 4); }

// Forward workspace: [schedule (sparse mode)] [max |V| bits per head] [inverse scale per
// head] [fp16 copy of V, BH x nkrows x d].
size_t attn_mfma_fwd_ws_bytes(const AttnArgs& a) {
  return attn_mfma_sched_bytes(a) + 2 * align256(size_t(a.BH) * 4) + align256(size_t(a.BH) * a.nkrows * D * 2);
}

// ws: attn_mfma_fwd_ws_bytes() bytes of device scratch, or null for the bf16 P V path (no
// copy of V; dense mode only, where no schedule is needed either).
hipError_t launch_attn_fwd_mfma(const AttnArgs& a_in, void* ws, hipStream_t s) {
  AttnArgs a = a_in;
  char* p = static_cast<char*>(ws);
  if (!ws && !a.dense) return hipErrorInvalidValue;  // the schedule needs the workspace
  if (!a.dense) {
    a.order_q = reinterpret_cast<int32_t*>(p);
    hipLaunchKernelGGL(k_schedule, dim3(a.BH), dim3(kSchedThreads), 0, s, a, const_cast<int32_t*>(a.order_q),
                       nullptr);
    p += attn_mfma_sched_bytes(a);
  }
  if (!ws) {
    hipLaunchKernelGGL(k_fwd<false>, dim3(a.nb * a.BH), dim3(NT), 0, s, a);
    return hipGetLastError();
  }
  uint32_t* vmax = reinterpret_cast<uint32_t*>(p);
  p += align256(size_t(a.BH) * 4);
  float* vinv = reinterpret_cast<float*>(p);
  p += align256(size_t(a.BH) * 4);
  a.v16 = p;
  a.vinv = vinv;
  const size_t cph = size_t(a.nkrows) * D / 8;  // 16-byte chunks per head
  // about 2048 workgroups in all, each head's chunks split evenly over its share
  const size_t per_head = a.BH >= 2048 ? 1 : size_t(2048 / a.BH);
  const size_t need = (cph + 255) / 256;
  const unsigned gx = unsigned(need < per_head ? need : per_head);
  hipLaunchKernelGGL(k_zero_u32, dim3((a.BH + 255) / 256), dim3(256), 0, s, vmax, a.BH);
  hipLaunchKernelGGL(k_vmax, dim3(gx, a.BH), dim3(256), 0, s, static_cast<const u32x4*>(a.v), cph, vmax);
  hipLaunchKernelGGL(k_v16, dim3(gx, a.BH), dim3(256), 0, s, static_cast<const u32x4*>(a.v),
                     static_cast<u32x4*>(const_cast<void*>(a.v16)), cph, vmax, vinv);
  hipLaunchKernelGGL(k_fwd<true>, dim3(a.nb * a.BH), dim3(NT), 0, s, a);
  return hipGetLastError();
}

// The forward's tile traffic without its arithmetic (measurement only; sparse mode).
hipError_t launch_gather_fwd_mfma(const AttnArgs& a_in, int32_t* sched, hipStream_t s) {
  AttnArgs a = a_in;
  a.order_q = sched;
  hipLaunchKernelGGL(k_schedule, dim3(a.BH), dim3(kSchedThreads), 0, s, a, sched, nullptr);
  hipLaunchKernelGGL(k_gather_fwd, dim3(a.nb * a.BH), dim3(NT), 0, s, a);
  return hipGetLastError();
}

// sched: 2 * attn_mfma_sched_bytes() bytes of device scratch (sparse mode)
hipError_t launch_attn_bwd_mfma(const AttnArgs& a_in, int32_t* sched, hipEvent_t* marks, hipStream_t s) {
  AttnArgs a = a_in;
  if (marks) (void)hipEventRecord(marks[0], s);
  if (!a.dense) {
    int32_t* order_q = sched;
    int32_t* order_k = sched + attn_mfma_sched_bytes(a) / 4;
    a.order_q = order_q;
    a.order_k = order_k;
    hipLaunchKernelGGL(k_schedule, dim3(2 * a.BH), dim3(kSchedThreads), 0, s, a, order_q, order_k);
  }
  const size_t rows = size_t(a.BH) * a.nrows;
  hipLaunchKernelGGL(k_bwd_pre_bf16, dim3(unsigned((rows + 15) / 16)), dim3(256), 0, s, a, rows);
  if (marks) (void)hipEventRecord(marks[1], s);
  hipLaunchKernelGGL(k_dkdv32, dim3(a.nb * a.BH), dim3(NT), 0, s, a);
  if (marks) (void)hipEventRecord(marks[2], s);
  hipLaunchKernelGGL(k_dq32, dim3(a.nb * a.BH), dim3(NT), 0, s, a);
  if (marks) (void)hipEventRecord(marks[3], s);
  return hipGetLastError();
}

}  // namespace prism
