// Internal declarations of libprism: device helpers shared by the kernels and the host
// launchers called by the C-ABI layer (prism_api.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/prism.h"

namespace prism {

constexpr int kMaxZoneVol = 4096;   // zone-local LDS map of the A2V norm
constexpr int kMaxSelectNb = 32768; // one score row of the selection kernel lives in registers (1024 x 32)
constexpr int kTileRows = 64;       // query/key rows per attention tile

// ----------------------------------------------------------------------------------
// Element access.  bf16 is stored as raw 16-bit words and widened by a shift; narrowing
// uses round-to-nearest-even.
// ----------------------------------------------------------------------------------
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x.bits) << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float f);
template <>
__device__ __forceinline__ float from_f32<float>(float f) {
  return f;
}
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) {
  uint32_t u = __float_as_uint(f);
  bf16_t r;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    r.bits = 0x7fc0;
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
    r.bits = uint16_t(u >> 16);
  }
  return r;
}

// Load 8 consecutive elements starting at p (16-byte aligned for bf16, 32 for f32).
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// The same for data read exactly once: non-temporal loads, which leave the caches' room
// to data that is read again
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load8_once(const bf16_t* p, float (&x)[8]) {
  const nt_u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8_once(const float* p, float (&x)[8]) {
  const nt_f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
  const nt_f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p + 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

// ----------------------------------------------------------------------------------
// Caller-provided device lists (valid counts, selection lists, reverse index) are
// clamped into range before they address memory: a malformed list gives unspecified
// results but no access outside the caller's buffers.
// ----------------------------------------------------------------------------------
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }
// Entries [start, start + cnt) of key block J's reverse list, inside [0, nb * k_max) and at
// most nb long.
struct RevRange {
  int start, cnt;
};
__device__ __forceinline__ RevRange rev_range(const int32_t* rp, int J, int nb, int k_max) {
  const long long cap = (long long)nb * k_max;
  const long long s = min(max((long long)rp[J], 0LL), cap);
  const long long e = min(max((long long)rp[J + 1], s), cap);
  return RevRange{int(s), int(min(e - s, (long long)nb))};
}

// ----------------------------------------------------------------------------------
// Reductions (64-lane wavefronts).
// ----------------------------------------------------------------------------------
// Reductions over the 64 lanes of a wavefront, every lane receiving the result, without
// the LDS crossbar: DPP moves within 16-lane rows (swap neighbours, swap pairs, mirror
// within 8 lanes, mirror within 16 lanes: each step pairs lanes that hold the partial
// results of disjoint groups), then v_permlane16_swap and v_permlane32_swap exchange
// rows and halves.  Every lane combines the same operands (a + b and b + a are equal),
// so all lanes get bitwise equal results.  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t lane_xor16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  auto bits = [](T x) { return __builtin_bit_cast(int, x); };
  auto from = [](int x) { return __builtin_bit_cast(T, x); };
  v = op(v, from(dpp_move<0xB1>(bits(v))));   // quad_perm [1,0,3,2]
  v = op(v, from(dpp_move<0x4E>(bits(v))));   // quad_perm [2,3,0,1]
  v = op(v, from(dpp_move<0x141>(bits(v))));  // row_half_mirror
  v = op(v, from(dpp_move<0x140>(bits(v))));  // row_mirror
  v = op(v, from(int(lane_xor16(uint32_t(bits(v))))));
  v = op(v, from(int(lane_xor32(uint32_t(bits(v))))));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ int wave_sum_i(int v) {
  return wave_reduce(v, [](int x, int y) { return x + y; });
}

// Sum over a workgroup of NT threads; `red` holds at least NT/64 floats.  Every thread
// gets the result.  Fixed order, so the result is deterministic.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  constexpr int NW = NT / 64;
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += red[i];
  return s;
}
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  constexpr int NW = NT / 64;
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) s = fmaxf(s, red[i]);
  return s;
}
template <int NT>
__device__ __forceinline__ int block_sum_i(int v, int* red) {
  constexpr int NW = NT / 64;
  v = wave_sum_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += red[i];
  return s;
}
// Exclusive prefix sum of one int per thread over the workgroup (thread order); the
// total is returned through *total.  `red` holds at least NT/64 + 1 ints.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* red, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  __syncthreads();
  if (lane == 63) red[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) off += red[i];
    tot += red[i];
  }
  *total = tot;
  return off + incl - v;
}

// ----------------------------------------------------------------------------------
// Host-side geometry shared by the launchers.
// ----------------------------------------------------------------------------------
struct Geo {
  int T, H, W, zt, zh, zw, nzt, nzh, nzw;
  int nZ, Vz, N;
};

struct ShapeTab {
  int n, vol;  // vol: the slot unit (every candidate's volume when uniform)
  int bt[PRISM_MAX_SHAPES], bh[PRISM_MAX_SHAPES], bw[PRISM_MAX_SHAPES];
  float lg[PRISM_MAX_SHAPES][3];  // log2 of each extent
  int feasible[PRISM_MAX_SHAPES];
  int cvol[PRISM_MAX_SHAPES];     // each candidate's own volume (a multiple of vol)
  int uniform;                    // every candidate holds vol tokens
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse_in;
  float* Dbuf;
  void* out;
  float* lse_out;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* bvalid;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  const int32_t* rev_ptr;
  const int32_t* rev_idx;
  int BH, nb, vol, k_max, nrows, d;
  int dense;  // 1: unpermuted [N][d] tensors, 64-row tiles, every block selected
  float scale;
  // Key side of a dense forward: rows and 64-row blocks of K/V per head (equal to nrows
  // and nb except for a cross-attention, whose keys are a different sequence).
  int nkrows, nkb;
  float* norm_out;  // forward only, nullable: L2 norm of each output row, float [BH][nrows]
  // Matrix-core kernels, sparse mode: the order in which workgroups take their owner
  // blocks, int32 [BH * nb] of bh * nb + block (query-major kernels: order_q, key-major:
  // order_k); null = the kernels' own fixed order.  Set by the launchers.
  const int32_t* order_q;
  const int32_t* order_k;
  // Matrix-core forward, fp16 P V path: V' as fp16 scaled per head by a power of two
  // ([BH][nkrows][d]) and the inverse scale of each head.  Set by the launcher.
  const void* v16;
  const float* vinv;
};

// Launchers (each returns the first HIP error of its launches).
// aux: the A2V output rows [BH][N][d] (dtype dt), or with from_norm the norm map float [BH][N]
hipError_t launch_zone_stats(const void* v, const void* aux, prism_dtype dt, int BH, int d, const Geo& g,
                             bool global_variance, bool from_norm, float* stats, float* vact, hipStream_t s);
hipError_t launch_assign_shapes(const float* stats, int BH, const Geo& g, const ShapeTab& tab,
                                const prism_shape_params& p, int32_t* shape_id, float* margin,
                                hipStream_t s);
// mixed volumes (unit 64, candidates of 64, 128 and 256 tokens) chosen by thresholds on
// the zone activity vact
hipError_t launch_assign_shapes_multi(const float* stats, const float* vact, int BH, const Geo& g,
                                      const ShapeTab& tab, const prism_shape_params& p, float tau_128,
                                      float tau_256, int32_t* shape_id, float* margin, hipStream_t s);
hipError_t launch_block_heads(const int32_t* unit_valid, const int32_t* shape_id, int BH, const Geo& g,
                              const ShapeTab& tab, int32_t* block_valid, hipStream_t s);
// pooled: optional out float [BH][nb][d], the mean of each unit's valid rows (forward only)
hipError_t launch_permute(const void* x, void* y, prism_dtype dt, int BH, int d, const Geo& g,
                          const ShapeTab& tab, const int32_t* shape_id, int inverse,
                          int32_t* block_valid, float* pooled, hipStream_t s);
hipError_t launch_select(const void* qp, const void* kp, prism_dtype dt, const int32_t* bvalid,
                         int BH, int nb, int vol, int d, float scale, const prism_select_params& p,
                         int32_t* sel_idx, int32_t* sel_cnt, int32_t* rev_ptr, int32_t* rev_idx,
                         float* sel_margin, void* ws, hipStream_t s);
// with pooled means given by the caller (qbar, kbar float [BH][nb][d])
hipError_t launch_select_pooled(const float* qbar, const float* kbar, const int32_t* bvalid, int BH, int nb, int d,
                                float scale, const prism_select_params& p, int32_t* sel_idx, int32_t* sel_cnt,
                                int32_t* rev_ptr, int32_t* rev_idx, float* sel_margin, void* ws, hipStream_t s);
size_t select_ws_bytes(int BH, int nb, int d, bool with_pooled);
// Attention: the bf16 / d=128 / 64-token path runs on MFMA kernels, everything else on the
// scalar kernels.  The forward needs no scratch; the backward's holds D (one float per row).
size_t attn_fwd_ws_bytes(const AttnArgs& a, prism_dtype dt);
size_t attn_bwd_ws_bytes(const AttnArgs& a, prism_dtype dt);
size_t tiles_ws_bytes(int BH, int nb, int vol);
size_t tiles_mixed_ws_bytes(int BH, int nb);
hipError_t launch_blocks_to_tiles_mixed(const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                        const int32_t* rev_ptr, const int32_t* rev_idx, int BH, int nb, int k_max,
                                        int max_units, int32_t* tile_idx, int32_t* tile_cnt, int32_t* tile_rev_ptr,
                                        int32_t* tile_rev_idx, void* ws, hipStream_t s);
hipError_t launch_blocks_to_tiles(const int32_t* bvalid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                  const int32_t* rev_ptr, const int32_t* rev_idx, int BH, int nb, int vol, int k_max,
                                  int32_t* tile_valid, int32_t* tile_idx, int32_t* tile_cnt, int32_t* tile_rev_ptr,
                                  int32_t* tile_rev_idx, void* ws, hipStream_t s);
// sched: device scratch for the workgroup schedule of a sparse launch (null in dense mode)
// ws: attn_mfma_fwd_ws_bytes() bytes, or null (dense mode only) for the bf16 P V path
hipError_t launch_attn_fwd_mfma(const AttnArgs& a, void* ws, hipStream_t s);
int attn_mfma_supported(const AttnArgs& a, prism_dtype dt);
hipError_t launch_attn_fwd(const AttnArgs& a, prism_dtype dt, void* ws, hipStream_t s);
hipError_t launch_attn_bwd(const AttnArgs& a, prism_dtype dt, void* ws, hipEvent_t* marks, hipStream_t s);

// Bytes of the matrix-core forward's workspace: the workgroup schedule (sparse mode), then
// the fp16 copy of V and its per-head scales.
size_t attn_mfma_fwd_ws_bytes(const AttnArgs& a);

// Measurement kernels (not part of the path): the matrix-core peak and clock, and the
// forward's tile traffic without arithmetic.
hipError_t launch_mfma_peak(int workgroups, int iters, unsigned long long* clocks, float* sink, hipStream_t s);
hipError_t launch_stream_read(const void* a, const void* b, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_gather_fwd_mfma(const AttnArgs& a, int32_t* sched, hipStream_t s);
size_t attn_mfma_sched_bytes(const AttnArgs& a);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace prism
