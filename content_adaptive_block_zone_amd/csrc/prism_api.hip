// C-ABI entry points of libprism (declared in include/prism.h).  Every call validates its
// arguments on the host, fills the launch descriptors and enqueues the kernels on the
// caller's stream.  No device memory is allocated here; errors are reported through
// prism_status plus a thread-local message.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "prism_internal.h"

using namespace prism;

// Scratch of the allocation-free backward (prism_sparse_attn_bwd_noalloc): a file-scope
// device array, one copy per GPU, held until the process ends.  Host code never passes
// the array's name to a kernel (in host code it is only a stand-in for the symbol): the
// device address of each GPU's copy is looked up once, with that GPU current, and kept.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

thread_local std::string g_err;

prism_status fail(prism_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

prism_status ok() {
  g_err.clear();
  return PRISM_OK;
}

prism_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PRISM_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool valid_dtype(prism_dtype dt) { return dt == PRISM_F32 || dt == PRISM_BF16; }
size_t esize(prism_dtype dt) { return dt == PRISM_BF16 ? 2 : 4; }

prism_status check_grid(const prism_grid* g, Geo* out) {
  if (!g) return fail(PRISM_ERR_ARG, "grid is null");
  if (g->T < 1 || g->H < 1 || g->W < 1) return fail(PRISM_ERR_ARG, "grid extents must be >= 1");
  if (g->zt < 1 || g->zh < 1 || g->zw < 1) return fail(PRISM_ERR_ARG, "zone extents must be >= 1");
  const int64_t vz = int64_t(g->zt) * g->zh * g->zw;
  if (vz > kMaxZoneVol) return fail(PRISM_ERR_SHAPE, "zone volume %lld exceeds %d", (long long)vz, kMaxZoneVol);
  const int64_t n = int64_t(g->T) * g->H * g->W;
  if (n > (int64_t(1) << 30)) return fail(PRISM_ERR_SHAPE, "grid too large");
  Geo o;
  o.T = g->T; o.H = g->H; o.W = g->W;
  o.zt = g->zt; o.zh = g->zh; o.zw = g->zw;
  o.nzt = (g->T + g->zt - 1) / g->zt;
  o.nzh = (g->H + g->zh - 1) / g->zh;
  o.nzw = (g->W + g->zw - 1) / g->zw;
  o.nZ = o.nzt * o.nzh * o.nzw;
  o.Vz = int(vz);
  o.N = int(n);
  if (out) *out = o;
  return PRISM_OK;
}

prism_status check_shapes(const prism_shapes* s, const Geo& g, ShapeTab* out) {
  if (!s) return fail(PRISM_ERR_ARG, "shapes is null");
  if (s->n < 1 || s->n > PRISM_MAX_SHAPES) return fail(PRISM_ERR_ARG, "shapes->n must be in [1, %d]", PRISM_MAX_SHAPES);
  if (s->vol < 1) return fail(PRISM_ERR_ARG, "shapes->vol must be >= 1");
  if (g.Vz % s->vol != 0) return fail(PRISM_ERR_SHAPE, "zone volume %d is not a multiple of block volume %d", g.Vz, s->vol);
  ShapeTab t = {};
  t.n = s->n;
  t.vol = s->vol;
  t.uniform = 1;
  int nfeas = 0;
  for (int c = 0; c < s->n; ++c) {
    if (s->bt[c] < 1 || s->bh[c] < 1 || s->bw[c] < 1) return fail(PRISM_ERR_ARG, "shape %d has an extent < 1", c);
    const int64_t cv = int64_t(s->bt[c]) * s->bh[c] * s->bw[c];
    // a candidate holds vol tokens, or (mixed sets) a multiple of vol that divides the zone
    if (cv % s->vol != 0 || cv > g.Vz || g.Vz % cv != 0)
      return fail(PRISM_ERR_SHAPE, "shape %d (%dx%dx%d) holds %lld tokens: not a multiple of vol=%d dividing the zone",
                  c, s->bt[c], s->bh[c], s->bw[c], (long long)cv, s->vol);
    t.cvol[c] = int(cv);
    if (cv != s->vol) t.uniform = 0;
    t.bt[c] = s->bt[c];
    t.bh[c] = s->bh[c];
    t.bw[c] = s->bw[c];
    t.lg[c][0] = float(std::log2(double(s->bt[c])));
    t.lg[c][1] = float(std::log2(double(s->bh[c])));
    t.lg[c][2] = float(std::log2(double(s->bw[c])));
    t.feasible[c] = (g.zt % s->bt[c] == 0) && (g.zh % s->bh[c] == 0) && (g.zw % s->bw[c] == 0);
    nfeas += t.feasible[c];
  }
  if (nfeas == 0) return fail(PRISM_ERR_SHAPE, "no candidate shape tiles the %dx%dx%d zone", g.zt, g.zh, g.zw);
  if (out) *out = t;
  return PRISM_OK;
}

// B*Hh heads times `units` workgroups (zones, blocks) per head must fit the launches'
// 32-bit grid and the kernels' 32-bit per-launch indices
bool heads_fit(int B, int Hh, int64_t units) {
  // each factor is bounded first, so that no product below can overflow int64
  const int64_t heads = int64_t(B) * int64_t(Hh);
  if (heads > int64_t(INT32_MAX) || units > int64_t(INT32_MAX)) return false;
  return heads * units <= int64_t(INT32_MAX);
}

prism_status check_heads(const char* who, int B, int Hh, int64_t units) {
  if (!heads_fit(B, Hh, units))
    return fail(PRISM_ERR_SHAPE, "%s: B*Hh = %lld heads of %lld units each exceed 2^31 - 1 in all", who,
                (long long)(int64_t(B) * Hh), (long long)units);
  return PRISM_OK;
}

bool supported_attn_d(int d) { return d == 64 || d == 128; }
bool supported_stats_d(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

}  // namespace

extern "C" {

const char* prism_last_error(void) { return g_err.c_str(); }

int64_t prism_num_zones(const prism_grid* grid) {
  Geo g;
  if (check_grid(grid, &g) != PRISM_OK) return -1;
  return g.nZ;
}

int64_t prism_num_blocks(const prism_grid* grid, const prism_shapes* shapes) {
  Geo g;
  if (check_grid(grid, &g) != PRISM_OK) return -1;
  if (check_shapes(shapes, g, nullptr) != PRISM_OK) return -1;
  return int64_t(g.nZ) * (g.Vz / shapes->vol);
}

static prism_status zone_stats_common(const char* who, bool global_variance, bool from_norm, const void* v,
                                      const void* aux, prism_dtype dtype, int B, int Hh, int d,
                                      const prism_grid* grid, float* stats, hipStream_t stream,
                                      float* vact = nullptr) {
  if (!v || !aux || !stats) return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (B < 1 || Hh < 1) return fail(PRISM_ERR_ARG, "%s: B and Hh must be >= 1", who);
  if (!valid_dtype(dtype)) return fail(PRISM_ERR_DTYPE, "%s: unknown dtype %d", who, int(dtype));
  if (!supported_stats_d(d)) return fail(PRISM_ERR_DTYPE, "%s: d=%d not in {32,64,128,256}", who, d);
  Geo g;
  prism_status st = check_grid(grid, &g);
  if (st != PRISM_OK) return st;
  st = check_heads(who, B, Hh, g.nZ);
  if (st != PRISM_OK) return st;
  return launched(launch_zone_stats(v, aux, dtype, B * Hh, d, g, global_variance, from_norm, stats, vact, stream),
                  who);
}

prism_status prism_zone_stats(const void* v, const void* a2v, prism_dtype dtype, int B, int Hh, int d,
                              const prism_grid* grid, float* stats, hipStream_t stream) {
  return zone_stats_common("prism_zone_stats", false, false, v, a2v, dtype, B, Hh, d, grid, stats, stream);
}

prism_status prism_zone_stats_global(const void* v, const void* a2v, prism_dtype dtype, int B, int Hh, int d,
                                     const prism_grid* grid, float* stats, hipStream_t stream) {
  return zone_stats_common("prism_zone_stats_global", true, false, v, a2v, dtype, B, Hh, d, grid, stats, stream);
}

prism_status prism_zone_stats_from_norm(const void* v, const float* a2v_norm, prism_dtype dtype, int B, int Hh,
                                        int d, const prism_grid* grid, int global_variance, float* stats,
                                        hipStream_t stream) {
  return zone_stats_common("prism_zone_stats_from_norm", global_variance != 0, true, v, a2v_norm, dtype, B, Hh,
                           d, grid, stats, stream);
}


prism_status prism_zone_stats_ex(const void* v, const void* aux, prism_dtype dtype, int B, int Hh, int d,
                                 const prism_grid* grid, int flags, float* stats, float* vact, hipStream_t stream) {
  if (flags & ~(PRISM_STATS_GLOBAL_VARIANCE | PRISM_STATS_FROM_NORM))
    return fail(PRISM_ERR_ARG, "prism_zone_stats_ex: unknown flags 0x%x", unsigned(flags));
  return zone_stats_common("prism_zone_stats_ex", (flags & PRISM_STATS_GLOBAL_VARIANCE) != 0,
                           (flags & PRISM_STATS_FROM_NORM) != 0, v, aux, dtype, B, Hh, d, grid, stats, stream, vact);
}

prism_status prism_assign_shapes(const float* stats, int B, int Hh, const prism_grid* grid,
                                 const prism_shapes* shapes, const prism_shape_params* params,
                                 int32_t* shape_id, float* margin, hipStream_t stream) {
  if (!stats || !shape_id || !params) return fail(PRISM_ERR_ARG, "prism_assign_shapes: null pointer");
  if (B < 1 || Hh < 1) return fail(PRISM_ERR_ARG, "prism_assign_shapes: B and Hh must be >= 1");
  Geo g;
  prism_status st = check_grid(grid, &g);
  if (st != PRISM_OK) return st;
  ShapeTab t;
  st = check_shapes(shapes, g, &t);
  if (st != PRISM_OK) return st;
  st = check_heads("prism_assign_shapes", B, Hh, g.nZ);
  if (st != PRISM_OK) return st;
  if (!t.uniform) return fail(PRISM_ERR_SHAPE, "prism_assign_shapes: candidates of several volumes (use prism_assign_shapes_multi)");
  const prism_shape_params p = *params;
  if (!std::isfinite(p.alpha) || !std::isfinite(p.tau_lo) || !std::isfinite(p.tau_hi) || !(p.tau_hi > p.tau_lo))
    return fail(PRISM_ERR_ARG, "prism_assign_shapes: need finite alpha and tau_hi > tau_lo");
  if (!(p.g_min > 0.f) || !(p.eps >= 0.f)) return fail(PRISM_ERR_ARG, "prism_assign_shapes: need g_min > 0, eps >= 0");
  return launched(launch_assign_shapes(stats, B * Hh, g, t, p, shape_id, margin, stream), "prism_assign_shapes");
}

prism_status prism_assign_shapes_multi(const float* stats, const float* vact, int B, int Hh, const prism_grid* grid,
                                       const prism_shapes* shapes, const prism_shape_params* params, float tau_128,
                                       float tau_256, int32_t* shape_id, float* margin, hipStream_t stream) {
  const char* who = "prism_assign_shapes_multi";
  if (!stats || !vact || !shape_id || !params) return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (B < 1 || Hh < 1) return fail(PRISM_ERR_ARG, "%s: B and Hh must be >= 1", who);
  Geo g;
  prism_status st = check_grid(grid, &g);
  if (st != PRISM_OK) return st;
  ShapeTab t;
  st = check_shapes(shapes, g, &t);
  if (st != PRISM_OK) return st;
  st = check_heads(who, B, Hh, g.nZ);
  if (st != PRISM_OK) return st;
  bool unit_feasible = false;
  for (int c = 0; c < t.n; ++c) {
    if (t.cvol[c] != t.vol && t.cvol[c] != 2 * t.vol && t.cvol[c] != 4 * t.vol)
      return fail(PRISM_ERR_SHAPE, "%s: candidate %d holds %d tokens, not 1, 2 or 4 units of %d", who, c, t.cvol[c], t.vol);
    unit_feasible |= t.feasible[c] && t.cvol[c] == t.vol;
  }
  if (!unit_feasible) return fail(PRISM_ERR_SHAPE, "%s: no candidate of the unit volume %d tiles the zone", who, t.vol);
  const prism_shape_params p = *params;
  if (!std::isfinite(p.alpha) || !std::isfinite(p.tau_lo) || !std::isfinite(p.tau_hi) || !(p.tau_hi > p.tau_lo))
    return fail(PRISM_ERR_ARG, "%s: need finite alpha and tau_hi > tau_lo", who);
  if (!(p.g_min > 0.f) || !(p.eps >= 0.f)) return fail(PRISM_ERR_ARG, "%s: need g_min > 0, eps >= 0", who);
  if (!(tau_256 > 0.f) || !(tau_128 >= tau_256) || !std::isfinite(tau_128))
    return fail(PRISM_ERR_ARG, "%s: need 0 < tau_256 <= tau_128 < inf", who);
  return launched(launch_assign_shapes_multi(stats, vact, B * Hh, g, t, p, tau_128, tau_256, shape_id, margin, stream),
                  who);
}

prism_status prism_block_heads(const int32_t* unit_valid, const int32_t* shape_id, int B, int Hh,
                               const prism_grid* grid, const prism_shapes* shapes, int32_t* block_valid,
                               hipStream_t stream) {
  const char* who = "prism_block_heads";
  if (!unit_valid || !shape_id || !block_valid) return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (B < 1 || Hh < 1) return fail(PRISM_ERR_ARG, "%s: B and Hh must be >= 1", who);
  Geo g;
  prism_status st = check_grid(grid, &g);
  if (st != PRISM_OK) return st;
  ShapeTab t;
  st = check_shapes(shapes, g, &t);
  if (st != PRISM_OK) return st;
  st = check_heads(who, B, Hh, int64_t(g.nZ) * (g.Vz / t.vol));
  if (st != PRISM_OK) return st;
  return launched(launch_block_heads(unit_valid, shape_id, B * Hh, g, t, block_valid, stream), who);
}

prism_status prism_permute(const void* x, void* y, prism_dtype dtype, int B, int Hh, int d,
                           const prism_grid* grid, const prism_shapes* shapes, const int32_t* shape_id,
                           int inverse, int32_t* block_valid, hipStream_t stream) {
  if (!x || !y || !shape_id) return fail(PRISM_ERR_ARG, "prism_permute: null pointer");
  if (B < 1 || Hh < 1 || d < 1) return fail(PRISM_ERR_ARG, "prism_permute: B, Hh, d must be >= 1");
  if (inverse != 0 && inverse != 1) return fail(PRISM_ERR_ARG, "prism_permute: inverse must be 0 or 1");
  if (!valid_dtype(dtype)) return fail(PRISM_ERR_DTYPE, "prism_permute: unknown dtype %d", int(dtype));
  if ((size_t(d) * esize(dtype)) % 16 != 0) return fail(PRISM_ERR_DTYPE, "prism_permute: d*sizeof(dtype) must be a multiple of 16");
  if (x == y) return fail(PRISM_ERR_ARG, "prism_permute: x and y must not alias");
  Geo g;
  prism_status st = check_grid(grid, &g);
  if (st != PRISM_OK) return st;
  ShapeTab t;
  st = check_shapes(shapes, g, &t);
  if (st != PRISM_OK) return st;
  st = check_heads("prism_permute", B, Hh, int64_t(g.nZ) * (g.Vz / t.vol));
  if (st != PRISM_OK) return st;
  return launched(launch_permute(x, y, dtype, B * Hh, d, g, t, shape_id, inverse, block_valid, nullptr, stream),
                  "prism_permute");
}

prism_status prism_permute_pool(const void* x, void* y, prism_dtype dtype, int B, int Hh, int d,
                                const prism_grid* grid, const prism_shapes* shapes, const int32_t* shape_id,
                                int32_t* block_valid, float* pooled, hipStream_t stream) {
  const char* who = "prism_permute_pool";
  if (!x || !y || !shape_id || !pooled) return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (B < 1 || Hh < 1 || d < 1) return fail(PRISM_ERR_ARG, "%s: B, Hh, d must be >= 1", who);
  if (!valid_dtype(dtype)) return fail(PRISM_ERR_DTYPE, "%s: unknown dtype %d", who, int(dtype));
  const size_t row_bytes = size_t(d) * esize(dtype);
  const size_t chunks = row_bytes / 16;
  if (row_bytes % 16 != 0 || chunks > 256 || (chunks & (chunks - 1)) != 0)
    return fail(PRISM_ERR_DTYPE, "%s: d*sizeof(dtype) must be 16 bytes times a power of two, at most 4096 bytes", who);
  if (x == y) return fail(PRISM_ERR_ARG, "%s: x and y must not alias", who);
  Geo g;
  prism_status st = check_grid(grid, &g);
  if (st != PRISM_OK) return st;
  ShapeTab t;
  st = check_shapes(shapes, g, &t);
  if (st != PRISM_OK) return st;
  if (!t.uniform) return fail(PRISM_ERR_SHAPE, "%s: candidates of several volumes (blocks span several units)", who);
  st = check_heads(who, B, Hh, int64_t(g.nZ) * (g.Vz / t.vol));
  if (st != PRISM_OK) return st;
  return launched(launch_permute(x, y, dtype, B * Hh, d, g, t, shape_id, 0, block_valid, pooled, stream), who);
}

size_t prism_select_workspace_size(int B, int Hh, int nb, int d) {
  if (B < 1 || Hh < 1 || nb < 1 || d < 1 || !heads_fit(B, Hh, nb)) return 0;
  return select_ws_bytes(B * Hh, nb, d, true);
}

size_t prism_select_pooled_workspace_size(int B, int Hh, int nb) {
  if (B < 1 || Hh < 1 || nb < 1 || !heads_fit(B, Hh, nb)) return 0;
  return select_ws_bytes(B * Hh, nb, 1, false);
}

prism_status prism_select_blocks(const void* qp, const void* kp, prism_dtype dtype, const int32_t* block_valid,
                                 int B, int Hh, int nb, int vol, int d, float scale,
                                 const prism_select_params* params, int32_t* sel_idx, int32_t* sel_cnt,
                                 int32_t* rev_ptr, int32_t* rev_idx, float* sel_margin, void* workspace,
                                 size_t ws_bytes, hipStream_t stream) {
  if (!qp || !kp || !block_valid || !params || !sel_idx || !sel_cnt || !rev_ptr || !rev_idx || !workspace)
    return fail(PRISM_ERR_ARG, "prism_select_blocks: null pointer");
  if (B < 1 || Hh < 1 || nb < 1 || vol < 1) return fail(PRISM_ERR_ARG, "prism_select_blocks: sizes must be >= 1");
  if (nb > kMaxSelectNb) return fail(PRISM_ERR_SHAPE, "prism_select_blocks: nb=%d exceeds %d", nb, kMaxSelectNb);
  if (check_heads("prism_select_blocks", B, Hh, nb) != PRISM_OK) return PRISM_ERR_SHAPE;
  if (!valid_dtype(dtype)) return fail(PRISM_ERR_DTYPE, "prism_select_blocks: unknown dtype %d", int(dtype));
  if (!supported_stats_d(d)) return fail(PRISM_ERR_DTYPE, "prism_select_blocks: d=%d not in {32,64,128,256}", d);
  const prism_select_params p = *params;
  if (!(p.top_p > 0.f && p.top_p <= 1.f)) return fail(PRISM_ERR_ARG, "prism_select_blocks: top_p must be in (0, 1]");
  if (p.k_min < 1 || p.k_max < p.k_min) return fail(PRISM_ERR_ARG, "prism_select_blocks: need 1 <= k_min <= k_max");
  if (!std::isfinite(scale)) return fail(PRISM_ERR_ARG, "prism_select_blocks: scale must be finite");
  if (ws_bytes < select_ws_bytes(B * Hh, nb, d, true))
    return fail(PRISM_ERR_ARG, "prism_select_blocks: workspace of %zu bytes < required %zu", ws_bytes,
                select_ws_bytes(B * Hh, nb, d, true));
  return launched(launch_select(qp, kp, dtype, block_valid, B * Hh, nb, vol, d, scale, p, sel_idx, sel_cnt,
                                rev_ptr, rev_idx, sel_margin, workspace, stream),
                  "prism_select_blocks");
}

prism_status prism_select_blocks_pooled(const float* qbar, const float* kbar, const int32_t* block_valid, int B,
                                        int Hh, int nb, int d, float scale, const prism_select_params* params,
                                        int32_t* sel_idx, int32_t* sel_cnt, int32_t* rev_ptr, int32_t* rev_idx,
                                        float* sel_margin, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const char* who = "prism_select_blocks_pooled";
  if (!qbar || !kbar || !block_valid || !params || !sel_idx || !sel_cnt || !rev_ptr || !rev_idx || !workspace)
    return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (B < 1 || Hh < 1 || nb < 1) return fail(PRISM_ERR_ARG, "%s: sizes must be >= 1", who);
  if (nb > kMaxSelectNb) return fail(PRISM_ERR_SHAPE, "%s: nb=%d exceeds %d", who, nb, kMaxSelectNb);
  if (check_heads(who, B, Hh, nb) != PRISM_OK) return PRISM_ERR_SHAPE;
  if (d < 1 || d % 16 != 0 || d > 4096) return fail(PRISM_ERR_DTYPE, "%s: d=%d must be a multiple of 16 up to 4096", who, d);
  const prism_select_params p = *params;
  if (!(p.top_p > 0.f && p.top_p <= 1.f)) return fail(PRISM_ERR_ARG, "%s: top_p must be in (0, 1]", who);
  if (p.k_min < 1 || p.k_max < p.k_min) return fail(PRISM_ERR_ARG, "%s: need 1 <= k_min <= k_max", who);
  if (!std::isfinite(scale)) return fail(PRISM_ERR_ARG, "%s: scale must be finite", who);
  const size_t need = select_ws_bytes(B * Hh, nb, d, false);
  if (ws_bytes < need) return fail(PRISM_ERR_ARG, "%s: workspace of %zu bytes < required %zu", who, ws_bytes, need);
  return launched(launch_select_pooled(qbar, kbar, block_valid, B * Hh, nb, d, scale, p, sel_idx, sel_cnt, rev_ptr,
                                       rev_idx, sel_margin, workspace, stream),
                  who);
}

static prism_status check_attn_common(const char* who, prism_dtype dtype, int B, int Hh, int nb, int vol, int d,
                                      int k_max, float scale) {
  if (B < 1 || Hh < 1 || nb < 1) return fail(PRISM_ERR_ARG, "%s: B, Hh, nb must be >= 1", who);
  if (!valid_dtype(dtype)) return fail(PRISM_ERR_DTYPE, "%s: unknown dtype %d", who, int(dtype));
  if (!supported_attn_d(d)) return fail(PRISM_ERR_DTYPE, "%s: d=%d not in {64,128}", who, d);
  if (vol < 1 || vol > kTileRows) return fail(PRISM_ERR_SHAPE, "%s: vol=%d must be in [1, %d]", who, vol, kTileRows);
  if ((size_t(vol) * d * esize(dtype)) % 16 != 0) return fail(PRISM_ERR_SHAPE, "%s: vol*d*sizeof(dtype) must be a multiple of 16", who);
  if (k_max < 1) return fail(PRISM_ERR_ARG, "%s: k_max must be >= 1", who);
  if (!std::isfinite(scale)) return fail(PRISM_ERR_ARG, "%s: scale must be finite", who);
  if (!heads_fit(B, Hh, int64_t(nb) * vol)) return fail(PRISM_ERR_SHAPE, "%s: too many rows", who);
  return PRISM_OK;
}

static AttnArgs sparse_args(int B, int Hh, int nb, int vol, int d, int k_max, float scale) {
  AttnArgs a = {};
  a.BH = B * Hh; a.nb = nb; a.vol = vol; a.k_max = k_max; a.nrows = nb * vol; a.d = d;
  a.dense = 0; a.scale = scale;
  a.nkrows = a.nrows; a.nkb = nb;
  return a;
}

static AttnArgs dense_args(int B, int Hh, int N, int d, float scale) {
  AttnArgs a = {};
  const int nb = (N + kTileRows - 1) / kTileRows;
  a.BH = B * Hh; a.nb = nb; a.vol = kTileRows; a.k_max = nb; a.nrows = N; a.d = d;
  a.dense = 1; a.scale = scale;
  a.nkrows = N; a.nkb = nb;
  return a;
}

size_t prism_fwd_workspace_size(int B, int Hh, int nb, int vol, int d, prism_dtype dtype) {
  if (B < 1 || Hh < 1 || nb < 1 || vol < 1 || !valid_dtype(dtype) || !heads_fit(B, Hh, int64_t(nb) * vol)) return 0;
  return attn_fwd_ws_bytes(sparse_args(B, Hh, nb, vol, d, 1, 1.f), dtype);
}

prism_status prism_sparse_attn_fwd(const void* qp, const void* kp, const void* vp, prism_dtype dtype,
                                   const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                   int k_max, int B, int Hh, int nb, int vol, int d, float scale, void* op,
                                   float* lse, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!qp || !kp || !vp || !block_valid || !sel_idx || !sel_cnt || !op || !lse)
    return fail(PRISM_ERR_ARG, "prism_sparse_attn_fwd: null pointer");
  prism_status st = check_attn_common("prism_sparse_attn_fwd", dtype, B, Hh, nb, vol, d, k_max, scale);
  if (st != PRISM_OK) return st;
  AttnArgs a = sparse_args(B, Hh, nb, vol, d, k_max, scale);
  const size_t need = attn_fwd_ws_bytes(a, dtype);
  if (ws_bytes < need || (need > 0 && !workspace))
    return fail(PRISM_ERR_ARG, "prism_sparse_attn_fwd: workspace of %zu bytes < required %zu", ws_bytes, need);
  a.q = qp; a.k = kp; a.v = vp; a.out = op; a.lse_out = lse;
  a.bvalid = block_valid; a.sel_idx = sel_idx; a.sel_cnt = sel_cnt;
  return launched(launch_attn_fwd(a, dtype, workspace, stream), "prism_sparse_attn_fwd");
}

size_t prism_bwd_workspace_size(int B, int Hh, int nb, int vol, int d, prism_dtype dtype) {
  if (B < 1 || Hh < 1 || nb < 1 || vol < 1 || !valid_dtype(dtype) || !heads_fit(B, Hh, int64_t(nb) * vol)) return 0;
  return attn_bwd_ws_bytes(sparse_args(B, Hh, nb, vol, d, 1, 1.f), dtype);
}

prism_status prism_sparse_attn_bwd(const void* qp, const void* kp, const void* vp, const void* op, const void* dop,
                                   const float* lse, prism_dtype dtype, const int32_t* block_valid,
                                   const int32_t* sel_idx, const int32_t* sel_cnt, int k_max,
                                   const int32_t* rev_ptr, const int32_t* rev_idx, int B, int Hh, int nb, int vol,
                                   int d, float scale, void* dqp, void* dkp, void* dvp, void* workspace,
                                   size_t ws_bytes, hipEvent_t* marks, hipStream_t stream) {
  if (!qp || !kp || !vp || !op || !dop || !lse || !block_valid || !sel_idx || !sel_cnt || !rev_ptr || !rev_idx ||
      !dqp || !dkp || !dvp || !workspace)
    return fail(PRISM_ERR_ARG, "prism_sparse_attn_bwd: null pointer");
  prism_status st = check_attn_common("prism_sparse_attn_bwd", dtype, B, Hh, nb, vol, d, k_max, scale);
  if (st != PRISM_OK) return st;
  AttnArgs a = sparse_args(B, Hh, nb, vol, d, k_max, scale);
  const size_t need = attn_bwd_ws_bytes(a, dtype);
  if (ws_bytes < need)
    return fail(PRISM_ERR_ARG, "prism_sparse_attn_bwd: workspace of %zu bytes < required %zu", ws_bytes, need);
  a.q = qp; a.k = kp; a.v = vp; a.o = op; a.dout = dop; a.lse_in = lse;
  a.dq = dqp; a.dk = dkp; a.dv = dvp;
  a.bvalid = block_valid; a.sel_idx = sel_idx; a.sel_cnt = sel_cnt; a.rev_ptr = rev_ptr; a.rev_idx = rev_idx;
  return launched(launch_attn_bwd(a, dtype, workspace, marks, stream), "prism_sparse_attn_bwd");
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch`, looked up on the first call on
// that GPU; the stream must belong to the current GPU.
prism_status noalloc_scratch(const char* who, hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PRISM_ERR_LAUNCH, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PRISM_ERR_ARG, "%s: device %d out of range", who, dev);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(PRISM_ERR_ARG, "%s: hipStreamGetDevice: %s", who, hipGetErrorString(e));
    if (int(sdev) != dev)
      return fail(PRISM_ERR_ARG, "%s: the stream belongs to device %d, the current device is %d", who, int(sdev), dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PRISM_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return PRISM_OK;
}
}  // namespace

prism_status prism_sparse_attn_bwd_noalloc(const void* qp, const void* kp, const void* vp, const void* op,
                                           const void* dop, const float* lse, prism_dtype dtype,
                                           const int32_t* block_valid, const int32_t* sel_idx,
                                           const int32_t* sel_cnt, int k_max, const int32_t* rev_ptr,
                                           const int32_t* rev_idx, int B, int Hh, int nb, int vol, int d,
                                           float scale, void* dqp, void* dkp, void* dvp, hipEvent_t* marks,
                                           hipStream_t stream) {
  const char* who = "prism_sparse_attn_bwd_noalloc";
  if (!qp || !kp || !vp || !op || !dop || !lse || !block_valid || !sel_idx || !sel_cnt || !rev_ptr || !rev_idx ||
      !dqp || !dkp || !dvp)
    return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  prism_status st = check_attn_common(who, dtype, B, Hh, nb, vol, d, k_max, scale);
  if (st != PRISM_OK) return st;
  AttnArgs a = sparse_args(B, Hh, nb, vol, d, k_max, scale);
  const size_t need = attn_bwd_ws_bytes(a, dtype);
  if (need > kNoallocScratchBytes)
    return fail(PRISM_ERR_SHAPE, "%s: needs %zu bytes of scratch; the static scratch holds %zu (use prism_sparse_attn_bwd)",
                who, need, kNoallocScratchBytes);
  void* ws = nullptr;
  st = noalloc_scratch(who, stream, &ws);
  if (st != PRISM_OK) return st;
  a.q = qp; a.k = kp; a.v = vp; a.o = op; a.dout = dop; a.lse_in = lse;
  a.dq = dqp; a.dk = dkp; a.dv = dvp;
  a.bvalid = block_valid; a.sel_idx = sel_idx; a.sel_cnt = sel_cnt; a.rev_ptr = rev_ptr; a.rev_idx = rev_idx;
  return launched(launch_attn_bwd(a, dtype, ws, marks, stream), who);
}

size_t prism_dense_fwd_workspace_size(int B, int Hh, int N, int d, prism_dtype dtype) {
  if (B < 1 || Hh < 1 || N < 1 || !valid_dtype(dtype) || !heads_fit(B, Hh, int64_t(N) + kTileRows)) return 0;
  return attn_fwd_ws_bytes(dense_args(B, Hh, N, d, 1.f), dtype);
}

prism_status prism_dense_attn_fwd(const void* q, const void* k, const void* v, prism_dtype dtype, int B, int Hh,
                                  int N, int d, float scale, void* o, float* lse, void* workspace, size_t ws_bytes,
                                  hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return fail(PRISM_ERR_ARG, "prism_dense_attn_fwd: null pointer");
  if (N < 1) return fail(PRISM_ERR_ARG, "prism_dense_attn_fwd: N must be >= 1");
  const int nb = (N + kTileRows - 1) / kTileRows;
  prism_status st = check_attn_common("prism_dense_attn_fwd", dtype, B, Hh, nb, kTileRows, d, 1, scale);
  if (st != PRISM_OK) return st;
  AttnArgs a = dense_args(B, Hh, N, d, scale);
  const size_t need = attn_fwd_ws_bytes(a, dtype);
  if (ws_bytes < need || (need > 0 && !workspace))
    return fail(PRISM_ERR_ARG, "prism_dense_attn_fwd: workspace of %zu bytes < required %zu", ws_bytes, need);
  a.q = q; a.k = k; a.v = v; a.out = o; a.lse_out = lse;
  return launched(launch_attn_fwd(a, dtype, workspace, stream), "prism_dense_attn_fwd");
}

size_t prism_dense_bwd_workspace_size(int B, int Hh, int N, int d, prism_dtype dtype) {
  if (B < 1 || Hh < 1 || N < 1 || !valid_dtype(dtype) || !heads_fit(B, Hh, int64_t(N) + kTileRows)) return 0;
  return attn_bwd_ws_bytes(dense_args(B, Hh, N, d, 1.f), dtype);
}

prism_status prism_dense_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                  const float* lse, prism_dtype dtype, int B, int Hh, int N, int d, float scale,
                                  void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes, hipEvent_t* marks,
                                  hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return fail(PRISM_ERR_ARG, "prism_dense_attn_bwd: null pointer");
  if (N < 1) return fail(PRISM_ERR_ARG, "prism_dense_attn_bwd: N must be >= 1");
  const int nb = (N + kTileRows - 1) / kTileRows;
  prism_status st = check_attn_common("prism_dense_attn_bwd", dtype, B, Hh, nb, kTileRows, d, 1, scale);
  if (st != PRISM_OK) return st;
  AttnArgs a = dense_args(B, Hh, N, d, scale);
  const size_t need = attn_bwd_ws_bytes(a, dtype);
  if (ws_bytes < need) return fail(PRISM_ERR_ARG, "prism_dense_attn_bwd: workspace of %zu bytes < required %zu", ws_bytes, need);
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse_in = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  return launched(launch_attn_bwd(a, dtype, workspace, marks, stream), "prism_dense_attn_bwd");
}

prism_status prism_a2v_attn_norm(const void* q, const void* ka, const void* va, prism_dtype dtype, int B, int Hh,
                                 int N, int Na, int d, float scale, void* o, float* a2v_norm,
                                 hipStream_t stream) {
  const char* who = "prism_a2v_attn_norm";
  if (!q || !ka || !va || !a2v_norm) return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (B < 1 || Hh < 1 || N < 1 || Na < 1) return fail(PRISM_ERR_ARG, "%s: B, Hh, N, Na must be >= 1", who);
  if (dtype != PRISM_BF16 || d != 128) return fail(PRISM_ERR_DTYPE, "%s: needs bf16 and d = 128", who);
  if (!std::isfinite(scale)) return fail(PRISM_ERR_ARG, "%s: scale must be finite", who);
  if (!heads_fit(B, Hh, int64_t(N) + kTileRows) || !heads_fit(B, Hh, int64_t(Na) + kTileRows))
    return fail(PRISM_ERR_SHAPE, "%s: too many rows", who);
  AttnArgs a = dense_args(B, Hh, N, d, scale);
  a.nkrows = Na;
  a.nkb = (Na + kTileRows - 1) / kTileRows;
  a.q = q; a.k = ka; a.v = va;
  a.out = o;
  a.lse_out = nullptr;
  a.norm_out = a2v_norm;
  return launched(launch_attn_fwd_mfma(a, nullptr, stream), who);  // dense: no schedule
}

prism_status prism_bench_mfma_peak(int workgroups, int iters, uint64_t* clocks, float* sink, hipStream_t stream) {
  const char* who = "prism_bench_mfma_peak";
  if (!clocks || !sink) return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1) return fail(PRISM_ERR_ARG, "%s: need 1 <= workgroups <= 2^20, iters >= 1", who);
  return launched(launch_mfma_peak(workgroups, iters, reinterpret_cast<unsigned long long*>(clocks), sink, stream), who);
}

prism_status prism_bench_stream_read(const void* a, const void* b, size_t bytes, uint32_t* sink,
                                    hipStream_t stream) {
  const char* who = "prism_bench_stream_read";
  if (!a || !b || !sink) return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (bytes == 0 || bytes % 16 != 0) return fail(PRISM_ERR_ARG, "%s: bytes must be a positive multiple of 16", who);
  return launched(launch_stream_read(a, b, bytes, sink, stream), who);
}

prism_status prism_bench_tile_gather(const void* qp, const void* kp, const void* vp, prism_dtype dtype,
                                     const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                     int k_max, int B, int Hh, int nb, int vol, int d, void* op, void* workspace,
                                     size_t ws_bytes, hipStream_t stream) {
  const char* who = "prism_bench_tile_gather";
  if (!qp || !kp || !vp || !block_valid || !sel_idx || !sel_cnt || !op || !workspace)
    return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  prism_status st = check_attn_common(who, dtype, B, Hh, nb, vol, d, k_max, 1.f);
  if (st != PRISM_OK) return st;
  AttnArgs a = sparse_args(B, Hh, nb, vol, d, k_max, 1.f);
  if (!attn_mfma_supported(a, dtype)) return fail(PRISM_ERR_DTYPE, "%s: needs bf16, d = 128 and vol = 64", who);
  const size_t need = attn_mfma_sched_bytes(a);
  if (ws_bytes < need) return fail(PRISM_ERR_ARG, "%s: workspace of %zu bytes < required %zu", who, ws_bytes, need);
  a.q = qp; a.k = kp; a.v = vp; a.out = op;
  a.bvalid = block_valid; a.sel_idx = sel_idx; a.sel_cnt = sel_cnt;
  return launched(launch_gather_fwd_mfma(a, static_cast<int32_t*>(workspace), stream), who);
}

size_t prism_tiles_workspace_size(int B, int Hh, int nb, int vol) {
  if (B < 1 || Hh < 1 || nb < 1 || vol < kTileRows || vol % kTileRows != 0 || !heads_fit(B, Hh, int64_t(nb) * vol))
    return 0;
  return tiles_ws_bytes(B * Hh, nb, vol);
}

prism_status prism_blocks_to_tiles(const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                   const int32_t* rev_ptr, const int32_t* rev_idx, int B, int Hh, int nb, int vol,
                                   int k_max, int32_t* tile_valid, int32_t* tile_idx, int32_t* tile_cnt,
                                   int32_t* tile_rev_ptr, int32_t* tile_rev_idx, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  const char* who = "prism_blocks_to_tiles";
  if (!block_valid || !sel_idx || !sel_cnt || !rev_ptr || !rev_idx || !tile_valid || !tile_idx || !tile_cnt ||
      !tile_rev_ptr || !tile_rev_idx || !workspace)
    return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (B < 1 || Hh < 1 || nb < 1 || k_max < 1) return fail(PRISM_ERR_ARG, "%s: B, Hh, nb, k_max must be >= 1", who);
  if (vol < kTileRows || vol % kTileRows != 0 || vol > 4096)
    return fail(PRISM_ERR_SHAPE, "%s: vol=%d must be a multiple of %d in [%d, 4096]", who, vol, kTileRows, kTileRows);
  const int g = vol / kTileRows;
  if (int64_t(B) * Hh * nb * g * int64_t(k_max) * g > int64_t(INT32_MAX))
    return fail(PRISM_ERR_SHAPE, "%s: tile lists exceed 2^31 entries", who);
  if (ws_bytes < tiles_ws_bytes(B * Hh, nb, vol)) return fail(PRISM_ERR_ARG, "%s: workspace too small", who);
  return launched(launch_blocks_to_tiles(block_valid, sel_idx, sel_cnt, rev_ptr, rev_idx, B * Hh, nb, vol, k_max,
                                         tile_valid, tile_idx, tile_cnt, tile_rev_ptr, tile_rev_idx, workspace, stream),
                  who);
}

size_t prism_tiles_mixed_workspace_size(int B, int Hh, int nb) {
  if (B < 1 || Hh < 1 || nb < 1 || !heads_fit(B, Hh, nb)) return 0;
  return tiles_mixed_ws_bytes(B * Hh, nb);
}

prism_status prism_blocks_to_tiles_mixed(const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                         const int32_t* rev_ptr, const int32_t* rev_idx, int B, int Hh, int nb,
                                         int k_max, int max_units, int32_t* tile_idx, int32_t* tile_cnt,
                                         int32_t* tile_rev_ptr, int32_t* tile_rev_idx, void* workspace,
                                         size_t ws_bytes, hipStream_t stream) {
  const char* who = "prism_blocks_to_tiles_mixed";
  if (!block_valid || !sel_idx || !sel_cnt || !rev_ptr || !rev_idx || !tile_idx || !tile_cnt || !tile_rev_ptr ||
      !tile_rev_idx || !workspace)
    return fail(PRISM_ERR_ARG, "%s: null pointer", who);
  if (B < 1 || Hh < 1 || nb < 1 || k_max < 1) return fail(PRISM_ERR_ARG, "%s: B, Hh, nb, k_max must be >= 1", who);
  if (max_units < 1 || max_units > 64) return fail(PRISM_ERR_ARG, "%s: max_units must be in [1, 64]", who);
  if (int64_t(B) * Hh * nb * int64_t(k_max) * max_units > int64_t(INT32_MAX))
    return fail(PRISM_ERR_SHAPE, "%s: tile lists exceed 2^31 entries", who);
  if (ws_bytes < tiles_mixed_ws_bytes(B * Hh, nb)) return fail(PRISM_ERR_ARG, "%s: workspace too small", who);
  return launched(launch_blocks_to_tiles_mixed(block_valid, sel_idx, sel_cnt, rev_ptr, rev_idx, B * Hh, nb, k_max,
                                               max_units, tile_idx, tile_cnt, tile_rev_ptr, tile_rev_idx, workspace,
                                               stream),
                  who);
}

}  // extern "C"
