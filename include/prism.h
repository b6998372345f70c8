/*
 * libprism: content-adaptive block-sparse video self-attention (Prism) for MI355X.
 *
 * The method (Prism paper, abstract and Figure 2 caption): the video token grid is cut
 * into spatiotemporal macro-zones; each zone gets a block shape chosen from the
 * per-axis variance of the video value features (Table 9 caption, r_{v,d}) and from the
 * norm of the audio-to-video cross-attention output (Table 9 caption, the gate a-bar and
 * the audio directional variance); tokens are permuted so that every block is a
 * contiguous run; block-pooled Q/K scores drive a hybrid Top-k/Top-p selection per
 * query block (Table 7 caption); exact softmax attention then runs over the selected
 * blocks, forward and backward.
 *
 * Conventions shared by every call.
 *   Memory     Every pointer is DEVICE memory allocated and owned by the caller, except
 *              the small descriptor structs (grid, shapes, params), which are HOST
 *              memory read during the call.  The library never allocates or frees device
 *              memory and keeps no state between calls.  Scratch space comes from the
 *              caller through (workspace, ws_bytes); its required size is returned by the
 *              matching *_workspace_size function.
 *   Layout     Token tensors are row-major [B][Hh][N][d] with tokens in t-major raster
 *              order n = (t*H + h)*W + w.  Permuted ("slot order") tensors are
 *              [B][Hh][Npad][d], Npad = nb * vol, where block I owns slots
 *              [I*vol, (I+1)*vol) and its valid rows come first (block_valid[I] of them).
 *   Streams    Each call enqueues its kernels on `stream` (may be 0) and returns without
 *              synchronizing.  Inputs must stay valid until that work has run.
 *   Errors     A call validates every argument on the host before launching anything and
 *              returns a prism_status; on failure nothing has been enqueued and
 *              prism_last_error() gives a message (thread-local, valid until the next call
 *              on that thread).  No C++ exception crosses this interface.
 *   dtypes     PRISM_BF16 (bfloat16 storage, float32 accumulation) or PRISM_F32.
 *              Statistics, pooled means, scores, LSE and D are always float32.
 *   Sizes      B*Hh heads times the zones, blocks or rows a call handles per head must
 *              stay below 2^31 (the launches' grids and per-launch indices are 32-bit);
 *              larger calls return PRISM_ERR_SHAPE and the *_workspace_size functions 0.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PRISM_OK = 0,
  PRISM_ERR_ARG = 1,    /* null pointer, negative size, parameter out of range */
  PRISM_ERR_DTYPE = 2,  /* unknown dtype or dtype/size combination not supported */
  PRISM_ERR_SHAPE = 3,  /* sizes inconsistent with each other (zone, shapes, nb, vol) */
  PRISM_ERR_LAUNCH = 4  /* the HIP runtime refused a launch */
} prism_status;

/* The last two enumerators only widen the type to every 32-bit value, so that any value a
 * caller passes is a valid prism_dtype object; the calls accept PRISM_F32 and PRISM_BF16
 * and reject everything else with PRISM_ERR_DTYPE. */
typedef enum {
  PRISM_F32 = 0,
  PRISM_BF16 = 1,
  PRISM_DTYPE_NONE = -1,
  PRISM_DTYPE_LAST = 0x7fffffff
} prism_dtype;

/* Flags of prism_zone_stats_ex. */
enum { PRISM_STATS_GLOBAL_VARIANCE = 1, PRISM_STATS_FROM_NORM = 2 };

/* Video latent grid (T, H, W) and macro-zone extents (zt, zh, zw).  Zones tile the grid
 * from the origin in t-major raster order; the grid is padded at its far edges up to a
 * multiple of the zone (abstract: spatiotemporal macro-zones). */
typedef struct {
  int32_t T, H, W;
  int32_t zt, zh, zw;
} prism_grid;

#define PRISM_MAX_SHAPES 32

/* Candidate block shapes (b_T, b_H, b_W), all holding `vol` tokens (Table 11 caption:
 * shapes b_T b_H b_W; one candidate set holds a single volume).  A candidate can be
 * assigned to a zone only if each extent divides the zone's extent.  List order is the
 * tie-break order. */
typedef struct {
  int32_t n, vol;
  int32_t bt[PRISM_MAX_SHAPES], bh[PRISM_MAX_SHAPES], bw[PRISM_MAX_SHAPES];
} prism_shapes;

/* Shape rule constants: power-law exponent alpha of b*_d ~ g_d^-alpha (Table 10 caption),
 * gate thresholds tau_lo/tau_hi on m_z / m-bar, guidance floor g_min, ratio guard eps.
 * The documented defaults are 0.5, 1, 2, 1e-3, 1e-12. */
typedef struct {
  float alpha, tau_lo, tau_hi, g_min, eps;
} prism_shape_params;

/* Hybrid selection (Table 7 caption): the Top-p count is the smallest number of key
 * blocks whose cumulative pooled attention weight strictly exceeds top_p, then clamped
 * to [k_min, k_max] and to the number of live key blocks.  0 < top_p <= 1,
 * 1 <= k_min <= k_max.  top_p = 1 keeps every live block before the clamp (the weights
 * sum to 1, so no proper prefix exceeds it, whatever the float32 rounding of the sum). */
typedef struct {
  float top_p;
  int32_t k_min, k_max;
} prism_select_params;

/* Number of zones and of blocks (nb = zones * zt*zh*zw / vol) for a grid and candidate
 * set.  Host-only helpers; return -1 on invalid arguments. */
int64_t prism_num_zones(const prism_grid* grid);
int64_t prism_num_blocks(const prism_grid* grid, const prism_shapes* shapes);

/* Zone statistics (abstract; Table 9 caption).
 * v, a2v   [B][Hh][N][d] value features and A2V cross-attention output, N = T*H*W.
 *          Any feature tensor may stand in for v (Table 9 caption: query or key features).
 * stats    out float [B][Hh][nZ][8]: r_v[t,h,w] (per-channel directional share of the
 *          lag-one semivariance of v, averaged over channels), gamma_a[t,h,w] (lag-one
 *          semivariance of the per-token norm ||a2v||), m_z (mean norm), n_z (valid
 *          tokens).  Neighbour pairs never cross a zone border or the grid edge.
 * Requires d in {32, 64, 128, 256} and zt*zh*zw <= 4096; PRISM_ERR_DTYPE / PRISM_ERR_SHAPE
 * otherwise. */
prism_status prism_zone_stats(const void* v, const void* a2v, prism_dtype dtype, int B, int Hh,
                              int d, const prism_grid* grid, float* stats, hipStream_t stream);

/* The "global variance" variant of the zone statistics (Table 9 caption: the feature
 * variance taken across all channels jointly instead of per channel): r_v[t,h,w] is the
 * share of each axis in the channel-mean lag-one semivariance, gamma_bar_d /
 * (sum_d gamma_bar_d + eps).  Everything else, arguments and errors included, as
 * prism_zone_stats. */
prism_status prism_zone_stats_global(const void* v, const void* a2v, prism_dtype dtype, int B, int Hh,
                                     int d, const prism_grid* grid, float* stats, hipStream_t stream);

/* Audio-to-video cross-attention emitting the per-token norm that guides the shapes
 * (abstract: feature norms of the A2V cross-attention output), so that the statistics
 * need not read the A2V output back.
 * q        [B][Hh][N][d]  video queries;  ka, va [B][Hh][Na][d] audio keys and values.
 * o        optional out [B][Hh][N][d]: softmax(q ka^T * scale) va (NULL: not written).
 * a2v_norm out float [B][Hh][N]: the L2 norm of each output row, from the fp32 output.
 * Dense over all Na keys (no selection).  Requires bf16 and d = 128 (PRISM_ERR_DTYPE). */
prism_status prism_a2v_attn_norm(const void* q, const void* ka, const void* va, prism_dtype dtype, int B,
                                 int Hh, int N, int Na, int d, float scale, void* o, float* a2v_norm,
                                 hipStream_t stream);

/* Zone statistics from the per-token A2V norm map (float [B][Hh][N], e.g. from
 * prism_a2v_attn_norm) instead of the A2V output rows; global_variance != 0 selects the
 * all-channel variant of prism_zone_stats_global.  Arguments, output and errors otherwise
 * as prism_zone_stats. */
prism_status prism_zone_stats_from_norm(const void* v, const float* a2v_norm, prism_dtype dtype, int B,
                                        int Hh, int d, const prism_grid* grid, int global_variance,
                                        float* stats, hipStream_t stream);

/* The zone statistics with every option: flags PRISM_STATS_GLOBAL_VARIANCE (as
 * prism_zone_stats_global) and PRISM_STATS_FROM_NORM (aux is the norm map float
 * [B][Hh][N], as prism_zone_stats_from_norm; otherwise the A2V output rows).
 * vact     optional out float [B][Hh][nZ]: the zone's video activity, the channel-mean
 *          lag-one semivariance of v summed over t, h and w (the magnitude the shares
 *          normalise away; input of prism_assign_shapes_multi).
 * Unknown flags: PRISM_ERR_ARG.  Arguments, output and errors otherwise as prism_zone_stats. */
prism_status prism_zone_stats_ex(const void* v, const void* aux, prism_dtype dtype, int B, int Hh, int d,
                                 const prism_grid* grid, int flags, float* stats, float* vact, hipStream_t stream);

/* Shape assignment (abstract: finer blocks along fast-varying, audio-coupled axes;
 * Table 10 caption: b*_d ~ g_d^-alpha and its quantization).
 * stats    float [B][Hh][nZ][8] from prism_zone_stats.
 * shape_id out int32 [B][Hh][nZ]: index into shapes of the feasible candidate nearest, in
 *          log2 extents, to lambda_d = log2(vol)/3 - alpha (log2 g_d - mean_d log2 g_d),
 *          where g_d = max((1 - a) r_v,d + a v-hat_a,d, g_min), a = clamp((m_z/m-bar -
 *          tau_lo)/(tau_hi - tau_lo), 0, 1), v-hat_a = gamma_a / (sum gamma_a + eps).
 * margin   optional out float [B][Hh][nZ]: (D_2 - D_1)/D_2 between best and runner-up. */
prism_status prism_assign_shapes(const float* stats, int B, int Hh, const prism_grid* grid,
                                 const prism_shapes* shapes, const prism_shape_params* params,
                                 int32_t* shape_id, float* margin, hipStream_t stream);

/* Shapes from a candidate table that mixes volumes: unit = shapes->vol (64), candidates
 * of 1, 2 or 4 units (the C_64 / C_128 / C_256 sets of Tables 9 and 11; Table 10 caption:
 * thresholds tau_128 / tau_256 of the assignment).  Per zone, activity = vact_z / (mean of
 * vact over the head's zones) + the audio gate; the block volume is 4 units if activity <
 * tau_256, 2 units if < tau_128, else 1 unit (a smaller one when no shape of the chosen
 * volume tiles the zone), and the shape is the Eq. 7 choice among that volume's
 * candidates, as in prism_assign_shapes.
 * vact     float [B][Hh][nZ] from prism_zone_stats_ex.
 * margin   optional out: the smaller of the shape margin and |activity - tau| / tau.
 * Errors: a candidate not of 1, 2 or 4 units or no unit-volume shape tiling the zone ->
 * PRISM_ERR_SHAPE; not 0 < tau_256 <= tau_128 -> PRISM_ERR_ARG. */
prism_status prism_assign_shapes_multi(const float* stats, const float* vact, int B, int Hh, const prism_grid* grid,
                                       const prism_shapes* shapes, const prism_shape_params* params, float tau_128,
                                       float tau_256, int32_t* shape_id, float* margin, hipStream_t stream);

/* Block-level valid counts for a mixed-volume assignment: each block is identified by
 * its first unit (shapes->vol slots), which receives the whole block's valid count; its
 * other units receive 0.
 * unit_valid  int32 [B][Hh][nb] per-unit counts from prism_permute(..., block_valid) with the
 *             same mixed table (nb = zones * zone volume / unit).
 * block_valid out int32 [B][Hh][nb]: the input of prism_select_blocks with vol = unit (a
 *             block's valid rows are contiguous from its first unit). */
prism_status prism_block_heads(const int32_t* unit_valid, const int32_t* shape_id, int B, int Hh,
                               const prism_grid* grid, const prism_shapes* shapes, int32_t* block_valid,
                               hipStream_t stream);

/* Token permutation into blocks (abstract: each block's tokens are contiguous).
 * Slot order: zones in raster order; a zone's blocks in raster order over its block grid;
 * inside a block, the tokens lying in the real grid first (raster order), then padding.
 * inverse == 0: x [B][Hh][N][d] -> y [B][Hh][Npad][d], zeros at padding slots.
 * inverse == 1: x [B][Hh][Npad][d] -> y [B][Hh][N][d], padding slots dropped.
 * block_valid optional out int32 [B][Hh][nb]: valid slots per block (0 = dead block).
 * shape_id  int32 [B][Hh][nZ] device array, each entry the index of a candidate that tiles
 *           the zone (as prism_assign_shapes writes).  This is not checked on the host; a
 *           zone whose id is out of range or names a candidate that does not tile it maps no
 *           token: its slots are written as padding (forward), its tokens are left as they
 *           were (inverse), and its blocks get block_valid 0.
 * Requires d * sizeof(dtype) % 16 == 0. */
prism_status prism_permute(const void* x, void* y, prism_dtype dtype, int B, int Hh, int d,
                           const prism_grid* grid, const prism_shapes* shapes,
                           const int32_t* shape_id, int inverse, int32_t* block_valid,
                           hipStream_t stream);

/* Forward permutation fused with the block pooling of the selection (abstract:
 * block-level features): prism_permute(..., inverse = 0, block_valid) that also writes
 * pooled  out float [B][Hh][nb][d]: the mean of each block's valid rows, summed in float32
 *         (0 for a dead block),
 * the input of prism_select_blocks_pooled.  Every candidate must hold shapes->vol tokens
 * (PRISM_ERR_SHAPE otherwise) and d * sizeof(dtype) must be 16 bytes times a power of two
 * up to 4096 bytes (PRISM_ERR_DTYPE).  block_valid may be NULL. */
prism_status prism_permute_pool(const void* x, void* y, prism_dtype dtype, int B, int Hh, int d,
                                const prism_grid* grid, const prism_shapes* shapes, const int32_t* shape_id,
                                int32_t* block_valid, float* pooled, hipStream_t stream);

/* (a4, a5) Block pooling and hybrid Top-k/Top-p selection (abstract; Figure 2 caption;
 * Table 7 caption).
 * qp, kp       [B][Hh][nb*vol][d] permuted Q and K.
 * block_valid  int32 [B][Hh][nb].  nb <= 32768 (a row of block scores is held in the
 *              registers of one workgroup), else PRISM_ERR_SHAPE.
 * Pooled means (float32) of each block's valid rows give scores scale * <Qbar_I, Kbar_J>
 * over live key blocks; softmax, then the hybrid count on the descending order (ties to
 * the lower block index).  Dead query blocks select nothing.
 * sel_idx  out int32 [B][Hh][nb][k_max], ascending, -1 padded;  sel_cnt out [B][Hh][nb].
 * rev_ptr  out int32 [B][Hh][nb+1] and rev_idx out int32 [B][Hh][nb*k_max]: for each key
 *          block, the query blocks that selected it, ascending (-1 padded).
 * sel_margin optional out float [B][Hh][nb]: smallest relative distance of the row's
 *          decision from flipping (gap at the cut, distance of the cumulative sum to p).
 * workspace    device scratch of prism_select_workspace_size() bytes: the pooled means,
 *          the float32 scores of one chunk of query blocks at a time (as many per head as
 *          fit 256 MB, at least 512), that chunk's selection bits and two ints per key
 *          block; linear in nb (no nb x nb matrix is formed). */
size_t prism_select_workspace_size(int B, int Hh, int nb, int d);
prism_status prism_select_blocks(const void* qp, const void* kp, prism_dtype dtype,
                                 const int32_t* block_valid, int B, int Hh, int nb, int vol, int d,
                                 float scale, const prism_select_params* params, int32_t* sel_idx,
                                 int32_t* sel_cnt, int32_t* rev_ptr, int32_t* rev_idx,
                                 float* sel_margin, void* workspace, size_t ws_bytes,
                                 hipStream_t stream);

/* prism_select_blocks from pooled means given by the caller (prism_permute_pool of Q and
 * K): qbar, kbar float [B][Hh][nb][d], d a multiple of 16 up to 4096.  Outputs, parameters
 * and errors as prism_select_blocks; workspace: prism_select_pooled_workspace_size() bytes
 * (the pooled means are not part of it). */
size_t prism_select_pooled_workspace_size(int B, int Hh, int nb);
prism_status prism_select_blocks_pooled(const float* qbar, const float* kbar, const int32_t* block_valid, int B,
                                        int Hh, int nb, int d, float scale, const prism_select_params* params,
                                        int32_t* sel_idx, int32_t* sel_cnt, int32_t* rev_ptr, int32_t* rev_idx,
                                        float* sel_margin, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Blocks of 128 or 256 tokens (the C_128 / C_256 candidate sets, Tables 9 and 11) run
 * through the attention as runs of vol/64 consecutive 64-row tiles.  This call expands a
 * block-level selection (from prism_select_blocks with that vol) and its reverse index to
 * tile level, for prism_sparse_attn_fwd / _bwd called with vol = 64, nb_t = nb*vol/64
 * tiles and k_max_t = k_max*vol/64:
 *   tile_valid   out int32 [B][Hh][nb_t]: valid rows of each tile (a block's valid rows
 *                come first, so its live tiles are the first ceil(n/64));
 *   tile_idx     out int32 [B][Hh][nb_t][k_max_t], ascending, -1 padded; tile_cnt [B][Hh][nb_t]:
 *                query tile (I,u) lists every live tile of every block I selected
 *                (nothing for a tile with no valid row);
 *   tile_rev_ptr out int32 [B][Hh][nb_t+1], tile_rev_idx out [B][Hh][nb_t*k_max_t]: the
 *                transpose of tile_idx, ascending per key tile.
 * vol must be a multiple of 64 in [64, 4096] (PRISM_ERR_SHAPE); workspace:
 * prism_tiles_workspace_size() bytes of device scratch. */
size_t prism_tiles_workspace_size(int B, int Hh, int nb, int vol);
prism_status prism_blocks_to_tiles(const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                   const int32_t* rev_ptr, const int32_t* rev_idx, int B, int Hh, int nb, int vol,
                                   int k_max, int32_t* tile_valid, int32_t* tile_idx, int32_t* tile_cnt,
                                   int32_t* tile_rev_ptr, int32_t* tile_rev_idx, void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* prism_blocks_to_tiles for a mixed-volume assignment, where blocks are identified by
 * their first 64-row unit (prism_block_heads) and own the following live units: tile
 * numbering is the unit numbering (nb tiles), tile_valid is the per-unit count from
 * prism_permute, and lists hold up to k_max * max_units tiles (max_units = the largest
 * block volume / 64).  Output layouts otherwise as prism_blocks_to_tiles; workspace:
 * prism_tiles_mixed_workspace_size() bytes. */
size_t prism_tiles_mixed_workspace_size(int B, int Hh, int nb);
prism_status prism_blocks_to_tiles_mixed(const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                         const int32_t* rev_ptr, const int32_t* rev_idx, int B, int Hh, int nb,
                                         int k_max, int max_units, int32_t* tile_idx, int32_t* tile_cnt,
                                         int32_t* tile_rev_ptr, int32_t* tile_rev_idx, void* workspace,
                                         size_t ws_bytes, hipStream_t stream);

/* Preconditions on the device lists of the attention calls (as prism_select_blocks and
 * prism_blocks_to_tiles write them; they are device data and are not read on the host):
 *   block_valid[I] in [0, vol];
 *   sel_cnt[I] in [0, k_max]; sel_idx[I][0:sel_cnt[I]] distinct block indices in [0, nb),
 *     ascending;
 *   rev_ptr[0] = 0, rev_ptr non-decreasing, rev_ptr[nb] <= nb * k_max; rev_idx[rev_ptr[J] :
 *     rev_ptr[J+1]] distinct query blocks in [0, nb), ascending, and exactly the query
 *     blocks whose sel_idx row holds J.
 * The kernels clamp every count, pointer and index into its range before using it, so a
 * malformed list cannot make them read or write outside the caller's buffers; the results
 * are then unspecified.  Ascending order is what the kernels' workgroup schedule and cache
 * reuse assume; any order gives the same results up to float32 summation order. */

/* Block-sparse attention forward (Figure 2 caption).  Query row i of block I attends
 * to every valid row of every block in sel_idx[I][0:sel_cnt[I]]:
 *   O_i = softmax_j(scale q_i.k_j) v_j,  lse_i = ln sum_j exp(scale q_i.k_j).
 * op   out [B][Hh][nb*vol][d] (zeros at padding rows);  lse out float [B][Hh][nb*vol]
 * (0 at padding rows).  Requires vol <= 64 and d in {64, 128}; bf16 with vol = 64 and
 * d = 128 runs on the matrix cores, with the P V product in fp16: P (below 2^8) rounded
 * to fp16 against a copy of V scaled per head by a power of two that keeps every bf16
 * value exact in fp16 (those more than 2^29 below the head's largest |V| excepted, whose
 * contribution is below the output's own rounding).  workspace:
 * prism_fwd_workspace_size() bytes of device scratch: on the matrix-core path B*Hh*nb
 * int32 (rounded up to 256 bytes), the order in which workgroups take their query blocks
 * (longest list first, changes no output), then two per-head words and the fp16 copy of
 * V (2 bytes per element of vp); 0 bytes otherwise, and workspace may then be NULL.
 * Too small: PRISM_ERR_ARG. */
size_t prism_fwd_workspace_size(int B, int Hh, int nb, int vol, int d, prism_dtype dtype);
prism_status prism_sparse_attn_fwd(const void* qp, const void* kp, const void* vp, prism_dtype dtype,
                                   const int32_t* block_valid, const int32_t* sel_idx,
                                   const int32_t* sel_cnt, int k_max, int B, int Hh, int nb, int vol,
                                   int d, float scale, void* op, float* lse, void* workspace,
                                   size_t ws_bytes, hipStream_t stream);

/* Block-sparse attention backward, selection held fixed.
 * With D_i = dO_i.O_i, P_ij = exp(scale q_i.k_j - lse_i), dS_ij = P_ij (dO_i.v_j - D_i):
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
 * dqp, dkp, dvp out [B][Hh][nb*vol][d] (zeros at padding rows).  dK/dV walk the reverse
 * index; no atomics, results are deterministic.
 * marks    optional array of 4 caller-created hipEvents recorded on `stream` before the
 *          D kernel (and the schedule kernel), after it, after the dK/dV kernel and after
 *          the dQ kernel.
 * workspace    device scratch of prism_bwd_workspace_size() bytes: D = rowsum(dO*O) per row,
 *          and on the matrix-core path the orders in which the dQ and dK/dV workgroups take
 *          their blocks (longest list first; they change no output). */
size_t prism_bwd_workspace_size(int B, int Hh, int nb, int vol, int d, prism_dtype dtype);
prism_status prism_sparse_attn_bwd(const void* qp, const void* kp, const void* vp, const void* op,
                                   const void* dop, const float* lse, prism_dtype dtype,
                                   const int32_t* block_valid, const int32_t* sel_idx,
                                   const int32_t* sel_cnt, int k_max, const int32_t* rev_ptr,
                                   const int32_t* rev_idx, int B, int Hh, int nb, int vol, int d,
                                   float scale, void* dqp, void* dkp, void* dvp, void* workspace,
                                   size_t ws_bytes, hipEvent_t* marks, hipStream_t stream);

/* prism_sparse_attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no workspace
 * argument, and no allocation in the call.  Its scratch (D and the two workgroup
 * schedules, prism_bwd_workspace_size() bytes) is a static device array of 32 MiB per
 * GPU, held until the process ends; a call that needs more returns PRISM_ERR_SHAPE
 * (about 8 million padded rows B*Hh*nb*vol).  The stream must belong to the current
 * device (PRISM_ERR_ARG otherwise).  Every call on one GPU uses that GPU's one array:
 * calls that overlap on a GPU (other streams, other host threads) race and must be
 * ordered by the caller.  Nothing in the scratch needs to start at zero: every entry is
 * written before it is read.  Arguments, outputs and other errors as
 * prism_sparse_attn_bwd. */
prism_status prism_sparse_attn_bwd_noalloc(const void* qp, const void* kp, const void* vp, const void* op,
                                           const void* dop, const float* lse, prism_dtype dtype,
                                           const int32_t* block_valid, const int32_t* sel_idx,
                                           const int32_t* sel_cnt, int k_max, const int32_t* rev_ptr,
                                           const int32_t* rev_idx, int B, int Hh, int nb, int vol, int d,
                                           float scale, void* dqp, void* dkp, void* dvp, hipEvent_t* marks,
                                           hipStream_t stream);

/* Dense attention comparator on unpermuted [B][Hh][N][d] tensors (every key attended),
 * the same kernels run with every block selected; used to measure the sparse path's
 * speedup.  lse float [B][Hh][N].  Requires d in {64, 128}.  The forward's workspace holds
 * the fp16 copy of V as for prism_sparse_attn_fwd (no schedule). */
size_t prism_dense_fwd_workspace_size(int B, int Hh, int N, int d, prism_dtype dtype);
prism_status prism_dense_attn_fwd(const void* q, const void* k, const void* v, prism_dtype dtype,
                                  int B, int Hh, int N, int d, float scale, void* o, float* lse,
                                  void* workspace, size_t ws_bytes, hipStream_t stream);
size_t prism_dense_bwd_workspace_size(int B, int Hh, int N, int d, prism_dtype dtype);
prism_status prism_dense_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                  const void* dout, const float* lse, prism_dtype dtype, int B,
                                  int Hh, int N, int d, float scale, void* dq, void* dk, void* dv,
                                  void* workspace, size_t ws_bytes, hipEvent_t* marks,
                                  hipStream_t stream);

/* Measurement kernels.  They are not steps of the method: they give the ceilings that the
 * attention and statistics kernels are compared with on the GPU at hand.
 *
 * prism_bench_mfma_peak: `workgroups` workgroups of 4 wavefronts, each wave issuing
 * `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 products (32768 flops
 * each), so the run does workgroups * 4 * iters * 4 * 32768 flops.  clocks (device,
 * uint64 [workgroups][2]) receives per workgroup the shader-clock cycles and the 100 MHz
 * reference ticks over its loop; sink (device, float [workgroups]) is never written in
 * practice and keeps the products from being removed.  Errors: null pointers,
 * workgroups outside [1, 2^20] or iters < 1 -> PRISM_ERR_ARG. */
prism_status prism_bench_mfma_peak(int workgroups, int iters, uint64_t* clocks, float* sink, hipStream_t stream);

/* prism_bench_tile_gather: the launch of prism_sparse_attn_fwd (workgroup schedule, grid,
 * LDS stages, the same copies of every listed K and V tile into LDS) with no arithmetic;
 * each query block's valid Q rows are copied to op.  Arguments as prism_sparse_attn_fwd
 * (no scale, no lse); bf16, d = 128 and vol = 64 only (PRISM_ERR_DTYPE otherwise);
 * workspace: prism_fwd_workspace_size() bytes.  Its time is the forward's memory traffic
 * alone with this launch. */
prism_status prism_bench_tile_gather(const void* qp, const void* kp, const void* vp, prism_dtype dtype,
                                     const int32_t* block_valid, const int32_t* sel_idx, const int32_t* sel_cnt,
                                     int k_max, int B, int Hh, int nb, int vol, int d, void* op, void* workspace,
                                     size_t ws_bytes, hipStream_t stream);

/* prism_bench_stream_read: reads `bytes` bytes of device buffer a and of device buffer b
 * front to back (2048 workgroups of 256 threads, grid-stride, 16-byte loads, two per
 * buffer in flight per thread): a plain contiguous read of 2 * bytes, the ceiling that a
 * memory-bound stage reading as many bytes (zone statistics: V and the A2V output) is
 * measured against.  sink (device, uint32 [PRISM_BENCH_STREAM_SINK]) receives a checksum
 * per wavefront, so the loads cannot be removed.  Errors: null pointers, bytes zero or not
 * a multiple of 16 -> PRISM_ERR_ARG. */
#define PRISM_BENCH_STREAM_SINK 8192
prism_status prism_bench_stream_read(const void* a, const void* b, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char* prism_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H */
