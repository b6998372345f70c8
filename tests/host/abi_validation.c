/* Host-side argument validation of libprism under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every call below has one bad argument (or sizes that
 * overflow the checks) and must return its error status before launching anything.  The
 * fake device pointers are never dereferenced.  Prints one line per case and exits
 * non-zero on the first unexpected status. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "prism.h"

static int failures = 0;

static void expect(const char* what, prism_status got, prism_status want) {
  const char* msg = prism_last_error();
  printf("%-52s status %d (want %d)  %s\n", what, (int)got, (int)want, msg);
  if (got != want || (want != PRISM_OK && (!msg || !msg[0]))) ++failures;
}

int main(void) {
  void* P = (void*)(uintptr_t)256;
  int32_t* I = (int32_t*)P;
  float* F = (float*)P;
  prism_grid g = {4, 8, 8, 2, 4, 8};
  prism_grid g_big = {1 << 12, 1 << 12, 1 << 12, 4, 16, 16};
  prism_grid g_zone = {4, 8, 8, 64, 64, 64};
  prism_grid g_neg = {4, -8, 8, 2, 4, 8};
  prism_shapes s;
  memset(&s, 0, sizeof s);
  s.n = 4; s.vol = 16;
  int bt[4] = {1, 2, 2, 4}, bh[4] = {4, 2, 4, 2}, bw[4] = {4, 4, 2, 2};
  for (int i = 0; i < 4; ++i) { s.bt[i] = bt[i]; s.bh[i] = bh[i]; s.bw[i] = bw[i]; }
  prism_shapes s_many = s;
  s_many.n = PRISM_MAX_SHAPES + 1;
  prism_shapes s_zero = s;
  s_zero.bt[1] = 0;
  prism_shape_params sp = {0.5f, 1.f, 2.f, 1e-3f, 1e-12f};
  prism_select_params sel = {0.9f, 2, 8};
  prism_select_params sel_bad = {0.f, 2, 8};

  expect("num_zones(null)", (prism_status)(prism_num_zones(NULL) == -1 ? 1 : 0), 1);
  expect("num_zones(negative extent)", (prism_status)(prism_num_zones(&g_neg) == -1 ? 1 : 0), 1);
  expect("num_blocks(33 shapes)", (prism_status)(prism_num_blocks(&g, &s_many) == -1 ? 1 : 0), 1);
  expect("zone_stats(grid too large)", prism_zone_stats(P, P, PRISM_BF16, 1, 1, 128, &g_big, F, 0), PRISM_ERR_SHAPE);
  expect("zone_stats(zone too large)", prism_zone_stats(P, P, PRISM_BF16, 1, 1, 128, &g_zone, F, 0), PRISM_ERR_SHAPE);
  expect("zone_stats(B = -1)", prism_zone_stats(P, P, PRISM_BF16, -1, 1, 128, &g, F, 0), PRISM_ERR_ARG);
  expect("zone_stats_ex(unknown flag)", prism_zone_stats_ex(P, P, PRISM_BF16, 1, 1, 128, &g, 64, F, NULL, 0),
         PRISM_ERR_ARG);
  expect("assign_shapes(zero extent)", prism_assign_shapes(F, 1, 1, &g, &s_zero, &sp, I, NULL, 0), PRISM_ERR_ARG);
  expect("assign_shapes(null params)", prism_assign_shapes(F, 1, 1, &g, &s, NULL, I, NULL, 0), PRISM_ERR_ARG);
  expect("permute(inverse = 7)", prism_permute(P, (char*)P + 64, PRISM_F32, 1, 1, 64, &g, &s, I, 7, NULL, 0),
         PRISM_ERR_ARG);
  expect("permute(dtype 9)", prism_permute(P, (char*)P + 64, (prism_dtype)9, 1, 1, 64, &g, &s, I, 0, NULL, 0),
         PRISM_ERR_DTYPE);
  expect("permute_pool(d = 3 bf16)", prism_permute_pool(P, (char*)P + 64, PRISM_BF16, 1, 1, 3, &g, &s, I, NULL, F, 0),
         PRISM_ERR_DTYPE);
  expect("select(nb = 2^31 - 1)", prism_select_blocks(P, P, PRISM_BF16, I, 1, 1, 0x7fffffff, 64, 128, 0.1f, &sel,
                                                     I, I, I, I, NULL, P, (size_t)-1, 0), PRISM_ERR_SHAPE);
  expect("select(top_p = 0)", prism_select_blocks(P, P, PRISM_BF16, I, 1, 1, 16, 64, 128, 0.1f, &sel_bad, I, I, I, I,
                                                  NULL, P, (size_t)1 << 30, 0), PRISM_ERR_ARG);
  expect("select_pooled(ws 0)", prism_select_blocks_pooled(F, F, I, 1, 1, 16, 128, 0.1f, &sel, I, I, I, I, NULL, P,
                                                           0, 0), PRISM_ERR_ARG);
  expect("select_ws_size(negative)", (prism_status)(prism_select_workspace_size(1, -1, 16, 128) == 0 ? 1 : 0), 1);
  expect("fwd(rows overflow)", prism_sparse_attn_fwd(P, P, P, PRISM_BF16, I, I, I, 8, 1 << 14, 1 << 14, 1 << 10, 64,
                                                     128, 0.1f, P, F, P, (size_t)-1, 0), PRISM_ERR_SHAPE);
  expect("fwd(k_max = 0)", prism_sparse_attn_fwd(P, P, P, PRISM_BF16, I, I, I, 0, 1, 1, 16, 64, 128, 0.1f, P, F, P,
                                                 (size_t)-1, 0), PRISM_ERR_ARG);
  expect("fwd(scale NaN)", prism_sparse_attn_fwd(P, P, P, PRISM_BF16, I, I, I, 8, 1, 1, 16, 64, 128, 0.f / 0.f, P, F,
                                                 P, (size_t)-1, 0), PRISM_ERR_ARG);
  expect("fwd(workspace 1 byte)", prism_sparse_attn_fwd(P, P, P, PRISM_BF16, I, I, I, 8, 1, 1, 16, 64, 128, 0.1f, P,
                                                        F, P, 1, 0), PRISM_ERR_ARG);
  expect("bwd(vol 65)", prism_sparse_attn_bwd(P, P, P, P, P, F, PRISM_BF16, I, I, I, 8, I, I, 1, 1, 16, 65, 128, 0.1f,
                                              P, P, P, P, (size_t)-1, NULL, 0), PRISM_ERR_SHAPE);
  expect("bwd_noalloc(past the scratch)",
         prism_sparse_attn_bwd_noalloc(P, P, P, P, P, F, PRISM_BF16, I, I, I, 8, I, I, 64, 64, 1024, 64, 128, 0.1f, P,
                                       P, P, NULL, 0), PRISM_ERR_SHAPE);
  expect("dense_fwd(N = 0)", prism_dense_attn_fwd(P, P, P, PRISM_BF16, 1, 1, 0, 128, 0.1f, P, F, P, (size_t)-1, 0),
         PRISM_ERR_ARG);
  expect("a2v_norm(Na overflow)", prism_a2v_attn_norm(P, P, P, PRISM_BF16, 1 << 16, 1 << 16, 64, 1 << 16, 128, 0.1f,
                                                      NULL, F, 0), PRISM_ERR_SHAPE);
  expect("blocks_to_tiles(lists overflow)",
         prism_blocks_to_tiles(I, I, I, I, I, 64, 64, 1 << 12, 256, 1 << 12, I, I, I, I, I, P, (size_t)-1, 0),
         PRISM_ERR_SHAPE);
  expect("tiles_mixed(max_units 65)",
         prism_blocks_to_tiles_mixed(I, I, I, I, I, 1, 1, 16, 8, 65, I, I, I, I, P, (size_t)-1, 0), PRISM_ERR_ARG);
  /* B*Hh heads times the per-head units past 2^31 - 1: an error (calls) or 0 (sizes), with
     no int product of B and Hh formed on the way */
  expect("zone_stats(B*Hh*zones overflow)", prism_zone_stats(P, P, PRISM_BF16, 1 << 16, 1 << 15, 128, &g, F, 0),
         PRISM_ERR_SHAPE);
  expect("assign_shapes(B*Hh overflow)", prism_assign_shapes(F, 0x7fffffff, 0x7fffffff, &g, &s, &sp, I, NULL, 0),
         PRISM_ERR_SHAPE);
  expect("permute(B*Hh*blocks overflow)",
         prism_permute(P, (char*)P + 64, PRISM_F32, 1 << 16, 1 << 14, 64, &g, &s, I, 0, NULL, 0), PRISM_ERR_SHAPE);
  expect("select_pooled(B*Hh*nb overflow)",
         prism_select_blocks_pooled(F, F, I, 1 << 16, 1 << 8, 1 << 8, 128, 0.1f, &sel, I, I, I, I, NULL, P,
                                    (size_t)-1, 0), PRISM_ERR_SHAPE);
  expect("fwd(B*Hh*rows = 2^31)", prism_sparse_attn_fwd(P, P, P, PRISM_BF16, I, I, I, 8, 1 << 15, 1 << 16, 1, 1,
                                                        128, 0.1f, P, F, P, (size_t)-1, 0), PRISM_ERR_SHAPE);
  expect("select_ws_size(B*Hh overflow)",
         (prism_status)(prism_select_workspace_size(0x7fffffff, 0x7fffffff, 16, 128) == 0 ? 1 : 0), 1);
  expect("select_pooled_ws_size(B*Hh*nb overflow)",
         (prism_status)(prism_select_pooled_workspace_size(1 << 16, 1 << 16, 16) == 0 ? 1 : 0), 1);
  expect("bwd_ws_size(nb*vol overflow)",
         (prism_status)(prism_bwd_workspace_size(1, 1, 1 << 26, 64, 128, PRISM_BF16) == 0 ? 1 : 0), 1);
  expect("fwd_ws_size(B*Hh overflow)",
         (prism_status)(prism_fwd_workspace_size(0x7fffffff, 2, 16, 64, 128, PRISM_BF16) == 0 ? 1 : 0), 1);
  expect("dense_bwd_ws_size(B*Hh*N overflow)",
         (prism_status)(prism_dense_bwd_workspace_size(1 << 16, 1 << 16, 64, 128, PRISM_BF16) == 0 ? 1 : 0), 1);
  expect("tiles_ws_size(B*Hh overflow)",
         (prism_status)(prism_tiles_workspace_size(0x7fffffff, 0x7fffffff, 16, 128) == 0 ? 1 : 0), 1);
  expect("tiles_mixed_ws_size(B*Hh overflow)",
         (prism_status)(prism_tiles_mixed_workspace_size(0x7fffffff, 0x7fffffff, 16) == 0 ? 1 : 0), 1);
  expect("bench_mfma(workgroups 0)", prism_bench_mfma_peak(0, 1, (uint64_t*)P, F, 0), PRISM_ERR_ARG);
  expect("bench_stream(bytes not a multiple of 16)", prism_bench_stream_read(P, P, 1000, (uint32_t*)P, 0), PRISM_ERR_ARG);
  expect("bench_stream(null sink)", prism_bench_stream_read(P, P, 1 << 20, NULL, 0), PRISM_ERR_ARG);
  printf("%d unexpected statuses\n", failures);
  return failures ? 1 : 0;
}
