/* A plain C11 consumer of include/veda.h, built with gcc by
 * tests/test_c_abi.py. It prints the ABI's struct layout as C lays it out,
 * then runs the host-only sizing calls on a layer read from stdin and prints
 * what they fill in, as "key=value" lines.
 *
 * stdin: "seq_len N", "span START T H W t h w" (packed order, target last,
 * box 0 0 0 for least padding), "budget GEN_RATIO GEN_TILES REF_RATIO
 * REF_TILES", "head N_HEADS HEAD_DIM". */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "veda.h"

#define FIELD(T, f) printf("offset.%s.%s=%zu\n", #T, #f, offsetof(T, f))

static void layout(void) {
  printf("sizeof.veda_span=%zu\n", sizeof(veda_span));
  FIELD(veda_span, start);
  FIELD(veda_span, grid);
  FIELD(veda_span, shape);
  printf("sizeof.veda_budget=%zu\n", sizeof(veda_budget));
  printf("sizeof.veda_plan_info=%zu\n", sizeof(veda_plan_info));
  FIELD(veda_plan_info, n_slots);
  FIELD(veda_plan_info, global_rows);
  FIELD(veda_plan_info, n_tiles);
  FIELD(veda_plan_info, n_spans);
  FIELD(veda_plan_info, spans);
  FIELD(veda_plan_info, span_tile0);
  printf("sizeof.veda_block=%zu\n", sizeof(veda_block));
  FIELD(veda_block, k_hi);
  FIELD(veda_block, frac);
  printf("sizeof.veda_select_info=%zu\n", sizeof(veda_select_info));
  FIELD(veda_select_info, widest);
  FIELD(veda_select_info, entries_per_head);
  FIELD(veda_select_info, workspace_bytes);
  FIELD(veda_select_info, blocks);
}

int main(void) {
  veda_span spans[VEDA_MAX_SPANS + 1];
  int n_spans = 0;
  long long seq_len = 0;
  veda_budget gen = {-1.0, -1.0}, ref = {-1.0, -1.0};
  int n_heads = 1, head_dim = 128;
  char line[256];

  printf("version=%s\n", veda_version());
  layout();
  while (fgets(line, sizeof line, stdin)) {
    veda_span s;
    memset(&s, 0, sizeof s);
    if (sscanf(line, "seq_len %lld", &seq_len) == 1) continue;
    if (sscanf(line, "span %lld %d %d %d %d %d %d", (long long *)&s.start, &s.grid[0], &s.grid[1],
               &s.grid[2], &s.shape[0], &s.shape[1], &s.shape[2]) == 7) {
      if (n_spans <= VEDA_MAX_SPANS) spans[n_spans++] = s;
      continue;
    }
    if (sscanf(line, "budget %lf %lf %lf %lf", &gen.ratio, &gen.tiles, &ref.ratio, &ref.tiles) == 4)
      continue;
    sscanf(line, "head %d %d", &n_heads, &head_dim);
  }

  veda_plan_info info;
  veda_status st = veda_plan_query(spans, n_spans, seq_len, &info);
  printf("plan_status=%d\n", (int)st);
  if (st != VEDA_OK) {
    printf("plan_error=%s\n", veda_last_error());
    return 0;
  }
  printf("n_slots=%lld\nn_tiles=%d\nn_video=%d\nn_ref=%d\nn_global=%d\n", (long long)info.n_slots,
         info.n_tiles, info.n_video, info.n_ref, info.n_global);
  printf("ref_tokens=%lld\ntarget_tokens=%lld\nglobal_rows=%lld\n", (long long)info.ref_tokens,
         (long long)info.target_tokens, (long long)info.global_rows);
  for (int i = 0; i < info.n_spans; ++i)
    printf("span%d.shape=%d,%d,%d\nspan%d.tile0=%d\n", i, info.spans[i].shape[0],
           info.spans[i].shape[1], info.spans[i].shape[2], i, info.span_tile0[i]);

  veda_select_info sel;
  st = veda_select_query(&info, gen, ref, head_dim, n_heads, &sel);
  printf("select_status=%d\n", (int)st);
  if (st != VEDA_OK) {
    printf("select_error=%s\n", veda_last_error());
    return 0;
  }
  printf("n_blocks=%d\nwidest=%d\nentries_per_head=%lld\nworkspace_bytes=%zu\n", sel.n_blocks,
         sel.widest, (long long)sel.entries_per_head, sel.workspace_bytes);
  for (int b = 0; b < sel.n_blocks; ++b)
    printf("block%d=%d,%d,%d,%d,%d,%.17g\n", b, sel.blocks[b].start, sel.blocks[b].stop,
           sel.blocks[b].keep_all, sel.blocks[b].k_lo, sel.blocks[b].k_hi, sel.blocks[b].frac);
  return 0;
}
