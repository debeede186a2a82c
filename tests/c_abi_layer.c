/* One layer through include/veda.h from plain C, on the GPU, with buffers
 * this program allocates itself: plan, select (pooling, logits, top-k) and
 * tile-skip attention, bf16 q, k, v. Built with gcc by tests/test_c_abi.py,
 * whose GPU test compares its output with the Python binding's, bit for bit.
 *
 * argv[1]: a directory holding
 *   layer.txt  "seq_len N", "span START T H W t h w" (packed order, target
 *              last), "budget GEN_RATIO GEN_TILES REF_RATIO REF_TILES",
 *              "head N_HEADS HEAD_DIM" (every head uses the target's box)
 *   q.bin, k.bin, v.bin   bf16 [S][N_HEADS][HEAD_DIM]
 *   pq.bin, pk.bin        float32 [N_HEADS][3 HEAD_DIM][HEAD_DIM]
 * writes out.bin there (bf16 [S][N_HEADS][HEAD_DIM]). Exit status 0 on
 * success; on a refusal or a HIP error it prints the reason and exits 1. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "veda.h"

static char dir[4096];

static int fail_hip(hipError_t e, const char *what) {
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 1;
}

static int fail_veda(veda_status st, const char *what) {
  fprintf(stderr, "%s: status %d: %s\n", what, (int)st, veda_last_error());
  return 1;
}

/* reads exactly `bytes` bytes of file `name` into a new host buffer */
static void *read_file(const char *name, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  void *p = malloc(bytes ? bytes : 1);
  size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

/* a device copy of `bytes` bytes of file `name`, or NULL */
static void *upload(const char *name, size_t bytes) {
  void *h = read_file(name, bytes), *d = NULL;
  if (!h) {
    fprintf(stderr, "cannot read %s (%zu bytes)\n", name, bytes);
    return NULL;
  }
  if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "cannot upload %s\n", name);
    d = NULL;
  }
  free(h);
  return d;
}

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  snprintf(dir, sizeof dir, "%s", argv[1]);

  veda_span spans[VEDA_MAX_SPANS + 1];
  int n_spans = 0, n_heads = 1, head_dim = 128;
  long long seq_len = 0;
  veda_budget gen = {-1.0, -1.0}, ref = {-1.0, -1.0};
  char path[4200], line[256];
  snprintf(path, sizeof path, "%s/layer.txt", dir);
  FILE *f = fopen(path, "r");
  if (!f) return fprintf(stderr, "cannot open %s\n", path), 1;
  while (fgets(line, sizeof line, f)) {
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
  fclose(f);
  if (n_heads < 1 || n_heads > VEDA_MAX_HEADS || seq_len < 1)
    return fprintf(stderr, "bad layer.txt\n"), 1;

  /* host side: layout and budgets, checked before anything is allocated */
  veda_plan_info info;
  veda_select_info sel;
  veda_status st = veda_plan_query(spans, n_spans, seq_len, &info);
  if (st != VEDA_OK) return fail_veda(st, "veda_plan_query");
  st = veda_select_query(&info, gen, ref, head_dim, n_heads, &sel);
  if (st != VEDA_OK) return fail_veda(st, "veda_select_query");

  const size_t elems = (size_t)seq_len * (size_t)n_heads * (size_t)head_dim;
  const size_t proj = (size_t)n_heads * 3u * (size_t)head_dim * (size_t)head_dim * sizeof(float);
  void *q = upload("q.bin", elems * 2), *k = upload("k.bin", elems * 2),
       *v = upload("v.bin", elems * 2);
  float *pq = (float *)upload("pq.bin", proj), *pk = (float *)upload("pk.bin", proj);
  if (!q || !k || !v || !pq || !pk) return 1;

  int32_t *heads = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_heads);
  for (int h = 0; h < n_heads; ++h) heads[h] = h;
  int32_t *perm = NULL, *vc = NULL, *ro = NULL, *cols = NULL;
  void *ws = NULL, *out = NULL;
  hipError_t e;
  if ((e = hipMalloc((void **)&perm, sizeof(int32_t) * (size_t)info.n_slots)) != hipSuccess ||
      (e = hipMalloc((void **)&vc, sizeof(int32_t) * (size_t)info.n_tiles)) != hipSuccess ||
      (e = hipMalloc((void **)&ro, sizeof(int32_t) * ((size_t)info.n_tiles + 1))) != hipSuccess ||
      (e = hipMalloc((void **)&cols, sizeof(int32_t) * (size_t)n_heads *
                                         (size_t)sel.entries_per_head)) != hipSuccess ||
      (e = hipMalloc(&ws, sel.workspace_bytes ? sel.workspace_bytes : 1)) != hipSuccess ||
      (e = hipMalloc(&out, elems * 2)) != hipSuccess)
    return fail_hip(e, "hipMalloc");

  hipStream_t stream;
  if ((e = hipStreamCreate(&stream)) != hipSuccess) return fail_hip(e, "hipStreamCreate");
  const int64_t ss = (int64_t)n_heads * head_dim, sh = head_dim;
  if ((st = veda_plan(&info, perm, vc, stream)) != VEDA_OK) return fail_veda(st, "veda_plan");
  if ((st = veda_select(&info, &sel, perm, vc, q, k, VEDA_BF16, ss, sh, n_heads, heads, pq, pk, ro,
                        cols, NULL, 0, ws, sel.workspace_bytes, stream)) != VEDA_OK)
    return fail_veda(st, "veda_select");
  if ((st = veda_attend(&info, &sel, perm, vc, q, k, v, out, VEDA_BF16, ss, sh, ss, sh, n_heads,
                        heads, ro, cols, 0.0f, stream)) != VEDA_OK)
    return fail_veda(st, "veda_attend");
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize");

  void *host = malloc(elems * 2);
  if ((e = hipMemcpy(host, out, elems * 2, hipMemcpyDeviceToHost)) != hipSuccess)
    return fail_hip(e, "hipMemcpy");
  snprintf(path, sizeof path, "%s/out.bin", dir);
  f = fopen(path, "wb");
  if (!f || fwrite(host, 1, elems * 2, f) != elems * 2) return fprintf(stderr, "cannot write out.bin\n"), 1;
  fclose(f);
  printf("ok n_tiles=%d entries_per_head=%lld\n", info.n_tiles, (long long)sel.entries_per_head);

  hipStreamDestroy(stream);
  hipFree(q), hipFree(k), hipFree(v), hipFree(pq), hipFree(pk);
  hipFree(perm), hipFree(vc), hipFree(ro), hipFree(cols), hipFree(ws), hipFree(out);
  free(heads), free(host);
  return 0;
}
