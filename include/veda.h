/*
 * veda.h - C ABI of the Veda learned block-sparse attention hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one on the page `veda_core.py` (the torch half of Veda on
 * ComfyUI): video tokens are packed into 128-token 3D tiles, tile pairs are
 * scored from triplet-pooled (mean | max | min) Q and K under per-head
 * projections, each query tile keeps a top-k of key tiles under a keep budget
 * (own tile always kept, fractional budgets spread evenly over rows, global
 * text rows dense both ways), and attention is computed only over the kept
 * 128x128 tile pairs.
 *
 * Three stages, three calls (plus host-only sizing queries):
 *   veda_plan    - tile packing: permutation of the sequence into tiles
 *   veda_select  - pooling, tile logits, top-k selection -> CSR tile lists
 *   veda_attend  - tile-skip attention over the CSR lists
 *
 * Conventions for every call:
 *   - Ownership: the caller allocates every device buffer and picks the
 *     stream. The library never allocates or frees device memory, keeps no
 *     device state between calls and never synchronises the stream.
 *   - Validation runs on the host first; a bad argument returns
 *     VEDA_ERR_INVALID (malformed request) or VEDA_ERR_UNSUPPORTED (valid
 *     but outside what the kernels handle) before anything is launched.
 *     After that a failed launch returns VEDA_ERR_DEVICE.
 *   - veda_last_error() returns the text of the last non-OK status of the
 *     calling thread (thread-local; valid until the thread's next call).
 *   - Row-major tensors: q, k, v, out are [S, H, D] views addressed as
 *     base + s*stride_s + h*stride_h + d (strides in elements, last dim
 *     contiguous).
 *   - All device buffers are plain device pointers on the current HIP device.
 */
#ifndef VEDA_H
#define VEDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VEDA_TILE 128
#define VEDA_MAX_SPANS 16
#define VEDA_MAX_BLOCKS 2
#define VEDA_MAX_HEADS 256

typedef enum {
  VEDA_OK = 0,
  VEDA_ERR_INVALID = 1,     /* malformed request (bad span list, budget, sizes) */
  VEDA_ERR_UNSUPPORTED = 2, /* valid but not handled (head_dim, alignment) */
  VEDA_ERR_DEVICE = 3       /* a HIP launch or call failed */
} veda_status;

typedef enum { VEDA_F32 = 0, VEDA_BF16 = 1 } veda_dtype;

/* One video span of the packed sequence: rows [start, start + T*H*W) hold a
 * (T, H, W) latent grid in t, h, w row-major order. shape = the tile box
 * (t, h, w) with t*h*w = 128, each a power of two; {0,0,0} asks for the
 * least-padding box (page `veda_core.py`, section "tiles",
 * least_padding_shape). */
typedef struct {
  int64_t start;
  int32_t grid[3];
  int32_t shape[3];
} veda_span;

/* A keep budget (page `veda_core.py`, section "budgets"): exactly one of
 * ratio / tiles is >= 0, the other negative (unset). ratio is the share of key
 * tiles KEPT (1 - sparsity); tiles is a per-row tile count. */
typedef struct {
  double ratio;
  double tiles;
} veda_budget;

/* The packed layout (page `veda_core.py`, section "tiles", build_layout).
 * Filled by veda_plan_query; plain data, copy freely. spans[] hold the
 * resolved boxes, the target span last. */
typedef struct {
  int64_t seq_len;
  int64_t n_slots;        /* n_tiles * 128 */
  int64_t ref_tokens;     /* real rows of all spans but the last */
  int64_t target_tokens;  /* real rows of the last span */
  int64_t global_rows;    /* rows no span covers */
  int32_t n_tiles, n_video, n_ref, n_global;
  int32_t n_spans;
  int32_t _pad;
  veda_span spans[VEDA_MAX_SPANS];
  int32_t span_tile0[VEDA_MAX_SPANS + 1]; /* first tile of each span; [n_spans] = n_video */
} veda_plan_info;

/* One column block of the selection (page `veda_core.py`, section
 * "selection", column_blocks / select): key tiles [start, stop) keep
 * k_lo + extra(r) tiles for query row r, extra(r) = floor((r+1) frac) >
 * floor(r frac) in doubles; keep_all = every tile of the block. */
typedef struct {
  int32_t start, stop;
  int32_t keep_all;
  int32_t k_lo, k_hi;
  int32_t _pad;
  double frac;
} veda_block;

/* Sizing of the selection output, filled by veda_select_query. */
typedef struct {
  int32_t n_blocks;
  int32_t head_dim;
  int32_t n_heads;        /* heads in this call (the group) */
  int32_t widest;         /* longest tile list of any row */
  int64_t entries_per_head; /* CSR entries of one head (row_offsets[n_tiles]) */
  size_t workspace_bytes; /* scratch veda_select needs (pooled + projected features, scores) */
  veda_block blocks[VEDA_MAX_BLOCKS];
} veda_select_info;

/* Text of the calling thread's last non-OK status ("" if none). */
const char *veda_last_error(void);

/* Library version string. */
const char *veda_version(void);

/* ---------------------------------------------------------------- plan --
 * Host only, synchronous. Validates the span list against seq_len and fills
 * `info`. Spans are in packed order with the target last; each must start at
 * or after the previous one's end and end within seq_len; at least one span
 * (page `veda_core.py`, section "tiles", build_layout).
 * Errors: INVALID for an empty/overlapping/overrunning list, a grid with a
 * non-positive side, a box that is not 128 power-of-two cells, seq_len
 * beyond 2^31 - 1 rows or more than VEDA_MAX_SPANS spans. */
veda_status veda_plan_query(const veda_span *spans, int32_t n_spans, int64_t seq_len,
                            veda_plan_info *info);

/* Builds the layout on the device (page `veda_core.py`, section "tiles",
 * span_tiles and build_layout):
 *   perm[n_slots]        int32: packed slot -> original row, -1 on padding.
 *                        Video tiles first (span order; boxes h-outer, w,
 *                        t-inner; cells t,h,w row-major; real rows a prefix
 *                        of each tile), then global rows ascending.
 *   valid_count[n_tiles] int32: real rows per tile (>= 1 for every tile).
 * Both are device buffers written in full. Asynchronous on `stream`. */
veda_status veda_plan(const veda_plan_info *info, int32_t *perm, int32_t *valid_count,
                      hipStream_t stream);

/* -------------------------------------------------------------- select --
 * Host only, synchronous. Resolves the column blocks and budget splits
 * (page `veda_core.py`, sections "budgets" and "selection": _per_row,
 * _split, column_blocks) and sizes the output for `n_heads` heads of width
 * `head_dim`. The reference budget is used only when the plan has reference
 * tiles. Errors: INVALID for a budget with neither or both fields set, or a
 * negative one; UNSUPPORTED for head_dim not in {64, 128}. */
veda_status veda_select_query(const veda_plan_info *info, veda_budget generated,
                              veda_budget reference, int32_t head_dim, int32_t n_heads,
                              veda_select_info *sel);

/* Scores tile pairs and selects key tiles for every query tile of the listed
 * heads (page `veda_core.py`, sections "predictor" and "selection": pool,
 * logits, select, block_mask, tile_index_list).
 *   q, k          device [S, H_total, D] in `dtype`, strides in elements.
 *   heads         HOST int32[n_heads]: which of the H_total heads, in order;
 *                 output index i refers to heads[i].
 *   proj_q/proj_k device float[n_heads][3D][D]: per-head projections
 *                 (x_hat = [mean|max|min] @ P + mean).
 *   row_offsets   device int32[n_tiles + 1], written: CSR row starts, the
 *                 same for every head.
 *   cols          device int32[n_heads * entries_per_head], written: for head
 *                 i, row a's kept key tiles in ascending order at
 *                 cols[i*entries_per_head + row_offsets[a] ...].
 *   scores        device double[n_heads][n_video][n_video] or NULL.
 *   scores_mode   0: compute logits into the workspace; 1: compute them and
 *                 also write them to `scores`; 2: skip pooling and scoring
 *                 and select from the given `scores`. In mode 0, when every
 *                 column block keeps all its tiles (ratio budgets >= 1), no
 *                 logit is needed and pooling and scoring are skipped.
 *   workspace     device scratch of at least sel->workspace_bytes (mode 2,
 *                 and mode 0 with every block keeping all, need none).
 * Selection is exact given the logits: rank by logit descending, lower
 * column first on ties; own tile +inf; logits and pooling are fp64.
 * Asynchronous on `stream`. */
veda_status veda_select(const veda_plan_info *info, const veda_select_info *sel,
                        const int32_t *perm, const int32_t *valid_count,
                        const void *q, const void *k, veda_dtype dtype,
                        int64_t stride_s, int64_t stride_h, int32_t n_heads_total,
                        const int32_t *heads, const float *proj_q, const float *proj_k,
                        int32_t *row_offsets, int32_t *cols,
                        double *scores, int32_t scores_mode,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* -------------------------------------------------------------- attend --
 * Tile-skip attention (page `veda_core.py`, reference_attend, which defines
 * the kernel's result): for head heads[i] and every query tile a, the real
 * query rows of a attend the real key rows of the tiles listed in row a of
 * the CSR, softmax(q.k * scale) v, and the result goes to out at the query's
 * original row. Padding slots are never read as keys and never written.
 *   q, k, v       device [S, H_total, D] in `dtype` (strides stride_s, stride_h).
 *   out           device [S, H_total, D] in `dtype` (out_stride_s, out_stride_h):
 *                 every row of the listed heads is written exactly once;
 *                 other heads are untouched.
 *   scale         softmax scale; <= 0 means head_dim^-1/2.
 * Every CSR row lists at least one tile (veda_select's rows always do; an
 * empty row leaves zeros). bf16 runs on MFMA (fp32 accumulate); f32 on the
 * vector ALU. Errors: UNSUPPORTED for head_dim not in {64, 128}; for bf16,
 * pointers/strides not 16-byte aligned, stride_s below head_dim or at least
 * 2^23 elements, seq_len of 2^24 rows or more, or one head's rows spanning
 * more than 3.5 GiB (rows are addressed with 32-bit offsets). Asynchronous
 * on `stream`. */
veda_status veda_attend(const veda_plan_info *info, const veda_select_info *sel,
                        const int32_t *perm, const int32_t *valid_count,
                        const void *q, const void *k, const void *v, void *out,
                        veda_dtype dtype, int64_t stride_s, int64_t stride_h,
                        int64_t out_stride_s, int64_t out_stride_h, int32_t n_heads_total,
                        const int32_t *heads, const int32_t *row_offsets, const int32_t *cols,
                        float scale, hipStream_t stream);

/* ---------------------------------------------------- attend, int8 Q.K^T --
 * veda_attend with the q.k products in int8, the approximate arithmetic the
 * news pages name for Veda's own kernel (an INT8 kernel, comfyui-wiki Veda
 * news, "Rendimiento" / "Performances"; the Vflash guide notes it gives no
 * exact-arithmetic guarantee). Same arguments and result as veda_attend
 * with bf16 q, k, v, out, up to the quantisation:
 *   key tile j of head heads[i]: s_k = max |k| over the tile's real rows
 *     divided by 127, codes rint(k / s_k) (round half to even), int8;
 *   query row r: s_q = max |q_r| / 127, codes rint(q_r / s_q);
 *   logit = (integer dot of the codes) * s_q * s_k * scale.
 * An all-zero row or tile has scale 0 and logits exactly 0. Probabilities,
 * row sums, P.V and the output are as in veda_attend's bf16 path.
 *   workspace  device scratch of at least the size veda_attend_int8_query
 *              gives, 16-byte aligned: the int8 codes of K in tile order
 *              (n_heads x n_tiles x 128 x head_dim bytes) and the per-tile
 *              scales (n_heads x n_tiles floats). Written in full by the
 *              call's first kernel, read by its second; nothing in it needs
 *              to start at zero. Calls that share one workspace on different
 *              streams race on it.
 * Errors: those of veda_attend for bf16; INVALID for a NULL or too small
 * workspace or dtype other than bf16 (there is no dtype argument: q, k, v
 * and out are bf16); UNSUPPORTED when one head's codes reach 2 GiB.
 * Asynchronous on `stream`. */
veda_status veda_attend_int8_query(const veda_plan_info *info, const veda_select_info *sel,
                                   size_t *workspace_bytes);
veda_status veda_attend_int8(const veda_plan_info *info, const veda_select_info *sel,
                             const int32_t *perm, const int32_t *valid_count,
                             const void *q, const void *k, const void *v, void *out,
                             int64_t stride_s, int64_t stride_h,
                             int64_t out_stride_s, int64_t out_stride_h, int32_t n_heads_total,
                             const int32_t *heads, const int32_t *row_offsets,
                             const int32_t *cols, float scale, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------- select, no allocation --
 * For callers that cannot allocate device memory or hand in a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. veda_select in scores_mode 0 (same arguments without scores
 * and workspace), with its scratch in one fixed device array of
 * VEDA_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends. The heads of a call are processed in chunks whose
 * pooled features, projections and logits fit the array (one head of the
 * 108,448-row headline layer, 870 video tiles, needs about 13 MB). Results
 * equal veda_select's bit for bit. Allocates nothing (no hipMalloc, no
 * hipFree). Every call on one GPU shares that GPU's array and leaves its
 * contents behind; nothing in it needs to start at zero (a call writes
 * everything it reads). Calls that overlap on one GPU (other streams or
 * threads) race on the array: serialise them. Errors: as veda_select;
 * UNSUPPORTED when one head's selection alone needs more than the array. */
#define VEDA_STATIC_SCRATCH_BYTES (64u << 20)
veda_status veda_select_static(const veda_plan_info *info, const veda_select_info *sel,
                               const int32_t *perm, const int32_t *valid_count,
                               const void *q, const void *k, veda_dtype dtype,
                               int64_t stride_s, int64_t stride_h, int32_t n_heads_total,
                               const int32_t *heads, const float *proj_q, const float *proj_k,
                               int32_t *row_offsets, int32_t *cols, hipStream_t stream);

/* ---------------------------------------------------- teacher and recall --
 * The tile-level teacher map that the news pages name as Veda's training
 * signal (full attention max-pooled onto the tiles; comfyui-wiki Veda news,
 * Spanish edition section "Qué hace Veda", French "Ce que fait Veda"), and
 * the recall of a selection against it. Not on the attention path: for
 * measuring how much of full attention the kept tiles cover.
 *
 * veda_teacher: for head heads[i], query tile a and key tile b,
 *   teacher[i][a][b] = max over the real rows r of a and the real rows j of b
 *                      of softmax_j(q_r . k_j * scale), the softmax over every
 *                      real row of the sequence (full attention).
 *   q, k    device bf16 [S, H_total, D] (strides in elements), D in {64, 128}.
 *   heads   HOST int32[n_heads].
 *   scale   softmax scale; <= 0 means head_dim^-1/2.
 *   teacher device float[n_heads][n_tiles][n_tiles], written in full.
 * Dense work: two passes of q.k over every tile pair (4 * 128^2 * D flop per
 * pair and head). Errors: UNSUPPORTED for f32 inputs or another head_dim.
 *
 * veda_recall: recall[i][a] = sum of teacher[i][a][b] over the tiles b in
 * row a of the CSR tile lists (as veda_select writes them, sel->n_heads
 * heads) divided by the sum over all b: the share of the teacher's
 * distribution the selection keeps. recall is device float[n_heads][n_tiles]. */
veda_status veda_teacher(const veda_plan_info *info, const int32_t *perm,
                         const int32_t *valid_count, const void *q, const void *k,
                         veda_dtype dtype, int64_t stride_s, int64_t stride_h,
                         int32_t n_heads_total, const int32_t *heads, int32_t n_heads,
                         int32_t head_dim, float scale, float *teacher, hipStream_t stream);
veda_status veda_recall(const veda_plan_info *info, const veda_select_info *sel,
                        const int32_t *row_offsets, const int32_t *cols, const float *teacher,
                        float *recall, hipStream_t stream);

/* Host only, synchronous: every check veda_attend makes (the arguments, the
 * head list, alignment and the bf16 path's addressing limits), with the same
 * arguments but no scale and no stream, and nothing launched. A layer made of
 * several calls can refuse a layout before it launches anything for it.
 * Pointers are tested for NULL and alignment only, never dereferenced.
 * Returns what veda_attend would return before launching. */
veda_status veda_attend_check(const veda_plan_info *info, const veda_select_info *sel,
                              const int32_t *perm, const int32_t *valid_count,
                              const void *q, const void *k, const void *v, const void *out,
                              veda_dtype dtype, int64_t stride_s, int64_t stride_h,
                              int64_t out_stride_s, int64_t out_stride_h, int32_t n_heads_total,
                              const int32_t *heads, const int32_t *row_offsets,
                              const int32_t *cols);

#ifdef __cplusplus
}
#endif

#endif /* VEDA_H */
