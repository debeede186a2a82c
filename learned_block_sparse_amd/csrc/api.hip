// C ABI of libveda (include/veda.h): the entry points that launch kernels.
// Each validates on the host first (host.cpp); the host-only entry points
// live in api_host.cpp.
#include <cmath>
#include <cstring>
#include <string>

#include "attend_i8.hpp"
#include "host.hpp"
#include "kernels.hpp"
#include "select_call.hpp"

using namespace veda;

namespace veda {

veda_status device_status(hipError_t e, const char *what) {
  if (e == hipSuccess) {
    clear_error();
    return VEDA_OK;
  }
  return fail(VEDA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

veda_status select_check(const veda_plan_info *info, const veda_select_info *sel,
                         const int32_t *perm, const int32_t *valid_count, const void *q,
                         const void *k, veda_dtype dtype, int64_t stride_s, int64_t stride_h,
                         int32_t n_heads_total, const int32_t *heads, const float *proj_q,
                         const float *proj_k, int32_t *row_offsets, int32_t *cols,
                         double *scores, int32_t scores_mode, SelectCall *c) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  if (!sel || sel->n_blocks <= 0)
    return fail(VEDA_ERR_INVALID, "select info is empty (call veda_select_query)");
  if (!perm || !valid_count || !row_offsets || !cols)
    return fail(VEDA_ERR_INVALID, "perm / valid_count / row_offsets / cols is NULL");
  if (scores_mode < 0 || scores_mode > 2)
    return fail(VEDA_ERR_INVALID, "scores_mode must be 0, 1 or 2");
  if (scores_mode != 0 && !scores) return fail(VEDA_ERR_INVALID, "scores is NULL");
  if (dtype != VEDA_F32 && dtype != VEDA_BF16) return fail(VEDA_ERR_INVALID, "unknown dtype");
  st = fill_heads(heads, sel->n_heads, n_heads_total, &c->heads);
  if (st != VEDA_OK) return st;
  // Blocks that keep every tile read no logits: when all of them do and no
  // logits are asked for, pooling and scoring are skipped.
  bool selects = false;
  for (int b = 0; b < sel->n_blocks; ++b) selects = selects || !sel->blocks[b].keep_all;
  c->scoring = scores_mode == 1 || (scores_mode == 0 && selects);
  if (c->scoring) {
    if ((st = check_tensor(q, dtype, stride_s, stride_h, "q")) != VEDA_OK) return st;
    if ((st = check_tensor(k, dtype, stride_s, stride_h, "k")) != VEDA_OK) return st;
    if (!proj_q || !proj_k) return fail(VEDA_ERR_INVALID, "proj_q / proj_k is NULL");
  }
  c->info = info;
  c->sel = sel;
  c->perm = perm;
  c->valid_count = valid_count;
  c->q = q;
  c->k = k;
  c->dtype = dtype;
  c->stride_s = stride_s;
  c->stride_h = stride_h;
  c->proj_q = proj_q;
  c->proj_k = proj_k;
  c->row_offsets = row_offsets;
  c->cols = cols;
  c->scores = scores;
  c->scores_mode = scores_mode;
  return VEDA_OK;
}

// Pooling, scoring and selection for heads [h0, h0 + nh) of a validated
// call; the workspace (when scoring) is laid out for nh heads.
veda_status select_range(const SelectCall &c, int32_t h0, int32_t nh, unsigned char *w,
                         hipStream_t stream) {
  const veda_plan_info *info = c.info;
  const int D = c.sel->head_dim;
  const int64_t nv = info->n_video;
  HeadList hl;
  std::memset(&hl, 0, sizeof(hl));
  for (int i = 0; i < nh; ++i) hl.h[i] = c.heads.h[h0 + i];
  double *scores = c.scores ? c.scores + size_t(h0) * nv * nv : nullptr;
  const double *score_src = scores;
  if (c.scoring) {
    const SelectWorkspace ws = select_workspace(info, D, nh);
    double *feat = reinterpret_cast<double *>(w + ws.feat_off);
    double *proj = reinterpret_cast<double *>(w + ws.proj_off);
    double *sc = reinterpret_cast<double *>(w + ws.score_off);
    PoolArgs pa;
    pa.x[0] = c.q;
    pa.x[1] = c.k;
    pa.stride_s = c.stride_s;
    pa.stride_h = c.stride_h;
    pa.n_heads = nh;
    pa.head_dim = D;
    pa.n_video = int32_t(nv);
    pa.is_bf16 = c.dtype == VEDA_BF16;
    pa.feat = feat;
    hipError_t e = launch_pool(pa, hl, c.perm, c.valid_count, stream);
    if (e != hipSuccess) return device_status(e, "pool launch");
    ProjectArgs pr;
    pr.feat = feat;
    pr.proj[0] = c.proj_q + size_t(h0) * 3 * D * D;
    pr.proj[1] = c.proj_k + size_t(h0) * 3 * D * D;
    pr.out = proj;
    pr.n_heads = nh;
    pr.head_dim = D;
    pr.n_video = int32_t(nv);
    e = launch_project(pr, stream);
    if (e != hipSuccess) return device_status(e, "project launch");
    ScoreArgs sa;
    sa.qh = proj;
    sa.kh = proj + size_t(nh) * nv * D;
    sa.scores = sc;
    sa.scores_copy = c.scores_mode == 1 ? scores : nullptr;
    sa.n_heads = nh;
    sa.head_dim = D;
    sa.n_video = int32_t(nv);
    sa.sqrt_d = std::sqrt(double(D));
    e = launch_scores(sa, stream);
    if (e != hipSuccess) return device_status(e, "score launch");
    score_src = sc;
  }
  SelectArgs se;
  se.scores = score_src;
  se.valid_count = c.valid_count;
  se.row_offsets = c.row_offsets;
  se.cols = c.cols + size_t(h0) * c.sel->entries_per_head;
  se.entries_per_head = c.sel->entries_per_head;
  se.n_heads = nh;
  se.n_video = int32_t(nv);
  se.n_tiles = info->n_tiles;
  se.n_global = info->n_global;
  se.n_blocks = c.sel->n_blocks;
  for (int b = 0; b < VEDA_MAX_BLOCKS; ++b) se.blocks[b] = c.sel->blocks[b];
  return device_status(launch_select(se, stream), "select launch");
}

}  // namespace veda

extern "C" {

veda_status veda_plan(const veda_plan_info *info, int32_t *perm, int32_t *valid_count,
                      hipStream_t stream) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  if (!perm || !valid_count) return fail(VEDA_ERR_INVALID, "perm / valid_count is NULL");
  PlanArgs a;
  std::memset(&a, 0, sizeof(a));
  a.seq_len = info->seq_len;
  a.n_spans = info->n_spans;
  a.n_video = info->n_video;
  a.n_tiles = info->n_tiles;
  a.global_rows = info->global_rows;
  int64_t prev_end = 0, prefix = 0;
  int ng = 0;
  for (int i = 0; i < info->n_spans; ++i) {
    const veda_span &s = info->spans[i];
    a.start[i] = s.start;
    for (int d = 0; d < 3; ++d) {
      a.grid[i][d] = s.grid[d];
      a.shape[i][d] = s.shape[d];
    }
    a.tile0[i] = info->span_tile0[i];
    // gap before this span
    a.gap_lo[ng] = prev_end;
    a.gap_prefix[ng] = prefix;
    prefix += s.start - prev_end;
    ++ng;
    prev_end = s.start + int64_t(s.grid[0]) * s.grid[1] * s.grid[2];
  }
  a.tile0[info->n_spans] = info->span_tile0[info->n_spans];
  a.gap_lo[ng] = prev_end;
  a.gap_prefix[ng] = prefix;
  prefix += info->seq_len - prev_end;
  ++ng;
  a.gap_prefix[ng] = prefix;
  a.n_gaps = ng;
  if (prefix != info->global_rows) return fail(VEDA_ERR_INVALID, "plan info is inconsistent");
  return device_status(launch_plan(a, perm, valid_count, stream), "veda_plan launch");
}

veda_status veda_select(const veda_plan_info *info, const veda_select_info *sel,
                        const int32_t *perm, const int32_t *valid_count, const void *q,
                        const void *k, veda_dtype dtype, int64_t stride_s, int64_t stride_h,
                        int32_t n_heads_total, const int32_t *heads, const float *proj_q,
                        const float *proj_k, int32_t *row_offsets, int32_t *cols,
                        double *scores, int32_t scores_mode, void *workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  SelectCall c;
  veda_status st = select_check(info, sel, perm, valid_count, q, k, dtype, stride_s, stride_h,
                                n_heads_total, heads, proj_q, proj_k, row_offsets, cols,
                                scores, scores_mode, &c);
  if (st != VEDA_OK) return st;
  if (c.scoring && (!workspace ||
                    workspace_bytes < select_workspace(info, sel->head_dim, sel->n_heads).total))
    return fail(VEDA_ERR_INVALID, "workspace smaller than veda_select_info.workspace_bytes");
  return select_range(c, 0, sel->n_heads, static_cast<unsigned char *>(workspace), stream);
}

veda_status veda_attend(const veda_plan_info *info, const veda_select_info *sel,
                        const int32_t *perm, const int32_t *valid_count, const void *q,
                        const void *k, const void *v, void *out, veda_dtype dtype,
                        int64_t stride_s, int64_t stride_h, int64_t out_stride_s,
                        int64_t out_stride_h, int32_t n_heads_total, const int32_t *heads,
                        const int32_t *row_offsets, const int32_t *cols, float scale,
                        hipStream_t stream) {
  AttendArgs a;
  HeadList hl;
  const veda_status st =
      attend_prepare(info, sel, perm, valid_count, q, k, v, out, dtype, stride_s, stride_h,
                     out_stride_s, out_stride_h, n_heads_total, heads, row_offsets, cols, scale,
                     &a, &hl);
  if (st != VEDA_OK) return st;
  const int D = sel->head_dim;
  hipError_t e = dtype == VEDA_BF16 ? launch_attend_bf16(a, hl, D, stream)
                                    : launch_attend_f32(a, hl, D, stream);
  return device_status(e, "attend launch");
}

veda_status veda_attend_int8(const veda_plan_info *info, const veda_select_info *sel,
                             const int32_t *perm, const int32_t *valid_count, const void *q,
                             const void *k, const void *v, void *out, int64_t stride_s,
                             int64_t stride_h, int64_t out_stride_s, int64_t out_stride_h,
                             int32_t n_heads_total, const int32_t *heads,
                             const int32_t *row_offsets, const int32_t *cols, float scale,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
  AttendArgs a;
  HeadList hl;
  veda_status st =
      attend_prepare(info, sel, perm, valid_count, q, k, v, out, VEDA_BF16, stride_s, stride_h,
                     out_stride_s, out_stride_h, n_heads_total, heads, row_offsets, cols, scale,
                     &a, &hl);
  if (st != VEDA_OK) return st;
  Int8Workspace w;
  if ((st = int8_workspace(info, sel, &w)) != VEDA_OK) return st;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(VEDA_ERR_INVALID, "workspace is NULL or not 16-byte aligned");
  if (workspace_bytes < w.total)
    return fail(VEDA_ERR_INVALID, "workspace smaller than veda_attend_int8_query's size");
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  QuantKArgs qa;
  qa.k = k;
  qa.stride_s = stride_s;
  qa.stride_h = stride_h;
  qa.perm = perm;
  qa.valid_count = valid_count;
  qa.kq = reinterpret_cast<signed char *>(ws + w.codes_off);
  qa.kscale = reinterpret_cast<float *>(ws + w.scale_off);
  qa.n_heads = sel->n_heads;
  qa.n_tiles = info->n_tiles;
  qa.head_dim = sel->head_dim;
  hipError_t e = launch_quant_k(qa, hl, stream);
  if (e != hipSuccess) return device_status(e, "int8 K quantisation launch");
  e = launch_attend_i8(a, hl, sel->head_dim, qa.kq, qa.kscale, stream);
  return device_status(e, "int8 attend launch");
}

}  // extern "C"

extern "C" {

veda_status veda_teacher(const veda_plan_info *info, const int32_t *perm,
                         const int32_t *valid_count, const void *q, const void *k,
                         veda_dtype dtype, int64_t stride_s, int64_t stride_h,
                         int32_t n_heads_total, const int32_t *heads, int32_t n_heads,
                         int32_t head_dim, float scale, float *teacher, hipStream_t stream) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  if (!perm || !valid_count || !teacher)
    return fail(VEDA_ERR_INVALID, "perm / valid_count / teacher is NULL");
  if (dtype != VEDA_BF16) return fail(VEDA_ERR_UNSUPPORTED, "the teacher map takes bf16 q and k");
  if (head_dim != 64 && head_dim != 128)
    return fail(VEDA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if ((st = check_tensor(q, dtype, stride_s, stride_h, "q")) != VEDA_OK) return st;
  if ((st = check_tensor(k, dtype, stride_s, stride_h, "k")) != VEDA_OK) return st;
  if (stride_s < head_dim) return fail(VEDA_ERR_UNSUPPORTED, "rows narrower than head_dim");
  HeadList hl;
  if ((st = fill_heads(heads, n_heads, n_heads_total, &hl)) != VEDA_OK) return st;
  if (int64_t(n_heads) * info->n_tiles * info->n_tiles > (int64_t(1) << 40))
    return fail(VEDA_ERR_UNSUPPORTED, "teacher map too large");
  if (!(scale > 0.0f)) scale = float(1.0 / std::sqrt(double(head_dim)));
  TeacherArgs a;
  a.q = q;
  a.k = k;
  a.stride_s = stride_s;
  a.stride_h = stride_h;
  a.perm = perm;
  a.valid_count = valid_count;
  a.teacher = teacher;
  a.n_heads = n_heads;
  a.n_tiles = info->n_tiles;
  a.scale_log2 = float(double(scale) * 1.4426950408889634);
  return device_status(launch_teacher(a, hl, head_dim, stream), "teacher launch");
}

veda_status veda_recall(const veda_plan_info *info, const veda_select_info *sel,
                        const int32_t *row_offsets, const int32_t *cols, const float *teacher,
                        float *recall, hipStream_t stream) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  if (!sel || sel->n_blocks <= 0)
    return fail(VEDA_ERR_INVALID, "select info is empty (call veda_select_query)");
  if (!row_offsets || !cols || !teacher || !recall)
    return fail(VEDA_ERR_INVALID, "row_offsets / cols / teacher / recall is NULL");
  RecallArgs a;
  a.teacher = teacher;
  a.row_offsets = row_offsets;
  a.cols = cols;
  a.entries_per_head = sel->entries_per_head;
  a.recall = recall;
  a.n_heads = sel->n_heads;
  a.n_tiles = info->n_tiles;
  return device_status(launch_recall(a, stream), "recall launch");
}

}  // extern "C"
