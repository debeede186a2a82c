// C ABI of libveda (include/veda.h): host validation, then launches.
#include <cmath>
#include <cstring>
#include <string>

#include "host.hpp"
#include "kernels.hpp"

using namespace veda;

namespace {

veda_status device_status(hipError_t e, const char *what) {
  if (e == hipSuccess) {
    clear_error();
    return VEDA_OK;
  }
  return fail(VEDA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

veda_status check_info(const veda_plan_info *info) {
  if (!info || info->n_spans <= 0 || info->n_spans > VEDA_MAX_SPANS || info->n_video <= 0 ||
      info->n_tiles < info->n_video)
    return fail(VEDA_ERR_INVALID, "plan info is empty or corrupt (call veda_plan_query)");
  return VEDA_OK;
}

// Tensors the kernels read 16 bytes at a time: base and both strides must keep
// every row 16-byte aligned.
veda_status check_tensor(const void *p, veda_dtype dt, int64_t ss, int64_t sh, const char *name) {
  if (!p) return fail(VEDA_ERR_INVALID, std::string(name) + " is NULL");
  const int64_t elt = dt == VEDA_BF16 ? 2 : 4;
  if (!aligned16(p) || (ss * elt) % 16 != 0 || (sh * elt) % 16 != 0)
    return fail(VEDA_ERR_UNSUPPORTED,
                std::string(name) + ": base and strides must be 16-byte aligned");
  return VEDA_OK;
}

veda_status fill_heads(const int32_t *heads, int32_t n_heads, int32_t n_heads_total,
                       HeadList *hl) {
  if (!heads) return fail(VEDA_ERR_INVALID, "heads is NULL");
  if (n_heads <= 0 || n_heads > VEDA_MAX_HEADS)
    return fail(VEDA_ERR_INVALID, "n_heads out of range");
  std::memset(hl, 0, sizeof(*hl));
  for (int i = 0; i < n_heads; ++i) {
    if (heads[i] < 0 || heads[i] >= n_heads_total)
      return fail(VEDA_ERR_INVALID, "head index " + std::to_string(heads[i]) + " not in [0, " +
                                        std::to_string(n_heads_total) + ")");
    hl->h[i] = heads[i];
  }
  return VEDA_OK;
}

}  // namespace

extern "C" {

const char *veda_last_error(void) { return last_error(); }

const char *veda_version(void) { return "veda-mi355x 0.1 (gfx950)"; }

veda_status veda_plan_query(const veda_span *spans, int32_t n_spans, int64_t seq_len,
                            veda_plan_info *info) {
  return plan_query(spans, n_spans, seq_len, info);
}

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

veda_status veda_select_query(const veda_plan_info *info, veda_budget generated,
                              veda_budget reference, int32_t head_dim, int32_t n_heads,
                              veda_select_info *sel) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  return select_query(info, generated, reference, head_dim, n_heads, sel);
}

veda_status veda_select(const veda_plan_info *info, const veda_select_info *sel,
                        const int32_t *perm, const int32_t *valid_count, const void *q,
                        const void *k, veda_dtype dtype, int64_t stride_s, int64_t stride_h,
                        int32_t n_heads_total, const int32_t *heads, const float *proj_q,
                        const float *proj_k, int32_t *row_offsets, int32_t *cols,
                        double *scores, int32_t scores_mode, void *workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  if (!sel || sel->n_blocks <= 0) return fail(VEDA_ERR_INVALID, "select info is empty (call veda_select_query)");
  if (!perm || !valid_count || !row_offsets || !cols)
    return fail(VEDA_ERR_INVALID, "perm / valid_count / row_offsets / cols is NULL");
  if (scores_mode < 0 || scores_mode > 2) return fail(VEDA_ERR_INVALID, "scores_mode must be 0, 1 or 2");
  if (scores_mode != 0 && !scores) return fail(VEDA_ERR_INVALID, "scores is NULL");
  if (dtype != VEDA_F32 && dtype != VEDA_BF16) return fail(VEDA_ERR_INVALID, "unknown dtype");
  HeadList hl;
  st = fill_heads(heads, sel->n_heads, n_heads_total, &hl);
  if (st != VEDA_OK) return st;
  const int D = sel->head_dim;
  const SelectWorkspace ws = select_workspace(info, D, sel->n_heads);
  const double *score_src = scores;
  if (scores_mode != 2) {
    if ((st = check_tensor(q, dtype, stride_s, stride_h, "q")) != VEDA_OK) return st;
    if ((st = check_tensor(k, dtype, stride_s, stride_h, "k")) != VEDA_OK) return st;
    if (!proj_q || !proj_k) return fail(VEDA_ERR_INVALID, "proj_q / proj_k is NULL");
    if (!workspace || workspace_bytes < ws.total)
      return fail(VEDA_ERR_INVALID, "workspace smaller than veda_select_info.workspace_bytes");
    unsigned char *w = static_cast<unsigned char *>(workspace);
    double *feat = reinterpret_cast<double *>(w + ws.feat_off);
    double *proj = reinterpret_cast<double *>(w + ws.proj_off);
    double *sc = reinterpret_cast<double *>(w + ws.score_off);
    PoolArgs pa;
    pa.x[0] = q;
    pa.x[1] = k;
    pa.stride_s = stride_s;
    pa.stride_h = stride_h;
    pa.n_heads = sel->n_heads;
    pa.head_dim = D;
    pa.n_video = info->n_video;
    pa.is_bf16 = dtype == VEDA_BF16;
    pa.feat = feat;
    hipError_t e = launch_pool(pa, hl, perm, valid_count, stream);
    if (e != hipSuccess) return device_status(e, "pool launch");
    ProjectArgs pr;
    pr.feat = feat;
    pr.proj[0] = proj_q;
    pr.proj[1] = proj_k;
    pr.out = proj;
    pr.n_heads = sel->n_heads;
    pr.head_dim = D;
    pr.n_video = info->n_video;
    e = launch_project(pr, stream);
    if (e != hipSuccess) return device_status(e, "project launch");
    ScoreArgs sa;
    sa.qh = proj;
    sa.kh = proj + size_t(sel->n_heads) * info->n_video * D;
    sa.scores = sc;
    sa.scores_copy = scores_mode == 1 ? scores : nullptr;
    sa.n_heads = sel->n_heads;
    sa.head_dim = D;
    sa.n_video = info->n_video;
    sa.sqrt_d = std::sqrt(double(D));
    e = launch_scores(sa, stream);
    if (e != hipSuccess) return device_status(e, "score launch");
    score_src = sc;
  }
  SelectArgs se;
  se.scores = score_src;
  se.valid_count = valid_count;
  se.row_offsets = row_offsets;
  se.cols = cols;
  se.entries_per_head = sel->entries_per_head;
  se.n_heads = sel->n_heads;
  se.n_video = info->n_video;
  se.n_tiles = info->n_tiles;
  se.n_global = info->n_global;
  se.n_blocks = sel->n_blocks;
  for (int b = 0; b < VEDA_MAX_BLOCKS; ++b) se.blocks[b] = sel->blocks[b];
  return device_status(launch_select(se, stream), "select launch");
}

veda_status veda_attend(const veda_plan_info *info, const veda_select_info *sel,
                        const int32_t *perm, const int32_t *valid_count, const void *q,
                        const void *k, const void *v, void *out, veda_dtype dtype,
                        int64_t stride_s, int64_t stride_h, int64_t out_stride_s,
                        int64_t out_stride_h, int32_t n_heads_total, const int32_t *heads,
                        const int32_t *row_offsets, const int32_t *cols, float scale,
                        hipStream_t stream) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  if (!sel || sel->n_blocks <= 0) return fail(VEDA_ERR_INVALID, "select info is empty (call veda_select_query)");
  if (!perm || !valid_count || !row_offsets || !cols)
    return fail(VEDA_ERR_INVALID, "perm / valid_count / row_offsets / cols is NULL");
  if (dtype != VEDA_F32 && dtype != VEDA_BF16) return fail(VEDA_ERR_INVALID, "unknown dtype");
  const int D = sel->head_dim;
  if (D != 64 && D != 128) return fail(VEDA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if ((st = check_tensor(q, dtype, stride_s, stride_h, "q")) != VEDA_OK) return st;
  if ((st = check_tensor(k, dtype, stride_s, stride_h, "k")) != VEDA_OK) return st;
  if ((st = check_tensor(v, dtype, stride_s, stride_h, "v")) != VEDA_OK) return st;
  if ((st = check_tensor(out, dtype, out_stride_s, out_stride_h, "out")) != VEDA_OK) return st;
  HeadList hl;
  st = fill_heads(heads, sel->n_heads, n_heads_total, &hl);
  if (st != VEDA_OK) return st;
  // K/V rows are read with 32-bit offsets from each head's first element.
  const int64_t elt = dtype == VEDA_BF16 ? 2 : 4;
  const int64_t kv_extent = ((info->seq_len - 1) * stride_s + D) * elt;
  if (dtype == VEDA_BF16 && kv_extent > int64_t(0xE0000000))
    return fail(VEDA_ERR_UNSUPPORTED, "q/k/v rows of one head span more than 3.5 GiB");
  // Row offsets are formed as row * pitch + chunk with 24-bit factors; a
  // padding slot is read as row seq_len, which must fall past the range above
  // (rows may not overlap) and still fit in 32 bits.
  if (dtype == VEDA_BF16 && (stride_s < D || stride_s * 2 >= (int64_t(1) << 24) ||
                             info->seq_len >= (int64_t(1) << 24) ||
                             (info->seq_len + 1) * stride_s * 2 > int64_t(0xFFFFFFFF)))
    return fail(VEDA_ERR_UNSUPPORTED,
                "bf16 attend needs D <= stride_s < 2^23 elements and seq_len < 2^24 rows");
  if (!(scale > 0.0f)) scale = float(1.0 / std::sqrt(double(D)));
  AttendArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.stride_s = stride_s;
  a.stride_h = stride_h;
  a.out_stride_s = out_stride_s;
  a.out_stride_h = out_stride_h;
  a.perm = perm;
  a.valid_count = valid_count;
  a.row_offsets = row_offsets;
  a.cols = cols;
  a.entries_per_head = sel->entries_per_head;
  a.n_heads = sel->n_heads;
  a.n_tiles = info->n_tiles;
  a.n_video = info->n_video;
  a.kv_bytes = uint32_t(kv_extent);
  a.pad_row = uint32_t(info->seq_len);
  a.scale = scale;
  a.scale_log2 = float(double(scale) * 1.4426950408889634);
  hipError_t e = dtype == VEDA_BF16 ? launch_attend_bf16(a, hl, D, stream)
                                    : launch_attend_f32(a, hl, D, stream);
  return device_status(e, "attend launch");
}

}  // extern "C"
