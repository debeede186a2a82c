// Host-side logic of libveda: validation, tile-box choice, layout sizing and
// the budget algebra. Plain C++ (no device code), so it also builds with g++
// for host-only sanitizer runs.
#pragma once

#include <cstdint>
#include <string>

#include "veda.h"

namespace veda {

struct AttendArgs;
struct HeadList;

// Thread-local text behind veda_last_error().
void set_error(const std::string &msg);
void clear_error();
const char *last_error();

// Records msg and returns st (for `return fail(...)`).
veda_status fail(veda_status st, const std::string &msg);

// Page `veda_core.py`, section "tiles": the 36 boxes, padded tile count and
// the least-padding choice.
int64_t tile_count(const int32_t grid[3], const int32_t shape[3]);
bool is_box(const int32_t shape[3]);
void least_padding_shape(const int32_t grid[3], int32_t out[3]);

// Fills info from a validated span list (build_layout's checks).
veda_status plan_query(const veda_span *spans, int32_t n_spans, int64_t seq_len,
                       veda_plan_info *info);

// Page `veda_core.py`, section "budgets", with Python's float semantics.
double per_row(veda_budget b, int64_t real_tokens, int32_t n_cols);
void split(double b, int32_t n_cols, int32_t *lo, int32_t *hi, double *frac);
double round12(double x);   // Python round(x, 12)
bool bresenham_extra(int64_t r, double frac);

// CSR row start of query tile r (0 <= r <= n_tiles), identical for every
// head: video rows keep k_lo + extra(r) per block plus every global tile,
// global rows keep every tile, and sum_{r' < r} extra(r') = floor(r * frac).
int64_t row_offset(const veda_plan_info *info, const veda_select_info *sel, int64_t r);

veda_status select_query(const veda_plan_info *info, veda_budget generated,
                         veda_budget reference, int32_t head_dim, int32_t n_heads,
                         veda_select_info *sel);

// Workspace layout of veda_select (byte offsets; all 256-byte aligned).
struct SelectWorkspace {
  size_t feat_off, feat_bytes;    // double [2][n_heads][n_video][3D]
  size_t proj_off, proj_bytes;    // double [2][n_heads][n_video][D]
  size_t score_off, score_bytes;  // double [n_heads][n_video][n_video]
  size_t total;
};
SelectWorkspace select_workspace(const veda_plan_info *info, int32_t head_dim, int32_t n_heads);

// Checks shared by the entry points (host only, no device access).
veda_status check_info(const veda_plan_info *info);
veda_status check_tensor(const void *p, veda_dtype dt, int64_t stride_s, int64_t stride_h,
                         const char *name);
veda_status fill_heads(const int32_t *heads, int32_t n_heads, int32_t n_heads_total,
                       HeadList *hl);

// Every check veda_attend makes, in order; on VEDA_OK fills the kernel
// arguments (veda_attend launches them, veda_attend_check discards them).
veda_status attend_prepare(const veda_plan_info *info, const veda_select_info *sel,
                           const int32_t *perm, const int32_t *valid_count, const void *q,
                           const void *k, const void *v, void *out, veda_dtype dtype,
                           int64_t stride_s, int64_t stride_h, int64_t out_stride_s,
                           int64_t out_stride_h, int32_t n_heads_total, const int32_t *heads,
                           const int32_t *row_offsets, const int32_t *cols, float scale,
                           AttendArgs *a, HeadList *hl);

// Workspace of veda_attend_int8: the int8 codes of K in tile order, then the
// per-tile scales (byte offsets; 256-byte aligned).
struct Int8Workspace {
  size_t codes_off, codes_bytes;   // int8 [n_heads][n_tiles][128][D]
  size_t scale_off, scale_bytes;   // float [n_heads][n_tiles]
  size_t total;
};
// Sizes it for sel->n_heads heads of width sel->head_dim; UNSUPPORTED when
// one head's codes reach 2^31 bytes (they are addressed with 32-bit offsets).
veda_status int8_workspace(const veda_plan_info *info, const veda_select_info *sel,
                           Int8Workspace *w);

}  // namespace veda
