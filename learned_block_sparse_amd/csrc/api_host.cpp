// C ABI of libveda (include/veda.h): the host-only entry points. They touch
// no device memory and launch nothing, so this file builds with a plain host
// compiler (and with the sanitizers for host-only test runs).
#include "host.hpp"
#include "kernels.hpp"

using namespace veda;

extern "C" {

const char *veda_last_error(void) { return last_error(); }

const char *veda_version(void) { return "veda-mi355x 0.2 (gfx950)"; }

veda_status veda_plan_query(const veda_span *spans, int32_t n_spans, int64_t seq_len,
                            veda_plan_info *info) {
  return plan_query(spans, n_spans, seq_len, info);
}

veda_status veda_select_query(const veda_plan_info *info, veda_budget generated,
                              veda_budget reference, int32_t head_dim, int32_t n_heads,
                              veda_select_info *sel) {
  veda_status st = check_info(info);
  if (st != VEDA_OK) return st;
  return select_query(info, generated, reference, head_dim, n_heads, sel);
}

veda_status veda_attend_check(const veda_plan_info *info, const veda_select_info *sel,
                              const int32_t *perm, const int32_t *valid_count, const void *q,
                              const void *k, const void *v, const void *out, veda_dtype dtype,
                              int64_t stride_s, int64_t stride_h, int64_t out_stride_s,
                              int64_t out_stride_h, int32_t n_heads_total, const int32_t *heads,
                              const int32_t *row_offsets, const int32_t *cols) {
  AttendArgs a;
  HeadList hl;
  const veda_status st =
      attend_prepare(info, sel, perm, valid_count, q, k, v, const_cast<void *>(out), dtype,
                     stride_s, stride_h, out_stride_s, out_stride_h, n_heads_total, heads,
                     row_offsets, cols, 0.0f, &a, &hl);
  if (st == VEDA_OK) clear_error();
  return st;
}

veda_status veda_attend_int8_query(const veda_plan_info *info, const veda_select_info *sel,
                                   size_t *workspace_bytes) {
  if (!workspace_bytes) return fail(VEDA_ERR_INVALID, "workspace_bytes is NULL");
  Int8Workspace w;
  const veda_status st = int8_workspace(info, sel, &w);
  if (st != VEDA_OK) return st;
  *workspace_bytes = w.total;
  clear_error();
  return VEDA_OK;
}

}  // extern "C"
