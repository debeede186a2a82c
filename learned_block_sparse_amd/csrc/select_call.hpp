// A validated veda_select call and the launch of one range of its heads:
// shared by veda_select (all heads, the caller's workspace) and its
// no-allocation variant (head chunks through a fixed device scratch).
#pragma once

#include "host.hpp"
#include "kernels.hpp"

namespace veda {

// A validated veda_select call.
struct SelectCall {
  const veda_plan_info *info;
  const veda_select_info *sel;
  const int32_t *perm, *valid_count;
  const void *q, *k;
  veda_dtype dtype;
  int64_t stride_s, stride_h;
  HeadList heads;
  const float *proj_q, *proj_k;
  int32_t *row_offsets, *cols;
  double *scores;
  int32_t scores_mode;
  bool scoring;   // pooling and scoring run (else selection reads `scores` or needs none)
};

veda_status device_status(hipError_t e, const char *what);

// Every check veda_select makes before launching; fills *c.
veda_status select_check(const veda_plan_info *info, const veda_select_info *sel,
                         const int32_t *perm, const int32_t *valid_count, const void *q,
                         const void *k, veda_dtype dtype, int64_t stride_s, int64_t stride_h,
                         int32_t n_heads_total, const int32_t *heads, const float *proj_q,
                         const float *proj_k, int32_t *row_offsets, int32_t *cols,
                         double *scores, int32_t scores_mode, SelectCall *c);

// Pooling, scoring and selection for heads [h0, h0 + nh) of a checked call,
// in that order on `stream`; when scoring, `workspace` holds at least
// select_workspace(info, head_dim, nh).total bytes.
veda_status select_range(const SelectCall &c, int32_t h0, int32_t nh, unsigned char *workspace,
                         hipStream_t stream);

}  // namespace veda
