// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "veda.h"

namespace veda {

// ----------------------------------------------------------------- plan --
struct PlanArgs {
  int64_t seq_len;
  int32_t n_spans, n_video, n_tiles;
  int32_t n_gaps;
  int64_t global_rows;
  int64_t start[VEDA_MAX_SPANS];
  int32_t grid[VEDA_MAX_SPANS][3];
  int32_t shape[VEDA_MAX_SPANS][3];
  int32_t tile0[VEDA_MAX_SPANS + 1];
  // Rows no span covers, as gaps: gap g is [gap_lo[g], gap_lo[g] + len) and
  // holds global rows gap_prefix[g] .. gap_prefix[g+1]-1.
  int64_t gap_lo[VEDA_MAX_SPANS + 1];
  int64_t gap_prefix[VEDA_MAX_SPANS + 2];
};

hipError_t launch_plan(const PlanArgs &a, int32_t *perm, int32_t *valid_count, hipStream_t s);

// --------------------------------------------------------------- select --
struct HeadList {
  int32_t h[VEDA_MAX_HEADS];
};

struct PoolArgs {
  const void *x[2];          // q, k
  int64_t stride_s, stride_h;
  int32_t n_heads, head_dim, n_video;
  int32_t is_bf16;
  double *feat;              // [2][n_heads][n_video][3D]
};
hipError_t launch_pool(const PoolArgs &a, const HeadList &heads, const int32_t *perm,
                       const int32_t *valid_count, hipStream_t s);

struct ProjectArgs {
  const double *feat;        // [2][n_heads][n_video][3D]
  const float *proj[2];      // [n_heads][3D][D]
  double *out;               // [2][n_heads][n_video][D]
  int32_t n_heads, head_dim, n_video;
};
hipError_t launch_project(const ProjectArgs &a, hipStream_t s);

struct ScoreArgs {
  const double *qh, *kh;     // [n_heads][n_video][D]
  double *scores;            // [n_heads][n_video][n_video]
  double *scores_copy;       // optional second destination (NULL)
  int32_t n_heads, head_dim, n_video;
  double sqrt_d;             // logits are dot / sqrt(D)
};
hipError_t launch_scores(const ScoreArgs &a, hipStream_t s);

struct SelectArgs {
  const double *scores;      // [n_heads][n_video][n_video]
  const int32_t *valid_count;
  int32_t *row_offsets;      // [n_tiles + 1]
  int32_t *cols;             // [n_heads][entries_per_head]
  int64_t entries_per_head;
  int32_t n_heads, n_video, n_tiles, n_global;
  int32_t n_blocks;
  veda_block blocks[VEDA_MAX_BLOCKS];
};
hipError_t launch_select(const SelectArgs &a, hipStream_t s);

// --------------------------------------------------------------- attend --
struct AttendArgs {
  const void *q, *k, *v;
  void *out;
  int64_t stride_s, stride_h, out_stride_s, out_stride_h;
  const int32_t *perm, *valid_count, *row_offsets, *cols;
  int64_t entries_per_head;
  int32_t n_heads, n_tiles, n_video;
  uint32_t kv_bytes;         // bytes from a head's first K/V element to the end of its last row
  uint32_t pad_row;          // a padding slot (row id -1) is fetched as this row, one past the last
  float scale_log2;          // softmax scale * log2(e)
  float scale;               // softmax scale
};
hipError_t launch_attend_bf16(const AttendArgs &a, const HeadList &heads, int head_dim,
                              hipStream_t s);
hipError_t launch_attend_f32(const AttendArgs &a, const HeadList &heads, int head_dim,
                             hipStream_t s);

// -------------------------------------------------------------- teacher --
struct TeacherArgs {
  const void *q, *k;          // bf16 [S, H, D] rows
  int64_t stride_s, stride_h;
  const int32_t *perm, *valid_count;
  float *teacher;             // [n_heads][n_tiles][n_tiles]
  int32_t n_heads, n_tiles;
  float scale_log2;           // softmax scale * log2(e)
};
hipError_t launch_teacher(const TeacherArgs &a, const HeadList &heads, int head_dim,
                          hipStream_t s);

struct RecallArgs {
  const float *teacher;       // [n_heads][n_tiles][n_tiles]
  const int32_t *row_offsets, *cols;
  int64_t entries_per_head;
  float *recall;              // [n_heads][n_tiles]
  int32_t n_heads, n_tiles;
};
hipError_t launch_recall(const RecallArgs &a, hipStream_t s);

}  // namespace veda
