// Launch interface of the INT8 Q.K^T variant of the attend stage
// (attend_i8.hip): K quantised per (head, key tile) by a pre-pass, Q per
// query row inside the attend kernel, S = K Q^T on int8 MFMA; the softmax
// and P V are those of the bf16 kernel.
#pragma once

#include "kernels.hpp"

namespace veda {

struct QuantKArgs {
  const void *k;              // bf16 [S, H, D] rows
  int64_t stride_s, stride_h;
  const int32_t *perm, *valid_count;
  signed char *kq;            // [n_heads][n_tiles][128][D] int8, tile order, padding rows 0
  float *kscale;              // [n_heads][n_tiles]: a tile's int8 unit in K's units
  int32_t n_heads, n_tiles, head_dim;
};
hipError_t launch_quant_k(const QuantKArgs &a, const HeadList &heads, hipStream_t s);

hipError_t launch_attend_i8(const AttendArgs &a, const HeadList &heads, int head_dim,
                            const signed char *kq, const float *kscale, hipStream_t s);

}  // namespace veda
