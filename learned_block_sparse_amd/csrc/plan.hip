// Tile packing on the device (page `veda_core.py`, section "tiles",
// span_tiles and build_layout), one thread per packed slot.
//
// Instead of materialising each padded box and compacting its real cells
// (what the page's tensor ops do), a slot is mapped in closed form: a box
// (bt, bh, bw) of box size (st, sh, sw) over grid (T, H, W) has real extents
// r = min(s, g - b*s) on each axis, so it holds rt*rh*rw real rows, and the
// q-th real row in t,h,w row-major order sits at
// (q / (rh*rw), (q / rw) % rh, q % rw) inside the box. Every box holds its
// origin cell, so no tile is empty. Global rows (covered by no span) are the
// gaps between spans, enumerated in ascending order.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace veda {

__global__ void __launch_bounds__(256) plan_kernel(PlanArgs a, int32_t *__restrict__ perm,
                                                   int32_t *__restrict__ valid_count) {
  const int64_t slot = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n_slots = int64_t(a.n_tiles) * VEDA_TILE;
  if (slot >= n_slots) return;
  const int32_t tile = int32_t(slot / VEDA_TILE);
  const int32_t q = int32_t(slot % VEDA_TILE);
  int32_t row = -1;
  int32_t count = 0;
  if (tile < a.n_video) {
    int sp = 0;
    while (sp + 1 < a.n_spans && tile >= a.tile0[sp + 1]) ++sp;
    const int32_t T = a.grid[sp][0], H = a.grid[sp][1], W = a.grid[sp][2];
    const int32_t st = a.shape[sp][0], sh = a.shape[sp][1], sw = a.shape[sp][2];
    const int32_t nbt = (T + st - 1) / st, nbw = (W + sw - 1) / sw;
    const int32_t b = tile - a.tile0[sp];
    // box order: h-box outermost, then w-box, then t-box innermost
    const int32_t bt = b % nbt;
    const int32_t bw = (b / nbt) % nbw;
    const int32_t bh = b / (nbt * nbw);
    const int32_t rt = min(st, T - bt * st), rh = min(sh, H - bh * sh), rw = min(sw, W - bw * sw);
    count = rt * rh * rw;
    if (q < count) {
      const int32_t dt = q / (rh * rw), dh = (q / rw) % rh, dw = q % rw;
      const int64_t t = int64_t(bt) * st + dt, h = int64_t(bh) * sh + dh, w = int64_t(bw) * sw + dw;
      row = int32_t(a.start[sp] + (t * H + h) * W + w);
    }
  } else {
    const int64_t g0 = int64_t(tile - a.n_video) * VEDA_TILE;
    const int64_t gi = g0 + q;
    count = int32_t(min<int64_t>(VEDA_TILE, a.global_rows - g0));
    if (gi < a.global_rows) {
      int g = 0;
      while (g + 1 < a.n_gaps && gi >= a.gap_prefix[g + 1]) ++g;
      row = int32_t(a.gap_lo[g] + (gi - a.gap_prefix[g]));
    }
  }
  perm[slot] = row;
  if (q == 0) valid_count[tile] = count;
}

hipError_t launch_plan(const PlanArgs &a, int32_t *perm, int32_t *valid_count, hipStream_t s) {
  const int64_t n_slots = int64_t(a.n_tiles) * VEDA_TILE;
  const int threads = 256;
  const int64_t blocks = (n_slots + threads - 1) / threads;
  hipLaunchKernelGGL(plan_kernel, dim3(unsigned(blocks)), dim3(threads), 0, s, a, perm,
                     valid_count);
  return hipGetLastError();
}

}  // namespace veda
