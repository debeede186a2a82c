// Predictor and selection kernels (page `veda_core.py`, sections "predictor"
// and "selection").
//
//   pool_kernel     - [mean | max | min] of each video tile's real rows, per
//                     head, for q and k; fp64 sums, exact max/min. Rows are
//                     read through the plan's permutation (no tile-ordered
//                     copy of q or k is ever made).
//   project_kernel  - x_hat = f @ P + mean per head and tile, fp64.
//   score_kernel    - logits q_hat . k_hat / sqrt(D), an fp64 GEMM per head.
//   select_kernel   - one wavefront per (head, query tile): per column block,
//                     an exact top-k by an 8-bit-digit radix select over
//                     order-preserving 64-bit keys, ties to the lower column,
//                     then the kept columns written in ascending order with
//                     the global tiles after them (the CSR tile list).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace veda {

// ------------------------------------------------------------------ pool --
// One wave per (video tile, q or k, head): 16-byte row reads, LPR lanes per
// head row, so one load instruction covers RPL rows and the unrolled loop
// keeps several of them in flight. Each lane folds its rows into fp64 sums
// (exact for bf16 inputs of ordinary range, so the order does not matter;
// f32 inputs to within fp64 rounding) and fp32 max / min; the RPL lane
// groups are then combined by lane exchanges, and the first group writes
// the features.
template <int D, bool BF16>
__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a, HeadList heads,
                                                   const int32_t *__restrict__ perm,
                                                   const int32_t *__restrict__ valid_count) {
  constexpr int VPL = BF16 ? 8 : 4;        // values per 16-byte read
  constexpr int LPR = D / VPL;             // lanes per head row
  constexpr int RPL = 64 / LPR;            // rows per load instruction
  __shared__ int32_t rows[VEDA_TILE];
  const int32_t tile = blockIdx.x;
  const int which = blockIdx.y;  // 0: q, 1: k
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int hi = blockIdx.z * 4 + wave;
  const int32_t count = valid_count[tile];
  if (threadIdx.x < VEDA_TILE) rows[threadIdx.x] = perm[int64_t(tile) * VEDA_TILE + threadIdx.x];
  __syncthreads();
  if (hi >= a.n_heads) return;
  const int c = (lane % LPR) * VPL;
  const int rsub = lane / LPR;
  const unsigned char *base = static_cast<const unsigned char *>(a.x[which]) +
                              (int64_t(heads.h[hi]) * a.stride_h + c) * (BF16 ? 2 : 4);
  const int64_t pitch = a.stride_s * (BF16 ? 2 : 4);
  double sum[VPL];
  float mx[VPL], mn[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    sum[v] = 0.0;
    mx[v] = -INFINITY;
    mn[v] = INFINITY;
  }
#pragma unroll 8
  for (int r = rsub; r < count; r += RPL) {
    const uint4 u = *reinterpret_cast<const uint4 *>(base + int64_t(rows[r]) * pitch);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float x[VPL];
    if constexpr (BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      sum[v] += double(x[v]);
      mx[v] = fmaxf(mx[v], x[v]);
      mn[v] = fminf(mn[v], x[v]);
    }
  }
#pragma unroll
  for (int m = LPR; m < 64; m *= 2) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      sum[v] += __shfl_xor(sum[v], m, 64);
      mx[v] = fmaxf(mx[v], __shfl_xor(mx[v], m, 64));
      mn[v] = fminf(mn[v], __shfl_xor(mn[v], m, 64));
    }
  }
  if (rsub != 0) return;
  double *f = a.feat + ((int64_t(which) * a.n_heads + hi) * a.n_video + tile) * (3 * D);
  const double n_rows = count > 0 ? double(count) : 1.0;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    f[c + v] = count > 0 ? sum[v] / n_rows : 0.0;
    f[D + c + v] = count > 0 ? double(mx[v]) : 0.0;
    f[2 * D + c + v] = count > 0 ? double(mn[v]) : 0.0;
  }
}

hipError_t launch_pool(const PoolArgs &a, const HeadList &heads, const int32_t *perm,
                       const int32_t *valid_count, hipStream_t s) {
  const dim3 grid(a.n_video, 2, (a.n_heads + 3) / 4);
  if (a.head_dim == 128) {
    if (a.is_bf16)
      hipLaunchKernelGGL((pool_kernel<128, true>), grid, dim3(256), 0, s, a, heads, perm, valid_count);
    else
      hipLaunchKernelGGL((pool_kernel<128, false>), grid, dim3(256), 0, s, a, heads, perm, valid_count);
  } else {
    if (a.is_bf16)
      hipLaunchKernelGGL((pool_kernel<64, true>), grid, dim3(256), 0, s, a, heads, perm, valid_count);
    else
      hipLaunchKernelGGL((pool_kernel<64, false>), grid, dim3(256), 0, s, a, heads, perm, valid_count);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------- project --
// fp64 GEMM C = A B for the two small products of the predictor (about 4 and
// 5 GFLOP at 870 video tiles): a 64 x 64 output tile per 256-thread block, K
// in steps of 16 staged in LDS k-major, each thread a 4 x 4 register tile
// whose four A values are contiguous and whose four B values are two
// contiguous pairs (two 16-byte LDS reads each).
// Two schedules of the same arithmetic: gemm_tile stages one step at a time
// (68 registers, one 17 KB buffer: seven blocks fit a CU), gemm_tile_pipelined
// keeps the next step's global reads in flight during the current step's
// products (two LDS buffers, four blocks per CU). The logits (K = D, many
// rounds of blocks) always run pipelined; the projection (K = 3D) only when
// its grid fits the chip in one round of four blocks per CU, and otherwise
// staged, so that all of its blocks stay resident (about five per CU at 870
// video tiles).
constexpr int GT = 64, GK = 16;

struct GemmTile {
  double acc[4][4];
};

// Output column of accumulator w of thread column tx: two pairs of adjacent
// columns 32 apart, so 16 lanes' 16-byte LDS reads of a B row cover 256
// contiguous bytes, one per bank (four adjacent columns per thread put lanes
// tx and tx + 8 on the same banks).
static_assert(GT == 64, "gemm_col covers 64 columns");
__device__ inline int gemm_col(int tx, int w) { return (w < 2 ? 2 * tx : 32 + 2 * tx - 2) + w; }

// A: [M][K] fp64 row-major. B element (k, n) from load_b(k, n); B_NK says
// B is stored n-major ([N][K], loaded k-fastest like A) rather than k-major.
template <bool B_NK, class LoadB>
__device__ inline void gemm_tile(const double *A, int M, int K, int i0, int j0, int N,
                                 LoadB load_b, GemmTile &t) {
  // rows padded to 66 doubles (528 B, still 16-byte aligned): the k-fastest
  // stores of 16 lanes then land in distinct banks
  __shared__ __attribute__((aligned(16))) double As[GK][GT + 2];
  __shared__ __attribute__((aligned(16))) double Bs[GK][GT + 2];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) t.acc[u][w] = 0.0;
  for (int k0 = 0; k0 < K; k0 += GK) {
    for (int idx = threadIdx.x; idx < GT * GK; idx += 256) {
      const int r = idx / GK, kk = idx % GK;   // A: 16 consecutive k of one row
      As[kk][r] = (i0 + r < M && k0 + kk < K) ? A[int64_t(i0 + r) * K + k0 + kk] : 0.0;
      if constexpr (B_NK) {
        Bs[kk][r] = (j0 + r < N && k0 + kk < K) ? load_b(k0 + kk, j0 + r) : 0.0;
      } else {
        const int kb = idx / GT, c = idx % GT;    // B: 64 consecutive n of one k
        Bs[kb][c] = (j0 + c < N && k0 + kb < K) ? load_b(k0 + kb, j0 + c) : 0.0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; ++kk) {
      const double2 a01 = *reinterpret_cast<const double2 *>(&As[kk][ty * 4]);
      const double2 a23 = *reinterpret_cast<const double2 *>(&As[kk][ty * 4 + 2]);
      const double2 b01 = *reinterpret_cast<const double2 *>(&Bs[kk][2 * tx]);
      const double2 b23 = *reinterpret_cast<const double2 *>(&Bs[kk][32 + 2 * tx]);
      const double av[4] = {a01.x, a01.y, a23.x, a23.y};
      const double bv[4] = {b01.x, b01.y, b23.x, b23.y};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) t.acc[u][w] = fma(av[u], bv[w], t.acc[u][w]);
    }
    __syncthreads();
  }
}

constexpr int GPER = GT * GK / 256;   // A (and B) elements one thread stages per k step

// gemm_tile with two LDS buffers: the global reads of step s + 1 are in
// flight (in registers) while step s multiplies out of LDS, and one barrier
// per step separates a buffer's reads from its next fill.
template <bool B_NK, class LoadB>
__device__ inline void gemm_tile_pipelined(const double *A, int M, int K, int i0, int j0, int N,
                                           LoadB load_b, GemmTile &t) {
  // rows padded to 66 doubles (528 B, still 16-byte aligned): the k-fastest
  // stores of 16 lanes then land in distinct banks
  __shared__ __attribute__((aligned(16))) double As[2][GK][GT + 2];
  __shared__ __attribute__((aligned(16))) double Bs[2][GK][GT + 2];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) t.acc[u][w] = 0.0;
  double ra[GPER], rb[GPER];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int e = 0; e < GPER; ++e) {
      const int idx = int(threadIdx.x) + 256 * e;
      const int r = idx / GK, kk = idx % GK;   // A: GK consecutive k of one row
      ra[e] = (i0 + r < M && k0 + kk < K) ? A[int64_t(i0 + r) * K + k0 + kk] : 0.0;
      if constexpr (B_NK) {
        rb[e] = (j0 + r < N && k0 + kk < K) ? load_b(k0 + kk, j0 + r) : 0.0;
      } else {
        const int kb = idx / GT, c = idx % GT;    // B: 64 consecutive n of one k
        rb[e] = (j0 + c < N && k0 + kb < K) ? load_b(k0 + kb, j0 + c) : 0.0;
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int e = 0; e < GPER; ++e) {
      const int idx = int(threadIdx.x) + 256 * e;
      const int r = idx / GK, kk = idx % GK;
      As[buf][kk][r] = ra[e];
      if constexpr (B_NK) {
        Bs[buf][kk][r] = rb[e];
      } else {
        const int kb = idx / GT, c = idx % GT;
        Bs[buf][kb][c] = rb[e];
      }
    }
  };
  fetch(0);
  stash(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += GK) {
    const bool more = k0 + GK < K;
    if (more) fetch(k0 + GK);
#pragma unroll 4
    for (int kk = 0; kk < GK; ++kk) {
      const double2 a01 = *reinterpret_cast<const double2 *>(&As[buf][kk][ty * 4]);
      const double2 a23 = *reinterpret_cast<const double2 *>(&As[buf][kk][ty * 4 + 2]);
      const double2 b01 = *reinterpret_cast<const double2 *>(&Bs[buf][kk][2 * tx]);
      const double2 b23 = *reinterpret_cast<const double2 *>(&Bs[buf][kk][32 + 2 * tx]);
      const double av[4] = {a01.x, a01.y, a23.x, a23.y};
      const double bv[4] = {b01.x, b01.y, b23.x, b23.y};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) t.acc[u][w] = fma(av[u], bv[w], t.acc[u][w]);
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
}

// Projection (page `veda_core.py`, § predictor, `logits`): x_hat = f P + mean,
// f = [mean | max | min] (3D wide), P [3D][D] per head; the mean is the first
// D features of f.
template <bool PIPELINED>
__global__ void __launch_bounds__(256) project_kernel(ProjectArgs a) {
  const int D = a.head_dim, K = 3 * D, nv = a.n_video;
  const int hi = blockIdx.z >> 1, which = blockIdx.z & 1;
  const int i0 = blockIdx.y * GT, j0 = blockIdx.x * GT;
  const double *F = a.feat + (int64_t(which) * a.n_heads + hi) * nv * K;
  const float *P = a.proj[which] + int64_t(hi) * K * D;
  auto load_p = [&](int k, int n) { return double(P[int64_t(k) * D + n]); };
  GemmTile t;
  if constexpr (PIPELINED)
    gemm_tile_pipelined<false>(F, nv, K, i0, j0, D, load_p, t);
  else
    gemm_tile<false>(F, nv, K, i0, j0, D, load_p, t);
  double *dst = a.out + (int64_t(which) * a.n_heads + hi) * nv * D;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ty * 4 + u;
    if (i >= nv) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int j = j0 + gemm_col(tx, w);
      if (j < D) dst[int64_t(i) * D + j] = t.acc[u][w] + F[int64_t(i) * K + j];
    }
  }
}

// Grids up to this many projection blocks fit the chip in one round at the
// pipelined schedule's four blocks per CU (256 CUs); larger ones run the
// staged schedule, whose seven blocks per CU keep them resident.
constexpr int64_t PROJECT_PIPELINED_MAX_BLOCKS = 1024;

hipError_t launch_project(const ProjectArgs &a, hipStream_t s) {
  const dim3 grid((a.head_dim + GT - 1) / GT, (a.n_video + GT - 1) / GT, 2 * a.n_heads);
  if (int64_t(grid.x) * grid.y * grid.z <= PROJECT_PIPELINED_MAX_BLOCKS)
    hipLaunchKernelGGL(project_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(project_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- scores --
// Logits (page `veda_core.py`, § predictor, `logits`): q_hat . k_hat / sqrt(D)
// for every pair of video tiles, per head.
__global__ void __launch_bounds__(256) score_kernel(ScoreArgs a) {
  const int hi = blockIdx.z;
  const int i0 = blockIdx.y * GT, j0 = blockIdx.x * GT;
  const int nv = a.n_video, D = a.head_dim;
  const double *A = a.qh + int64_t(hi) * nv * D;
  const double *B = a.kh + int64_t(hi) * nv * D;
  GemmTile t;
  gemm_tile_pipelined<true>(A, nv, D, i0, j0, nv, [&](int k, int n) { return B[int64_t(n) * D + k]; }, t);
  double *C = a.scores + int64_t(hi) * nv * nv;
  double *C2 = a.scores_copy ? a.scores_copy + int64_t(hi) * nv * nv : nullptr;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ty * 4 + u;
    if (i >= nv) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int j = j0 + gemm_col(tx, w);
      if (j >= nv) continue;
      const double v = t.acc[u][w] / a.sqrt_d;
      C[int64_t(i) * nv + j] = v;
      if (C2) C2[int64_t(i) * nv + j] = v;
    }
  }
}

hipError_t launch_scores(const ScoreArgs &a, hipStream_t s) {
  const int nb = (a.n_video + GT - 1) / GT;
  hipLaunchKernelGGL(score_kernel, dim3(nb, nb, a.n_heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- select --
constexpr int SEL_WAVES = 4;
constexpr int SEL_REG_KEYS = 32;                 // most keys per lane held in registers

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Order-preserving map of a double to an unsigned key (larger value, larger
// key). -0.0 is folded onto +0.0 first so that equal values tie.
__device__ inline uint64_t order_key(double s) {
  s = s + 0.0;
  uint64_t u = __double_as_longlong(s);
  return (u >> 63) ? ~u : (u | (uint64_t(1) << 63));
}

__device__ inline int64_t row_offset_dev(const SelectArgs &a, int64_t r) {
  const int64_t nv = a.n_video;
  const int64_t rv = r < nv ? r : nv;
  int64_t off = 0;
  for (int b = 0; b < a.n_blocks; ++b) {
    const veda_block &k = a.blocks[b];
    if (k.keep_all) off += rv * int64_t(k.stop - k.start);
    else off += rv * int64_t(k.k_lo) + int64_t(floor(double(rv) * k.frac));
  }
  off += rv * int64_t(a.n_global);
  if (r > nv) off += (r - nv) * int64_t(a.n_tiles);
  return off;
}

struct RowKeys {
  const double *srow;   // scores of this row, block columns start at srow[start]
  const int32_t *vc;
  int32_t start, own;   // own = column of the row's own tile inside the block, or -1
  __device__ uint64_t key_of(double s, int32_t count, int j) const {
    if (count <= 0) s = -INFINITY;
    if (j == own) s = INFINITY;
    return order_key(s);
  }
  __device__ uint64_t compute(int j) const { return key_of(srow[start + j], vc[start + j], j); }
};

// A wave's row keeps its keys in registers, key j of the block in slot j / 64
// of lane j % 64, so every pass reads them without memory traffic and the
// workgroup needs LDS only for its histograms. SLOTS (8, 16 or 32 keys per
// lane) is sized to the call's widest selecting block, so narrow layouts hold
// fewer registers and fit more waves; a block wider than 64 SLOTS recomputes
// its keys on every pass.
template <int SLOTS>
__global__ void __launch_bounds__(64 * SEL_WAVES) select_kernel(SelectArgs a) {
  __shared__ int32_t hist_lds[SEL_WAVES][256];
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int64_t r = int64_t(blockIdx.x) * SEL_WAVES + wave;
  const int hi = blockIdx.y;
  if (r >= a.n_tiles) return;
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  const int64_t off = row_offset_dev(a, r);
  if (hi == 0 && lane == 0) {
    a.row_offsets[r] = int32_t(off);
    if (r == a.n_tiles - 1) a.row_offsets[r + 1] = int32_t(row_offset_dev(a, r + 1));
  }
  int32_t *out = a.cols + int64_t(hi) * a.entries_per_head + off;
  int64_t pos = 0;
  // Appends the non-empty tiles of [c0, c1) in order.
  auto emit_all = [&](int32_t c0, int32_t c1) {
    for (int32_t base = c0; base < c1; base += 64) {
      const int32_t j = base + lane;
      const bool keep = j < c1 && a.valid_count[j] > 0;
      const uint64_t km = __ballot(keep);
      if (keep) out[pos + __popcll(km & lt_mask)] = j;
      pos += __popcll(km);
    }
  };
  if (r >= a.n_video) {          // global rows see every non-empty tile
    emit_all(0, a.n_tiles);
    return;
  }
  int32_t *hist = hist_lds[wave];
  uint64_t kreg[SLOTS];
  for (int b = 0; b < a.n_blocks; ++b) {
    const veda_block blk = a.blocks[b];
    const int32_t n = blk.stop - blk.start;
    if (blk.keep_all) {
      emit_all(blk.start, blk.stop);
      continue;
    }
    const bool extra = floor(double(r + 1) * blk.frac) > floor(double(r) * blk.frac);
    int32_t k = min(blk.k_lo + (extra ? 1 : 0), blk.k_hi);
    RowKeys rk;
    rk.srow = a.scores + (int64_t(hi) * a.n_video + r) * a.n_video;
    rk.vc = a.valid_count;
    rk.start = blk.start;
    rk.own = (r >= blk.start && r < blk.stop) ? int32_t(r - blk.start) : -1;
    const bool in_regs = n <= 64 * SLOTS;
    if (in_regs) {
      // eight logits per lane in flight at a time (slots past the block
      // re-read its last column; their keys are never used)
#pragma unroll
      for (int u0 = 0; u0 < SLOTS; u0 += 8) {
        if (64 * u0 >= n) break;
        double sv[8];
        int32_t cv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = min(lane + 64 * (u0 + u), n - 1);
          sv[u] = rk.srow[rk.start + j];
          cv[u] = rk.vc[rk.start + j];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) kreg[u0 + u] = rk.key_of(sv[u], cv[u], lane + 64 * (u0 + u));
      }
    }
    // Radix select of the k-th largest key, 8 bits at a time from the top.
    uint64_t prefix = 0, mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = lane; i < 256; i += 64) hist[i] = 0;
      wave_sync();
      if (in_regs) {
#pragma unroll
        for (int u = 0; u < SLOTS; ++u) {
          if (64 * u >= n) break;
          if (lane + 64 * u < n && (kreg[u] & mask) == prefix)
            atomicAdd(&hist[(kreg[u] >> shift) & 255], 1);
        }
      } else {
        for (int j = lane; j < n; j += 64) {
          const uint64_t key = rk.compute(j);
          if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
        }
      }
      wave_sync();
      const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                c3 = hist[4 * lane + 3];
      const int tot = c0 + c1 + c2 + c3;
      int incl = tot;   // inclusive suffix sum: keys in digits >= 4*lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_down(incl, o, 64);
        if (lane + o < 64) incl += t;
      }
      const int excl = incl - tot;
      const uint64_t hit = __ballot(excl < k && k <= incl);
      const int L = __ffsll((unsigned long long)hit) - 1;
      int digit = 0, above = 0, bucket = 0;
      if (lane == L) {
        int run = excl;
        const int c[4] = {c0, c1, c2, c3};
        for (int q = 3; q >= 0; --q) {
          if (run + c[q] >= k) {
            digit = 4 * lane + q;
            above = run;
            bucket = c[q];
            break;
          }
          run += c[q];
        }
      }
      // L is uniform (from a ballot): scalar lane reads, no LDS round trip
      digit = __builtin_amdgcn_readlane(digit, L);
      above = __builtin_amdgcn_readlane(above, L);
      bucket = __builtin_amdgcn_readlane(bucket, L);
      prefix |= uint64_t(digit) << shift;
      mask |= uint64_t(255) << shift;
      k -= above;
      wave_sync();
      if (bucket == k) break;   // the whole bucket is kept: no finer digit needed
    }
    // Emit: keys above the prefix, and the first k keys equal to it by column,
    // in column order (slot by slot, lanes in order within a slot).
    const uint64_t neg_inf = order_key(-INFINITY);
    int eq_before = 0;
    auto emit_key = [&](int j, uint64_t key) {
      const bool valid = j < n;
      const uint64_t mk = key & mask;
      const bool gt = valid && mk > prefix;
      const bool eq = valid && mk == prefix;
      const uint64_t eqm = __ballot(eq);
      const int eqrank = eq_before + __popcll(eqm & lt_mask);
      const bool keep = (gt || (eq && eqrank < k)) && key != neg_inf;
      const uint64_t km = __ballot(keep);
      if (keep) out[pos + __popcll(km & lt_mask)] = blk.start + j;
      pos += __popcll(km);
      eq_before += __popcll(eqm);
    };
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < SLOTS; ++u) {
        if (64 * u >= n) break;
        emit_key(lane + 64 * u, kreg[u]);
      }
    } else {
      for (int base = 0; base < n; base += 64 * 8) {
        uint64_t kv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kv[u] = rk.compute(min(base + 64 * u + lane, n - 1));
#pragma unroll
        for (int u = 0; u < 8; ++u) emit_key(base + 64 * u + lane, kv[u]);
      }
    }
    wave_sync();
  }
  emit_all(a.n_video, a.n_tiles);
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  dim3 grid((a.n_tiles + SEL_WAVES - 1) / SEL_WAVES, a.n_heads);
  int32_t widest = 0;
  for (int b = 0; b < a.n_blocks; ++b)
    if (!a.blocks[b].keep_all) widest = max(widest, a.blocks[b].stop - a.blocks[b].start);
  if (widest <= 64 * 8)
    hipLaunchKernelGGL(select_kernel<8>, grid, dim3(64 * SEL_WAVES), 0, s, a);
  else if (widest <= 64 * 16)
    hipLaunchKernelGGL(select_kernel<16>, grid, dim3(64 * SEL_WAVES), 0, s, a);
  else
    hipLaunchKernelGGL(select_kernel<SEL_REG_KEYS>, grid, dim3(64 * SEL_WAVES), 0, s, a);
  return hipGetLastError();
}

}  // namespace veda
