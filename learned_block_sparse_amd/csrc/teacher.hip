// Tile-level teacher map and recall. The news pages describe Veda's
// training signal in one sentence: full attention, max-pooled onto the
// tiles, gives a tile-level teacher distribution (comfyui-wiki Veda news,
// Spanish edition section "Qué hace Veda", French edition "Ce que fait
// Veda"). Here, per head:
//   P[i, j]  = softmax over every real key row j of q_i . k_j / sqrt(D)
//   T[a, b]  = max of P[i, j] over the real rows i of query tile a and the
//              real rows j of key tile b
//   recall_a = sum over the kept tiles b of row a of T[a, b] / sum_b T[a, b]
//
// teacher_kernel: one workgroup (4 waves) per (head, query tile); wave w
// owns query rows 32w .. 32w+31. Two passes over every key tile, S^T = K Q^T
// by v_mfma_f32_32x32x16_bf16 (K staged in LDS, Q in registers), so a lane
// holds 64 scores of one query row (keys split with the lane 32 apart):
//   pass 1: each row's max m and sum l of exp2(c s - m) over all real keys;
//   pass 2: per key tile, each row's largest score s_max, whose probability
//           exp2(c s_max - m) / l is the row's largest in that tile; the max
//           over the tile's real query rows is T[a, b].
// recall_kernel: one wavefront per (head, query tile) reduces a row of T
// over all tiles and over the row's CSR tile list.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace veda {

namespace {

typedef __bf16 tbf16x8 __attribute__((ext_vector_type(8)));
typedef float tf32x16 __attribute__((ext_vector_type(16)));

constexpr int TW = 4;   // waves per workgroup

// 16-byte chunk c of K row r sits at chunk position c ^ swz(r): the A-operand
// reads (one chunk position of 32 consecutive rows) then spread over the
// banks. Rows are D*2 bytes: 16 chunks at D = 128, 8 at D = 64.
template <int D>
__device__ inline int chunk_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

// The lane 32 apart holds the other half of the same query's keys; with both
// operands x, v_permlane32_swap returns x of both lanes.
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(64 * TW) teacher_kernel(TeacherArgs a, HeadList heads) {
  constexpr int ROW = 2 * D;                  // bytes per K row
  constexpr int CHUNKS = D / 8;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) unsigned char Ks[128 * ROW];
  __shared__ float red[TW];
  const int tile = blockIdx.x, hi = blockIdx.y;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int g = lane / 32, l32 = lane % 32;
  const int64_t hoff = int64_t(heads.h[hi]) * a.stride_h;
  const uint16_t *qb = static_cast<const uint16_t *>(a.q) + hoff;
  const uint16_t *kb_ = static_cast<const uint16_t *>(a.k) + hoff;

  const int qi = wave * 32 + l32;
  const bool q_real = qi < a.valid_count[tile];
  const int32_t qrow = q_real ? a.perm[int64_t(tile) * 128 + qi] : -1;
  tbf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow >= 0)
      u = *reinterpret_cast<const uint4 *>(qb + int64_t(qrow) * a.stride_s + ks * 16 + g * 8);
    qf[ks] = __builtin_bit_cast(tbf16x8, u);
  }

  // Stages key tile b in LDS (padding rows as zeros) and forms this wave's
  // scores, the padding keys set to -inf.
  tf32x16 s[4];
  auto scores = [&](int b) {
    __syncthreads();   // the previous tile's reads are done
    const int32_t *pb = a.perm + int64_t(b) * 128;
    for (int c = threadIdx.x; c < 128 * CHUNKS; c += 64 * TW) {
      const int r = c / CHUNKS, ch = c % CHUNKS;
      const int32_t row = pb[r];
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row >= 0) u = *reinterpret_cast<const uint4 *>(kb_ + int64_t(row) * a.stride_s + ch * 8);
      *reinterpret_cast<uint4 *>(Ks + r * ROW + 16 * (ch ^ chunk_swz<D>(r))) = u;
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int r = kb * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const tbf16x8 A = *reinterpret_cast<const tbf16x8 *>(
            Ks + r * ROW + 16 * ((2 * ks + g) ^ chunk_swz<D>(r)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // lane l holds keys kb*32 + 8(i/4) + 4(l/32) + i%4 of query l % 32
    const int vc = a.valid_count[b];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + 8 * (i / 4) + 4 * g + (i % 4) >= vc) s[kb][i] = -INFINITY;
  };
  auto row_max = [&]() {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    return halves_max(mx);
  };

  // pass 1: row statistics in log2 units (c = scale * log2(e))
  const float c = a.scale_log2;
  float m = -INFINITY, l = 0.0f;
  for (int b = 0; b < a.n_tiles; ++b) {
    scores(b);
    const float m_new = fmaxf(m, row_max() * c);
    float sum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += exp2f(fmaf(s[kb][i], c, -m_new));
    l = l * exp2f(m - m_new) + halves_sum(sum);
    m = m_new;
  }
  const float inv_l = 1.0f / l;

  // pass 2: the largest probability of each key tile, max over query rows
  float *out = a.teacher + (int64_t(hi) * a.n_tiles + tile) * a.n_tiles;
  for (int b = 0; b < a.n_tiles; ++b) {
    scores(b);
    float p = q_real ? exp2f(fmaf(row_max(), c, -m)) * inv_l : 0.0f;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) p = fmaxf(p, __shfl_xor(p, off, 64));
    if (lane == 0) red[wave] = p;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = red[0];
      for (int w = 1; w < TW; ++w) t = fmaxf(t, red[w]);
      out[b] = t;
    }
  }
}

__global__ void __launch_bounds__(256) recall_kernel(RecallArgs a) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t unit = int64_t(blockIdx.x) * 4 + wave;   // (head, query tile)
  if (unit >= int64_t(a.n_heads) * a.n_tiles) return;
  const int hi = int(unit / a.n_tiles), tile = int(unit % a.n_tiles);
  const float *trow = a.teacher + unit * a.n_tiles;
  float all = 0.0f, kept = 0.0f;
  for (int b = lane; b < a.n_tiles; b += 64) all += trow[b];
  const int32_t *cols = a.cols + int64_t(hi) * a.entries_per_head;
  for (int e = a.row_offsets[tile] + lane; e < a.row_offsets[tile + 1]; e += 64)
    kept += trow[cols[e]];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    all += __shfl_xor(all, off, 64);
    kept += __shfl_xor(kept, off, 64);
  }
  if (lane == 0) a.recall[unit] = all > 0.0f ? kept / all : 0.0f;
}

hipError_t launch_teacher(const TeacherArgs &a, const HeadList &heads, int head_dim,
                          hipStream_t s) {
  const dim3 grid(a.n_tiles, a.n_heads);
  if (head_dim == 128)
    hipLaunchKernelGGL(teacher_kernel<128>, grid, dim3(64 * TW), 0, s, a, heads);
  else
    hipLaunchKernelGGL(teacher_kernel<64>, grid, dim3(64 * TW), 0, s, a, heads);
  return hipGetLastError();
}

hipError_t launch_recall(const RecallArgs &a, hipStream_t s) {
  const int64_t units = int64_t(a.n_heads) * a.n_tiles;
  hipLaunchKernelGGL(recall_kernel, dim3(unsigned((units + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace veda
