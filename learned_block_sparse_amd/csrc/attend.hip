// Tile-skip attention (page `veda_core.py`, reference_attend defines the
// result; the pages' own kernel streams only the selected K/V tiles). One
// workgroup per (head, query tile); it walks the query tile's CSR list of
// kept key tiles with an online softmax, reading q/k/v rows through the
// plan's permutation and writing each real query row's output straight to
// its original row (no tile-ordered copies, no scatter pass).
//
// bf16 kernel (MFMA, gfx950):
//   4 wavefronts x 32 query rows. Per kept key tile, K (128 x D) and V are
//   staged in LDS. Scores are formed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, the wave's Q held
//   in registers as B), so each lane holds 64 scores of ONE query row: the
//   row max and row sum are in-lane reductions plus one exchange with the
//   lane 32 apart. The probabilities, converted to bf16, are already laid
//   out as the B operand of O^T += V^T P^T; V is stored transposed in LDS
//   with keys permuted inside each 16-key group ({0-3, 8-11 | 4-7, 12-15})
//   so that each A operand is one 16-byte LDS read.
// f32 kernel (vector ALU): 2 threads per query row, keys in chunks of 32.
#include "kernels.hpp"

namespace veda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Dispatch order: the heavy global query tiles (they see every tile) first,
// then the video tiles. Video tiles are remapped so that each of the 8 XCDs
// (which take workgroups round-robin) works through a contiguous range of
// (head, query tile): neighbouring query tiles share most key tiles, and the
// shared tiles then stay in that XCD's L2.
struct BlockMap {
  int32_t hi, tile;
  bool live;
};

__device__ inline BlockMap map_block(const AttendArgs &a, uint32_t b) {
  BlockMap m{0, 0, false};
  const uint32_t G = uint32_t(a.n_heads) * uint32_t(a.n_tiles - a.n_video);
  const uint32_t Gp = (G + 7u) & ~7u;
  if (b < Gp) {
    if (b >= G) return m;
    const uint32_t ng = uint32_t(a.n_tiles - a.n_video);
    m.hi = int32_t(b / ng);
    m.tile = a.n_video + int32_t(b % ng);
    m.live = true;
    return m;
  }
  const uint32_t bv = b - Gp;
  const uint32_t NV = uint32_t(a.n_heads) * uint32_t(a.n_video);
  const uint32_t per = (NV + 7u) / 8u;
  const uint32_t logical = (bv % 8u) * per + bv / 8u;
  if (logical >= NV) return m;
  m.hi = int32_t(logical / uint32_t(a.n_video));
  m.tile = int32_t(logical % uint32_t(a.n_video));
  m.live = true;
  return m;
}

__host__ inline uint32_t grid_blocks(const AttendArgs &a) {
  const uint32_t G = uint32_t(a.n_heads) * uint32_t(a.n_tiles - a.n_video);
  const uint32_t Gp = (G + 7u) & ~7u;
  const uint32_t NV = uint32_t(a.n_heads) * uint32_t(a.n_video);
  return Gp + 8u * ((NV + 7u) / 8u);
}

// --------------------------------------------------------------- bf16 MFMA --
template <int D>
struct Bf16Cfg {
  static constexpr int KPITCH = D * 2 + 16;        // bytes per K row in LDS
  static constexpr int VPITCH = VEDA_TILE * 2 + 16;  // bytes per V^T row (one d)
  static constexpr int K_UNITS = VEDA_TILE * D / 8 / 256;  // 16-byte K loads per thread
  static constexpr int V_UNITS = 32 * (D / 8) / 256;       // 4-row V groups per thread
  static constexpr int LDS_BYTES = VEDA_TILE * KPITCH + D * VPITCH;
};

__device__ inline uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

template <int D>
__global__ void __launch_bounds__(256, 2) attend_bf16_kernel(AttendArgs a, HeadList heads) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS_BYTES];
  unsigned char *k_lds = lds;
  unsigned char *v_lds = lds + VEDA_TILE * C::KPITCH;

  const BlockMap bm = map_block(a, blockIdx.x);
  if (!bm.live) return;
  const int hi = bm.hi, tile = bm.tile;
  const int64_t hoff = int64_t(heads.h[hi]) * a.stride_h;
  const uint16_t *qb = static_cast<const uint16_t *>(a.q) + hoff;
  const uint16_t *kb_ = static_cast<const uint16_t *>(a.k) + hoff;
  const uint16_t *vb = static_cast<const uint16_t *>(a.v) + hoff;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int g = lane / 32, l32 = lane % 32;

  // Q fragment (B operand of S^T = K Q^T): lane holds q[row][16*ks + 8*g .. +8].
  const int32_t vc_q = a.valid_count[tile];
  const int qi = wave * 32 + l32;
  const int32_t qrow = qi < vc_q ? a.perm[int64_t(tile) * VEDA_TILE + qi] : -1;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow >= 0) u = ld16(qb + int64_t(qrow) * a.stride_s + ks * 16 + g * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, u);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const int32_t t_begin = a.row_offsets[tile], t_end = a.row_offsets[tile + 1];
  const int32_t *list = a.cols + int64_t(hi) * a.entries_per_head;

  uint4 kreg[C::K_UNITS];
  uint4 vreg[C::V_UNITS][4];
  auto load_tile = [&](int32_t j) {
    const int32_t vc = a.valid_count[j];
    const int32_t *pj = a.perm + int64_t(j) * VEDA_TILE;
#pragma unroll
    for (int it = 0; it < C::K_UNITS; ++it) {
      const int u = tid + 256 * it;
      const int key = u / (D / 8), dc = u % (D / 8);
      uint4 x = make_uint4(0, 0, 0, 0);
      if (key < vc) x = ld16(kb_ + int64_t(pj[key]) * a.stride_s + dc * 8);
      kreg[it] = x;
    }
#pragma unroll
    for (int it = 0; it < C::V_UNITS; ++it) {
      const int u = tid + 256 * it;
      const int c = u % 32, dc = u / 32;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 4 * c + rr;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (key < vc) x = ld16(vb + int64_t(pj[key]) * a.stride_s + dc * 8);
        vreg[it][rr] = x;
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::K_UNITS; ++it) {
      const int u = tid + 256 * it;
      const int key = u / (D / 8), dc = u % (D / 8);
      *reinterpret_cast<uint4 *>(k_lds + key * C::KPITCH + dc * 16) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < C::V_UNITS; ++it) {
      const int u = tid + 256 * it;
      const int c = u % 32, dc = u / 32;
      // keys 4c..4c+3 go to position (16*(c/4) + 4*blk) with blk = {0,2,1,3}[c%4]
      const int cq = c % 4;
      const int posblk = (cq == 1) ? 2 : (cq == 2) ? 1 : cq;
      const int col = 16 * (c / 4) + 4 * posblk;
      const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&vreg[it][0]);
      const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&vreg[it][1]);
      const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&vreg[it][2]);
      const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&vreg[it][3]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // d = 8*dc + 2w (low halves) and 8*dc + 2w + 1 (high halves)
        uint2 lo, hi2;
        lo.x = (r0[w] & 0xffffu) | (r1[w] << 16);
        lo.y = (r2[w] & 0xffffu) | (r3[w] << 16);
        hi2.x = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
        hi2.y = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
        const int d0 = 8 * dc + 2 * w;
        *reinterpret_cast<uint2 *>(v_lds + d0 * C::VPITCH + col * 2) = lo;
        *reinterpret_cast<uint2 *>(v_lds + (d0 + 1) * C::VPITCH + col * 2) = hi2;
      }
    }
  };

  if (t_begin < t_end) load_tile(list[t_begin]);
  for (int32_t t = t_begin; t < t_end; ++t) {
    const int32_t vcj = a.valid_count[list[t]];
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < t_end) load_tile(list[t + 1]);

    // S^T = K Q^T for 4 blocks of 32 keys
    f32x16 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 A = *reinterpret_cast<const bf16x8 *>(
            k_lds + (kb * 32 + l32) * C::KPITCH + (ks * 16 + g * 8) * 2);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[ks], s[kb], 0, 0, 0);
      }
    }
    if (vcj < VEDA_TILE) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 8 * (i / 4) + 4 * g + (i % 4);
          if (key >= vcj) s[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float rs = 0.0f;
    bf16x8 pb[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, -m_new));
        rs += p;
        pb[kb][i / 8][i % 8] = static_cast<__bf16>(p);
      }
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bf16x8 A = *reinterpret_cast<const bf16x8 *>(
              v_lds + (db * 32 + l32) * C::VPITCH + (kb * 32 + e * 16 + g * 8) * 2);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, pb[kb][e], o[db], 0, 0, 0);
        }
  }

  if (qrow < 0) return;
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  uint16_t *ob = static_cast<uint16_t *>(a.out) + int64_t(qrow) * a.out_stride_s +
                 int64_t(heads.h[hi]) * a.out_stride_h;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int d = db * 32 + 8 * p + 4 * g;
      uint16_t h4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        h4[r] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(o[db][4 * p + r] * inv));
      uint2 w;
      w.x = uint32_t(h4[0]) | (uint32_t(h4[1]) << 16);
      w.y = uint32_t(h4[2]) | (uint32_t(h4[3]) << 16);
      *reinterpret_cast<uint2 *>(ob + d) = w;
    }
}

hipError_t launch_attend_bf16(const AttendArgs &a, const HeadList &heads, int head_dim,
                              hipStream_t s) {
  const dim3 grid(grid_blocks(a));
  if (head_dim == 128)
    hipLaunchKernelGGL(attend_bf16_kernel<128>, grid, dim3(256), 0, s, a, heads);
  else
    hipLaunchKernelGGL(attend_bf16_kernel<64>, grid, dim3(256), 0, s, a, heads);
  return hipGetLastError();
}

// ------------------------------------------------------------ f32 (VALU) --
constexpr int F32_CHUNK = 32;

template <int D>
__global__ void __launch_bounds__(256) attend_f32_kernel(AttendArgs a, HeadList heads) {
  constexpr int HD = D / 2;
  __shared__ float ks[F32_CHUNK][D + 4];
  __shared__ float vs[F32_CHUNK][D + 4];
  const BlockMap bm = map_block(a, blockIdx.x);
  if (!bm.live) return;
  const int hi = bm.hi, tile = bm.tile;
  const int64_t hoff = int64_t(heads.h[hi]) * a.stride_h;
  const float *qb = static_cast<const float *>(a.q) + hoff;
  const float *kbase = static_cast<const float *>(a.k) + hoff;
  const float *vbase = static_cast<const float *>(a.v) + hoff;
  const int tid = threadIdx.x;
  const int qi = tid / 2, half = tid % 2;
  const int32_t vc_q = a.valid_count[tile];
  const int32_t qrow = qi < vc_q ? a.perm[int64_t(tile) * VEDA_TILE + qi] : -1;
  float qv[HD], o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qv[d] = qrow >= 0 ? qb[int64_t(qrow) * a.stride_s + half * HD + d] : 0.0f;
    o[d] = 0.0f;
  }
  float m_run = -INFINITY, l_run = 0.0f;
  const int32_t t_begin = a.row_offsets[tile], t_end = a.row_offsets[tile + 1];
  const int32_t *list = a.cols + int64_t(hi) * a.entries_per_head;
  for (int32_t t = t_begin; t < t_end; ++t) {
    const int32_t j = list[t];
    const int32_t vcj = a.valid_count[j];
    const int32_t *pj = a.perm + int64_t(j) * VEDA_TILE;
    for (int c0 = 0; c0 < vcj; c0 += F32_CHUNK) {
      __syncthreads();
      for (int idx = tid; idx < F32_CHUNK * (D / 4); idx += 256) {
        const int r = idx / (D / 4), c4 = idx % (D / 4);
        float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
        if (c0 + r < vcj) {
          const int64_t row = pj[c0 + r];
          kx = *reinterpret_cast<const float4 *>(kbase + row * a.stride_s + c4 * 4);
          vx = *reinterpret_cast<const float4 *>(vbase + row * a.stride_s + c4 * 4);
        }
        ks[r][c4 * 4 + 0] = kx.x; ks[r][c4 * 4 + 1] = kx.y;
        ks[r][c4 * 4 + 2] = kx.z; ks[r][c4 * 4 + 3] = kx.w;
        vs[r][c4 * 4 + 0] = vx.x; vs[r][c4 * 4 + 1] = vx.y;
        vs[r][c4 * 4 + 2] = vx.z; vs[r][c4 * 4 + 3] = vx.w;
      }
      __syncthreads();
      float sc[F32_CHUNK];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < F32_CHUNK; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc = fmaf(qv[d], ks[r][half * HD + d], acc);
        acc += __shfl_xor(acc, 1, 64);
        sc[r] = (c0 + r < vcj) ? acc * a.scale : -INFINITY;
        mx = fmaxf(mx, sc[r]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = expf(m_run - m_new);
      m_run = m_new;
      float rs = 0.0f;
#pragma unroll
      for (int d = 0; d < HD; ++d) o[d] *= alpha;
#pragma unroll
      for (int r = 0; r < F32_CHUNK; ++r) {
        const float p = expf(sc[r] - m_new);
        rs += p;
#pragma unroll
        for (int d = 0; d < HD; ++d) o[d] = fmaf(p, vs[r][half * HD + d], o[d]);
      }
      l_run = l_run * alpha + rs;
    }
  }
  if (qrow < 0) return;
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  float *ob = static_cast<float *>(a.out) + int64_t(qrow) * a.out_stride_s +
              int64_t(heads.h[hi]) * a.out_stride_h + half * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) ob[d] = o[d] * inv;
}

hipError_t launch_attend_f32(const AttendArgs &a, const HeadList &heads, int head_dim,
                             hipStream_t s) {
  const dim3 grid(grid_blocks(a));
  if (head_dim == 128)
    hipLaunchKernelGGL(attend_f32_kernel<128>, grid, dim3(256), 0, s, a, heads);
  else
    hipLaunchKernelGGL(attend_f32_kernel<64>, grid, dim3(256), 0, s, a, heads);
  return hipGetLastError();
}

}  // namespace veda
