// Tile-skip attention (page `veda_core.py`, reference_attend defines the
// result; the pages' own kernel streams only the selected K/V tiles). One
// workgroup per (head, query tile); it walks the query tile's CSR list of
// kept key tiles with an online softmax, reading q/k/v rows through the
// plan's permutation and writing each real query row's output straight to
// its original row (no tile-ordered copies, no scatter pass).
//
// bf16 kernel (MFMA, gfx950): scores are formed transposed, S^T = K Q^T,
//   with v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, the wave's Q
//   held in registers as B), so each lane holds the scores of ONE query row:
//   row max and row sum are in-lane reductions plus one exchange with the
//   lane 32 apart, and the probabilities, converted to bf16, are already laid
//   out as the B operand of O^T += V^T P^T. Details at the kernel.
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
// 8 wavefronts (2 per SIMD): wave w takes query rows 32*(w%4) .. +31 and key
// half w/4 (keys 64*(w/4) .. +63) of every kept tile, with its own online
// softmax state; the two halves are merged through LDS at the end. Two
// waves per SIMD let one wave's softmax (VALU) run while the other's MFMAs
// execute.
//
// K and V tiles are double-buffered in LDS, row-major, each 16-byte chunk c of
// row r stored at chunk position c ^ swz(r) so that both access patterns are
// free of bank conflicts:
//   K: the A operand of S^T = K Q^T, one 16-byte read of 8 d-values per lane
//      for 32 consecutive rows;
//   V: the A operand of O^T += V^T P^T, built by ds_read_b64_tr_b16. Within a
//      16-lane group that instruction hands lane i, element j, the (i%4)-th
//      16-bit value of the 8 bytes addressed by lane i/4 + 4j; with source
//      lane s pointing at row (key) k0 + s/4, columns d0 + 4*(s%4), lane i
//      receives V[k0 + j][d0 + i] for j = 0..3: four keys of one column.
// Tiles are staged through registers: the loads of tile t+2's rows are
// issued while tile t is computed and written to the free buffer one
// iteration later, so no wave waits on a global load it just issued. The
// row ids (perm) are fetched one tile further ahead, one per lane, and
// broadcast within the wave by shuffles.
template <int D>
struct Bf16Cfg {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CHUNKS = D / 8;                        // 16-byte chunks per row
  static constexpr int TILE_BYTES = VEDA_TILE * ROW_BYTES;
  static constexpr int BUF_BYTES = 2 * TILE_BYTES;            // K then V
  static constexpr int LDS_BYTES = 2 * BUF_BYTES;             // double-buffered
  static constexpr int ROWS_PER_LOAD = 64 / CHUNKS;           // rows one 64-lane load covers
  static constexpr int LOADS = 16 / ROWS_PER_LOAD;            // loads per wave per tensor
  static constexpr int DB = D / 32;                           // 32-wide d blocks of O^T
};

template <int D>
__device__ inline int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ inline int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

__device__ inline uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Rows of padding slots read zeros from here, as the page's tile-ordered
// copies hold zeros in padding slots.
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[128] = {};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline s16x4 ds_read_tr(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

template <int D>
__global__ void __launch_bounds__(512, 1) attend_bf16_kernel(AttendArgs a, HeadList heads) {
  using C = Bf16Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

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
  const int qg = wave & 3, kh = wave >> 2;

  // Q fragment (B operand of S^T = K Q^T): q[row][16*ks + 8*g .. +8]
  const int32_t vc_q = a.valid_count[tile];
  const int qi = qg * 32 + l32;
  const int32_t qrow = qi < vc_q ? a.perm[int64_t(tile) * VEDA_TILE + qi] : -1;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qrow >= 0) u = ld16(qb + int64_t(qrow) * a.stride_s + ks * 16 + g * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, u);
  }

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const int32_t t_begin = a.row_offsets[tile], t_end = a.row_offsets[tile + 1];
  const int32_t *list = a.cols + int64_t(hi) * a.entries_per_head;
  const int n_t = t_end - t_begin;

  // Row ids: lane holds perm[j*128 + 16*wave + lane%16] of a tile j.
  auto fetch_rows = [&](int idx) -> int32_t {
    if (idx >= n_t) return -1;
    const int32_t j = list[t_begin + idx];
    return a.perm[int64_t(j) * VEDA_TILE + 16 * wave + (lane & 15)];
  };
  uint4 kreg[C::LOADS], vreg[C::LOADS];
  auto issue_loads = [&](int32_t rows) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int r = C::ROWS_PER_LOAD * i + lane / C::CHUNKS;   // row within the wave's 16
      const int c = lane % C::CHUNKS;
      const int32_t rid = __shfl(rows, r, 64);
      const uint16_t *ks = rid >= 0 ? kb_ + int64_t(rid) * a.stride_s + c * 8 : g_zero_row + c * 8;
      const uint16_t *vs = rid >= 0 ? vb + int64_t(rid) * a.stride_s + c * 8 : g_zero_row + c * 8;
      kreg[i] = ld16(ks);
      vreg[i] = ld16(vs);
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char *kd = lds + buf * C::BUF_BYTES;
    unsigned char *vd = kd + C::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int row = 16 * wave + C::ROWS_PER_LOAD * i + lane / C::CHUNKS;
      const int c = lane % C::CHUNKS;
      *reinterpret_cast<uint4 *>(kd + row * C::ROW_BYTES + ((c ^ swz_k<D>(row)) << 4)) = kreg[i];
      *reinterpret_cast<uint4 *>(vd + row * C::ROW_BYTES + ((c ^ swz_v<D>(row)) << 4)) = vreg[i];
    }
  };

  // prologue: tile 0 staged into buffer 0, tile 1's loads in flight
  int32_t rows_next = fetch_rows(0);
  issue_loads(rows_next);
  rows_next = fetch_rows(1);
  store_tile(0);
  int32_t rows_after = fetch_rows(2);
  if (n_t > 1) issue_loads(rows_next);
  __syncthreads();

  for (int it = 0; it < n_t; ++it) {
    const int buf = it & 1;
    const unsigned char *kd = lds + buf * C::BUF_BYTES;
    const unsigned char *vd = kd + C::TILE_BYTES;
    const int32_t vcj = a.valid_count[list[t_begin + it]];

    // S^T = K Q^T over this wave's 64 keys (two 32-key blocks)
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = kh * 64 + kb * 32 + l32;
        const int c = 2 * ks + g;
        const bf16x8 A = *reinterpret_cast<const bf16x8 *>(
            kd + row * C::ROW_BYTES + ((c ^ swz_k<D>(row)) << 4));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[ks], s[kb], 0, 0, 0);
      }

    // stage tile it+1 into the free buffer (its last readers finished before
    // the barrier that ended the previous iteration), then start tile it+2
    if (it + 1 < n_t) {
      store_tile(buf ^ 1);
      if (it + 2 < n_t) issue_loads(rows_after);
      rows_after = fetch_rows(it + 3);
    }

    if (vcj < VEDA_TILE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kh * 64 + kb * 32 + 8 * (i / 4) + 4 * g + (i % 4);
          if (key >= vcj) s[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale_log2;
    // Lazy rescale: keep the running max unless this tile exceeds it by more
    // than 2^8; probabilities then stay <= 256, exact in fp32 and bf16 range.
    if (mx > m_run + 8.0f) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
      m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    // a key half that has seen only padding keeps m_run = -inf; its scores
    // are all -inf then, and exp2(-inf - 0) = 0 avoids -inf + inf
    const float m_use = m_run == -INFINITY ? 0.0f : m_run;
    float rs = 0.0f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, -m_use));
        rs += p;
        pb[kb][i / 8][i % 8] = static_cast<__bf16>(p);
      }
    l_run += rs + __shfl_xor(rs, 32, 64);

    // O^T += V^T P^T over the wave's 64 keys (4 k-steps of 16)
    const int G = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const int kb = kstep >> 1, e = kstep & 1;
      const int row0 = kh * 64 + kb * 32 + e * 16 + 4 * (G >> 1) + (s16 >> 2);
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int d = db * 32 + 16 * (G & 1) + 4 * (s16 & 3);
        const int c = d >> 3, h8 = (d >> 2) & 1;
        const s16x4 lo = ds_read_tr(vd + row0 * C::ROW_BYTES + ((c ^ swz_v<D>(row0)) << 4) + h8 * 8);
        const int row1 = row0 + 8;
        const s16x4 hi4 = ds_read_tr(vd + row1 * C::ROW_BYTES + ((c ^ swz_v<D>(row1)) << 4) + h8 * 8);
        const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3],
                                                              hi4[0], hi4[1], hi4[2], hi4[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[kb][e],
                                                       o[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Merge the two key halves: waves 4..7 hand (m, l, O^T) to waves 0..3.
  float *xm = reinterpret_cast<float *>(lds);                    // [4][64] m, then [4][64] l
  float *xo = xm + 2 * 4 * 64;                                   // [4][DB*16][64]
  if (kh == 1) {
    xm[qg * 64 + lane] = m_run;
    xm[256 + qg * 64 + lane] = l_run;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) xo[(qg * C::DB * 16 + db * 16 + i) * 64 + lane] = o[db][i];
  }
  __syncthreads();
  if (kh == 1 || qrow < 0) return;
  const float m1 = xm[qg * 64 + lane], l1 = xm[256 + qg * 64 + lane];
  const float m = fmaxf(m_run, m1);
  const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
  const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
  const float l = l_run * a0 + l1 * a1;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  uint16_t *ob = static_cast<uint16_t *>(a.out) + int64_t(qrow) * a.out_stride_s +
                 int64_t(heads.h[hi]) * a.out_stride_h;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int d = db * 32 + 8 * p + 4 * g;
      uint16_t h4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float o1 = xo[(qg * C::DB * 16 + db * 16 + 4 * p + r) * 64 + lane];
        const float v = (o[db][4 * p + r] * a0 + o1 * a1) * inv;
        h4[r] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
      }
      uint2 w;
      w.x = uint32_t(h4[0]) | (uint32_t(h4[1]) << 16);
      w.y = uint32_t(h4[2]) | (uint32_t(h4[3]) << 16);
      *reinterpret_cast<uint2 *>(ob + d) = w;
    }
}

hipError_t launch_attend_bf16(const AttendArgs &a, const HeadList &heads, int head_dim,
                              hipStream_t s) {
  const dim3 grid(grid_blocks(a));
  hipError_t e;
  if (head_dim == 128) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(attend_bf16_kernel<128>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Bf16Cfg<128>::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_bf16_kernel<128>, grid, dim3(512), Bf16Cfg<128>::LDS_BYTES, s, a,
                       heads);
  } else {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(attend_bf16_kernel<64>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Bf16Cfg<64>::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_bf16_kernel<64>, grid, dim3(512), Bf16Cfg<64>::LDS_BYTES, s, a,
                       heads);
  }
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
