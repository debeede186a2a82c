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
// softmax state; the two halves are merged through LDS at the end.
//
// K and V tiles arrive in LDS by direct buffer-to-LDS loads (no register
// staging) into four separate arrays K0, K1, V0, V1 (double buffers). Such a
// load writes 64 lanes x 16 bytes contiguously, so rows are stored unpadded
// and each 16-byte chunk c of row r sits at chunk position c ^ swz(r), which
// keeps both read patterns free of bank conflicts (64 banks):
//   K: the A operand of S^T = K Q^T, one 16-byte read of 8 d-values per lane
//      across 32 consecutive rows (swz spreads 16 consecutive rows over all
//      16 positions);
//   V: the A operand of O^T += V^T P^T, built by ds_read_b64_tr_b16. Within a
//      16-lane group that instruction hands lane i, element j, the (i%4)-th
//      16-bit value of the 8 bytes addressed by lane i/4 + 4j; with source
//      lane s pointing at row (key) k0 + s/4, columns d0 + 4*(s%4), lane i
//      receives V[k0 + j][d0 + i] for j = 0..3: four keys of one column (swz
//      gives the four rows of a read disjoint chunk positions).
// Rows are fetched with 32-bit offsets from a per-head buffer descriptor; a
// padding slot gets an offset past the descriptor's range, which the
// hardware returns as zeros (the page's tile-ordered copies hold zeros in
// padding slots).
template <int D>
struct Bf16Cfg {
  static constexpr int ROW = D * 2;                          // bytes per row
  static constexpr int TILE_BYTES = VEDA_TILE * ROW;
  static constexpr int ROWS_PER_LOAD = 1024 / ROW;           // rows one 64-lane load covers
  static constexpr int LOADS = 16 / ROWS_PER_LOAD;           // loads per wave per tensor
  static constexpr int CHUNKS = D / 8;                       // 16-byte chunks per row
  static constexpr int DB = D / 32;                          // 32-wide d blocks of O^T
  static constexpr int KS = D / 16;                          // 16-wide k steps of S^T
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Exchange with the lane 32 apart through v_permlane32_swap (VALU; no LDS
// round trip): with both operands x, the two results hold x from each half,
// so their max / sum is the same in lanes l and l + 32.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline s16x4 ds_read_tr(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

template <int D>
__global__ void __launch_bounds__(512, 1) attend_bf16_kernel(AttendArgs a, HeadList heads) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char K0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char K1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char V0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char V1[C::TILE_BYTES];

  const BlockMap bm = map_block(a, blockIdx.x);
  if (!bm.live) return;
  const int hi = bm.hi, tile = bm.tile;
  const int64_t hoff = int64_t(heads.h[hi]) * a.stride_h;
  const uint16_t *qb = static_cast<const uint16_t *>(a.q) + hoff;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(static_cast<const uint16_t *>(a.k) + hoff), 0, int(a.kv_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(static_cast<const uint16_t *>(a.v) + hoff), 0, int(a.kv_bytes), 0x00020000);
  const uint32_t row_bytes = uint32_t(a.stride_s) * 2u;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // scalar: LDS bases stay in SGPRs
  const int lane = tid % 64;
  const int g = lane / 32, l32 = lane % 32;
  const int qg = wave & 3, kh = wave >> 2;

  // Q fragment (B operand of S^T = K Q^T): q[row][16*ks + 8*g .. +8]
  const int32_t vc_q = a.valid_count[tile];
  const int qi = qg * 32 + l32;
  const int32_t qrow = qi < vc_q ? a.perm[int64_t(tile) * VEDA_TILE + qi] : -1;
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
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

  // Load mapping: wave w fills rows 16w .. 16w+15 of a tile with LOADS
  // direct loads per tensor; load i lands at bytes (16w + R*i)*ROW + 16*lane
  // (R = rows per load), i.e. row 16w + R*i + lane/CHUNKS, chunk position
  // lane%CHUNKS, which holds global chunk position ^ swz(row).
  const int ld_row = lane / C::CHUNKS, ld_pos = lane % C::CHUNKS;
  uint32_t k_chunk[C::LOADS], v_chunk[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int row = 16 * wave + C::ROWS_PER_LOAD * i + ld_row;
    k_chunk[i] = 16u * uint32_t(ld_pos ^ swz_k<D>(row));
    v_chunk[i] = 16u * uint32_t(ld_pos ^ swz_v<D>(row));
  }
  // Row ids of the LOADS rows this lane fetches in a tile (-1 on padding).
  struct Rows {
    int32_t r[C::LOADS];
  };
  auto rows_of = [&](int32_t j) {
    Rows out;
    const int32_t *pj = a.perm + int64_t(j) * VEDA_TILE + 16 * wave + ld_row;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) out.r[i] = pj[C::ROWS_PER_LOAD * i];
    return out;
  };
  // Byte offsets are formed only when the loads are issued, an iteration
  // after the row ids were fetched, so fetching row ids never stalls a wave.
  // A padding row (id -1) gives 2^32 - row_bytes + chunk, past the
  // descriptor's range (the host keeps row_bytes <= 2^29, every chunk below
  // row_bytes and the range below 0xE0000000), so it reads as zeros.
  auto dma = [&](const __amdgpu_buffer_rsrc_t &rsrc, unsigned char *dst, const Rows &rows,
                 const uint32_t (&chunk)[C::LOADS]) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const uint32_t off = uint32_t(rows.r[i]) * row_bytes + chunk[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_void *)(dst + (16 * wave + C::ROWS_PER_LOAD * i) * C::ROW), 16, off, 0, 0, 0);
    }
  };

  // Compute-side read offsets (per lane; swizzled positions).
  // K: row kh*64 + kb*32 + l32, chunk 2ks + g -> position (2ks + g) ^ swz(row);
  // swz(row) depends only on l32, so the offset is base ^ (32 ks) per k step.
  const int krow = kh * 64 + l32;
  const uint32_t k_base = uint32_t(krow * C::ROW);
  const uint32_t k_sw = uint32_t(swz_k<D>(krow));
  uint32_t k_off[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) k_off[ks] = k_base + 16u * ((uint32_t(2 * ks + g)) ^ k_sw);
  // V: rows kh*64 + kb*32 + e*16 + 4*(G/2) + s16/4 (+8 for the upper four
  // keys), columns db*32 + 16*(G%2) + 4*(s16%4).
  const int G = lane >> 4, s16 = lane & 15;
  const int vrow = kh * 64 + 4 * (G >> 1) + (s16 >> 2);
  const int vcol = 16 * (G & 1) + 4 * (s16 & 3);
  uint32_t v_off[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int d = db * 32 + vcol;
    v_off[db] = uint32_t(vrow * C::ROW) + 16u * uint32_t((d >> 3) ^ swz_v<D>(vrow)) + 8u * ((d >> 2) & 1);
  }

  // List positions past the end read the last entry again: the extra tiles
  // are loaded and discarded, which keeps the pipeline free of branches.
  auto list_at = [&](int idx) -> int32_t { return list[t_begin + min(idx, n_t - 1)]; };

  // S^T = K Q^T over this wave's 64 keys of the tile in `kbuf`
  auto scores = [&](const unsigned char *kbuf, f32x16 (&sn)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[kb][i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 A = *reinterpret_cast<const bf16x8 *>(kbuf + k_off[ks] + kb * 32 * C::ROW);
        sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[ks], sn[kb], 0, 0, 0);
      }
  };

  // Pipeline. At the top of iteration t (after a barrier): S(t) is in
  // registers, K(t+1) and V(t) are in LDS (K buffer (t+1)%2, V buffer t%2),
  // and the row ids of tiles t+1 and t+2 are known. Iteration t starts the
  // loads of K(t+2) into K buffer t%2 (last read by S(t), an iteration ago)
  // and V(t+1) into V buffer (t+1)%2 (last read by P(t-1)V(t-1)), forms S(t+1)
  // interleaved with the softmax of tile t, then P(t)V(t), and fetches the
  // row ids of tile t+3. The barrier closing the iteration waits for its own
  // loads, so they have the whole iteration to land.
  f32x16 sA[2], sB[2];
  Rows rows1 = rows_of(list_at(1)), rows2 = rows_of(list_at(2));
  {
    const Rows rows0 = rows_of(list_at(0));
    dma(rk, K0, rows0, k_chunk);
    dma(rv, V0, rows0, v_chunk);
    dma(rk, K1, rows1, k_chunk);
    __syncthreads();
    scores(K0, sA);
  }
  int32_t j3 = list_at(3);
  int32_t vc0 = a.valid_count[list_at(0)], vc1 = a.valid_count[list_at(1)],
          vc2 = a.valid_count[list_at(2)];
  __syncthreads();

  auto iteration = [&](const int t, unsigned char *kn, unsigned char *kfree,
                       const unsigned char *vcur, unsigned char *vfree, f32x16 (&sc)[2],
                       f32x16 (&sn)[2]) {
    dma(rk, kfree, rows2, k_chunk);
    dma(rv, vfree, rows1, v_chunk);
    rows1 = rows2;
    rows2 = rows_of(j3);
    const int32_t vc_new = a.valid_count[j3];
    j3 = list_at(t + 4);

    // mask padding keys of tile t (only partial tiles; the empty asm keeps
    // the branch from being flattened into selects on every tile)
    if (vc0 < VEDA_TILE) {
      asm volatile("" ::: "memory");
      // key kh*64 + 4g + (kb*32 + 8(i/4) + i%4) is padding when the constant
      // part reaches vc0 - (kh*64 + 4g)
      const int thr = vc0 - (kh * 64 + 4 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i / 4) + (i % 4) >= thr) sc[kb][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = pair_max(mx) * a.scale_log2;
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

    // S(t+1): independent of the softmax below, so its MFMAs overlap it
    scores(kn, sn);

    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], a.scale_log2, -m_use));
        pb[kb][i / 8][i % 8] = static_cast<__bf16>(p);
      }
    // row sum of the bf16 probabilities that enter P V
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const bf16x2 pr = {pb[kb][e][2 * q2], pb[kb][e][2 * q2 + 1]};
          rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
        }
    l_run += pair_sum(rs);

    // O^T += V^T P^T over the wave's 64 keys of tile t (4 k-steps of 16)
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const int kb = kstep >> 1, e = kstep & 1;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const unsigned char *p0 = vcur + v_off[db] + (kb * 32 + e * 16) * C::ROW;
        const s16x4 lo = ds_read_tr(p0);
        const s16x4 hi4 = ds_read_tr(p0 + 8 * C::ROW);
        const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3],
                                                              hi4[0], hi4[1], hi4[2], hi4[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[kb][e],
                                                       o[db], 0, 0, 0);
      }
    }
    vc0 = vc1;
    vc1 = vc2;
    vc2 = vc_new;
    // Instruction order for the block above: each S(t+1) MFMA with the read
    // of a K fragment and a few softmax VALU ops, then each P V MFMA with its
    // two transposed reads. Groups: 0x100 LDS read, 0x008 MFMA, 0x002 VALU.
    // LDS reads run ahead of the MFMAs that consume them (four K fragments
    // first; the spare read slots of the S phase start on V fragments).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * C::KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 4 * C::DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
    __syncthreads();
  };

  int t = 0;
  for (; t + 1 < n_t; t += 2) {
    iteration(t, K1, K0, V0, V1, sA, sB);
    iteration(t + 1, K0, K1, V1, V0, sB, sA);
  }
  if (t < n_t) iteration(t, K1, K0, V0, V1, sA, sB);

  // Merge the two key halves: waves 4..7 hand (m, l, O^T) to waves 0..3,
  // through K0/K1 (O^T, 16 KB per wave) and V0 (m, l).
  float *xm = reinterpret_cast<float *>(V0) + qg * 128;
  float *xo = reinterpret_cast<float *>((qg < 2 ? K0 : K1) + (qg & 1) * (C::DB * 16 * 64 * 4));
  if (kh == 1) {
    xm[lane] = m_run;
    xm[64 + lane] = l_run;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) xo[(db * 16 + i) * 64 + lane] = o[db][i];
  }
  __syncthreads();
  if (kh == 1 || qrow < 0) return;
  const float m1 = xm[lane], l1 = xm[64 + lane];
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
        const float o1 = xo[(db * 16 + 4 * p + r) * 64 + lane];
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
  if (head_dim == 128)
    hipLaunchKernelGGL(attend_bf16_kernel<128>, grid, dim3(512), 0, s, a, heads);
  else
    hipLaunchKernelGGL(attend_bf16_kernel<64>, grid, dim3(512), 0, s, a, heads);
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
