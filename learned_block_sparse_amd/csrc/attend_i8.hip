// Tile-skip attention with Q.K^T in int8 (the news pages name the Veda
// kernel an INT8 Triton kernel and call it approximate: comfyui-wiki Veda
// news, "Rendimiento" / "Performances" sections, and the Vflash guide's note
// that the kernel gives no exact-arithmetic guarantee). The result it
// approximates is that of the bf16 kernel (attend.hip): softmax(q.k * scale)
// v over the kept key tiles, output at each query's original row.
//
// Quantisation (symmetric, round to nearest even, no zero point):
//   key tile j of head h: s_k = max |k| over its real rows / 127,
//                         k8 = rint(k / s_k)      (quant_k_kernel, a pre-pass)
//   query row i:          s_q = max |q_i| / 127, q8 = rint(q_i / s_q)
//                                                (in the attend kernel's prologue)
//   logit(i, key r of j) = (q8_i . k8_r) * s_q * s_k * scale
// The integer dot is exact (int32 accumulation: |q8.k8| <= 128 * 127^2 <
// 2^24, so its conversion to fp32 is exact too). A row or tile of zeros gets
// scale 0 and codes 0, and its logits are exactly 0, as they should be.
// Probabilities, row sums, P V and the output are those of the bf16 kernel:
// bf16 probabilities, fp32 accumulation, sums of the same rounded values.
//
// Kernel layout: the bf16 kernel's ping-pong workgroup (two groups of four
// waves, a head pair, four barrier-closed half-phases per kept tile) with
// three changes:
//   - K arrives as int8 rows in tile order from the pre-pass's buffer, so a
//     tile is 128 x D bytes (half the bf16 tile) and is fetched without row
//     ids: one contiguous range per tile, the tile's byte offset a scalar.
//   - S^T = K Q^T runs on v_mfma_i32_32x32x32_i8, which does twice the
//     multiply-adds of v_mfma_f32_32x32x16_bf16 in the same time: half the
//     MFMA work of the S half-phase. Lane l holds A/B operand bytes of row
//     (l % 32), k = 16 (l / 32) + j, j = 0..15; the accumulator layout is
//     that of the bf16 MFMA.
//   - In half-phase A the int32 scores are converted to fp32 and each lane's
//     logits scale by c * s_q * s_k (c = scale * log2 e), a per-lane,
//     per-tile factor, in place of the bf16 kernel's constant c.
#include <hip/hip_runtime.h>

#include "attend_common.hpp"
#include "attend_i8.hpp"

namespace veda {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef const __attribute__((address_space(4))) float const_f32;

template <int D>
struct I8Cfg {
  // K, int8
  static constexpr int KROW = D;                              // bytes per row
  static constexpr int KTILE = VEDA_TILE * KROW;
  static constexpr int KRPL = 1024 / KROW;                    // rows one 64-lane load covers
  static constexpr int NK = 32 / KRPL;                        // K loads per wave per tile
  static constexpr int KCHUNKS = D / 16;                      // 16-byte chunks per row
  static constexpr int KK = D / 32;                           // 32-wide k steps of S^T
  // V, bf16 (as in the bf16 kernel)
  static constexpr int ROW = D * 2;
  static constexpr int TILE_BYTES = VEDA_TILE * ROW;
  static constexpr int ROWS_PER_LOAD = 1024 / ROW;
  static constexpr int NL = 2 * (16 / ROWS_PER_LOAD);         // V loads per wave per tile
  static constexpr int DB = D / 32;
};

// Chunk position of 16-byte chunk c of int8 K row r: c ^ swz8(r). The S
// reads take one chunk position of 32 consecutive rows; 256 bytes of LDS
// (all 64 banks) hold 256 / D rows, and swz8 spreads 16 consecutive rows
// over all 16 16-byte slots of those bytes.
template <int D>
__device__ inline int swz8(int row) {
  return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
// V rows as in the bf16 kernel
template <int D>
__device__ inline int swz_v8(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

__device__ inline const_f32 *as_const_f(const float *p) { return (const_f32 *)(p); }

// int8 code of x * inv, rounded to nearest even, within [-127, 127]
__device__ inline int q8_code(float x, float inv) {
  return int(fminf(fmaxf(rintf(x * inv), -127.0f), 127.0f));
}
__device__ inline uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t(a) & 0xffu) | ((uint32_t(b) & 0xffu) << 8) | ((uint32_t(c) & 0xffu) << 16) |
         (uint32_t(d) << 24);
}
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace

// ------------------------------------------------------------- pre-pass --
// One workgroup (256 threads) per (key tile, head): the tile's 128 rows
// (padding rows as zeros) read through the plan's permutation in 16-byte
// chunks, 16 rows per pass of the workgroup, the tile's absmax reduced over
// the workgroup, then the codes written in tile order (8 bytes per chunk).
template <int D>
__global__ void __launch_bounds__(256) quant_k_kernel(QuantKArgs a, HeadList heads) {
  constexpr int CH = D / 8;                         // bf16 chunks per row
  constexpr int PER = VEDA_TILE * CH / 256;         // chunks per thread
  __shared__ float red[4];
  const int j = blockIdx.x, hi = blockIdx.y;
  const int tid = threadIdx.x;
  const uint16_t *kb = static_cast<const uint16_t *>(a.k) + int64_t(heads.h[hi]) * a.stride_h;
  const int32_t *pj = a.perm + int64_t(j) * VEDA_TILE;
  const int vc = a.valid_count[j];
  uint4 u[PER];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + 256 * i, r = c / CH, ch = c % CH;
    u[i] = make_uint4(0, 0, 0, 0);
    if (r < vc)
      u[i] = *reinterpret_cast<const uint4 *>(kb + int64_t(pj[r]) * a.stride_s + ch * 8);
    const uint32_t w[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (tid % 64 == 0) red[tid / 64] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  const int64_t unit = int64_t(hi) * a.n_tiles + j;
  signed char *out = a.kq + unit * (VEDA_TILE * D);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + 256 * i, r = c / CH, ch = c % CH;
    const uint32_t w[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
    uint2 o;
    o.x = pack4(q8_code(bf16_lo(w[0]), inv), q8_code(bf16_hi(w[0]), inv),
                q8_code(bf16_lo(w[1]), inv), q8_code(bf16_hi(w[1]), inv));
    o.y = pack4(q8_code(bf16_lo(w[2]), inv), q8_code(bf16_hi(w[2]), inv),
                q8_code(bf16_lo(w[3]), inv), q8_code(bf16_hi(w[3]), inv));
    *reinterpret_cast<uint2 *>(out + r * D + ch * 8) = o;
  }
  if (tid == 0) a.kscale[unit] = amax / 127.0f;
}

hipError_t launch_quant_k(const QuantKArgs &a, const HeadList &heads, hipStream_t s) {
  const dim3 grid(a.n_tiles, a.n_heads);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(quant_k_kernel<128>, grid, dim3(256), 0, s, a, heads);
  else
    hipLaunchKernelGGL(quant_k_kernel<64>, grid, dim3(256), 0, s, a, heads);
  return hipGetLastError();
}

// --------------------------------------------------------------- attend --
template <int D, int GROUP>
__device__ __attribute__((always_inline)) inline void attend_i8_group(
    const AttendArgs &a, const HeadList &heads, const signed char *kq, const float *kscale,
    int32_t pair, int32_t tile, int wave) {
  using C = I8Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char Kb[C::KTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char Vb[C::TILE_BYTES];

  // The second group of the last pair of an odd head count repeats the first
  // group's head (it keeps the schedule) and writes nothing.
  const int32_t hi_raw = 2 * pair + GROUP;
  const bool shadow = hi_raw >= a.n_heads;
  const int32_t hi = shadow ? hi_raw - 1 : hi_raw;
  const int64_t hoff = int64_t(heads.h[hi]) * a.stride_h;
  const uint16_t *qb = static_cast<const uint16_t *>(a.q) + hoff;
  // this head's int8 K tiles: n_tiles x 128 x D bytes (below 2^31, host-checked)
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<signed char *>(kq + int64_t(hi) * a.n_tiles * C::KTILE), 0,
      a.n_tiles * C::KTILE, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(static_cast<const uint16_t *>(a.v) + hoff), 0, int(a.kv_bytes), 0x00020000);
  const uint32_t row_bytes = uint32_t(a.stride_s) * 2u;
  const const_f32 *sk_of = as_const_f(kscale + int64_t(hi) * a.n_tiles);

  const int lane = threadIdx.x % 64;
  const int g = lane / 32, l32 = lane % 32;

  // Q row of this lane (query 32 wave + l32), the half d = 32 kk + 16 g + j:
  // its absmax with the other half's (lane l32 + 32) gives s_q, then the
  // codes form the B operand of S^T = K Q^T.
  const int32_t vc_q = a.valid_count[tile];
  const int qi = wave * 32 + l32;
  const int32_t qrow = qi < vc_q ? a.perm[int64_t(tile) * VEDA_TILE + qi] : -1;
  i32x4 qf[C::KK];
  float qlog2;   // c * s_q: this lane's logit factor before the key tile's s_k
  {
    uint4 u[C::KK][2];
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u[kk][h] = make_uint4(0, 0, 0, 0);
        if (qrow >= 0) u[kk][h] = ld16(qb + int64_t(qrow) * a.stride_s + 32 * kk + 16 * g + 8 * h);
        const uint32_t w[4] = {u[kk][h].x, u[kk][h].y, u[kk][h].z, u[kk][h].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
      }
    amax = pair_max(amax);
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    qlog2 = (amax / 127.0f) * a.scale_log2;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {u[kk][h].x, u[kk][h].y, u[kk][h].z, u[kk][h].w};
        qf[kk][2 * h] = int(pack4(q8_code(bf16_lo(w[0]), inv), q8_code(bf16_hi(w[0]), inv),
                                  q8_code(bf16_lo(w[1]), inv), q8_code(bf16_hi(w[1]), inv)));
        qf[kk][2 * h + 1] = int(pack4(q8_code(bf16_lo(w[2]), inv), q8_code(bf16_hi(w[2]), inv),
                                      q8_code(bf16_lo(w[3]), inv), q8_code(bf16_hi(w[3]), inv)));
      }
  }

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float m_run = -INFINITY;
  // Row sums of the bf16-rounded probabilities (v_dot2_f32_bf16 with (1, 1))
  // in the P V half-phase, as in the bf16 kernel.
  float racc[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  const int32_t t_begin = a.row_offsets[tile], t_end = a.row_offsets[tile + 1];
  const const_i32 *list = as_const(a.cols + int64_t(hi) * a.entries_per_head);
  const const_i32 *vcount = as_const(a.valid_count);
  const int n_t = t_end - t_begin;

  // Load mapping. K: wave w fills rows 32w .. 32w+31 with NK loads; load i
  // lands at bytes (32w + KRPL i) KROW + 16 lane, i.e. row 32w + KRPL i +
  // lane / KCHUNKS, chunk position lane % KCHUNKS, and fetches the chunk
  // that belongs there from the tile-ordered buffer (tile j at scalar offset
  // j * KTILE). V: as in the bf16 kernel, through the row ids.
  const int kld_row = lane / C::KCHUNKS, kld_pos = lane % C::KCHUNKS;
  uint32_t k_src[C::NK];
#pragma unroll
  for (int i = 0; i < C::NK; ++i) {
    const int row = 32 * wave + C::KRPL * i + kld_row;
    k_src[i] = uint32_t(row * C::KROW + 16 * (kld_pos ^ swz8<D>(row)));
  }
  const int ld_row = lane / (D / 8), ld_pos = lane % (D / 8);
  uint32_t v_chunk[C::NL];
#pragma unroll
  for (int i = 0; i < C::NL; ++i) {
    const int row = 32 * wave + C::ROWS_PER_LOAD * i + ld_row;
    v_chunk[i] = 16u * uint32_t(ld_pos ^ swz_v8<D>(row));
  }
  struct Rows {
    int32_t r[C::NL];
  };
  auto list_at = [&](int idx) -> int32_t { return list[t_begin + min(idx, n_t - 1)]; };
  auto rows_of = [&](int32_t j) {
    Rows out;
    const int32_t *pj = a.perm + int64_t(j) * VEDA_TILE + 32 * wave + ld_row;
#pragma unroll
    for (int i = 0; i < C::NL; ++i) out.r[i] = pj[C::ROWS_PER_LOAD * i];
    return out;
  };
  auto dma_k = [&](int32_t j, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rk, (lds_void *)(Kb + (32 * wave + C::KRPL * i) * C::KROW), 16, k_src[i],
        j * C::KTILE, 0, 0);
  };
  // a padding row (id -1) is fetched as row pad_row, past the descriptor's
  // range: zeros (as in the bf16 kernel)
  auto dma_v = [&](int32_t row, int i) {
    const uint32_t r = min(uint32_t(row), a.pad_row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rv, (lds_void *)(Vb + (32 * wave + C::ROWS_PER_LOAD * i) * C::ROW), 16,
        __umul24(r, row_bytes) + v_chunk[i], 0, 0, 0);
  };

  // S reads: row kb*32 + l32, chunk 2 kk + g (swz8 depends on l32 only)
  const uint32_t k_sw = uint32_t(swz8<D>(l32));
  auto k_off = [&](int kk) -> uint32_t {
    return uint32_t(l32 * C::KROW) + 16u * ((uint32_t(2 * kk + g)) ^ k_sw);
  };
  const int G = lane >> 4, s16 = lane & 15;
  const int vrow = 4 * (G >> 1) + (s16 >> 2);
  const int vcol = 16 * (G & 1) + 4 * (s16 & 3);
  uint32_t v_off[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int d = db * 32 + vcol;
    v_off[db] = uint32_t(vrow * C::ROW) + 16u * uint32_t((d >> 3) ^ swz_v8<D>(vrow)) + 8u * ((d >> 2) & 1);
  }

  i32x16 si[4];
  f32x16 s[4];
  bf16x8 pb[4][2];
  // S^T = K Q^T in int32 for the key tile in Kb, the reads of each k step
  // issued one step ahead of its MFMAs, the V loads of `rows` spread over
  // the k steps (NL / KK per step).
  auto scores_with_v = [&](const Rows &rows) {
    constexpr int VPS = C::NL / C::KK;
    i32x4 A[2][4];
    auto read_k = [&](int kk, i32x4 (&dst)[4]) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        dst[kb] = *reinterpret_cast<const i32x4 *>(Kb + k_off(kk) + kb * 32 * C::KROW);
    };
    read_k(0, A[0]);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      if (kk + 1 < C::KK) read_k(kk + 1, A[(kk + 1) & 1]);
#pragma unroll
      for (int v = 0; v < VPS; ++v) dma_v(rows.r[VPS * kk + v], VPS * kk + v);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        si[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[kk & 1][kb], qf[kk],
                                                       kk == 0 ? i32x16{} : si[kb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      if (kk + 1 < C::KK) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, VPS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };
  auto scores = [&]() {
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const i32x4 A = *reinterpret_cast<const i32x4 *>(Kb + k_off(kk) + kb * 32 * C::KROW);
        si[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, qf[kk], kk == 0 ? i32x16{} : si[kb], 0,
                                                       0, 0);
      }
  };
  // lane factor of the current tile: c s_q s_k, kept above zero so that a
  // masked key (-inf) never meets a zero factor
  float f_cur = 0.0f;
  auto exps8 = [&](int kb, int h) {
#pragma unroll
    for (int i = 8 * h; i < 8 * h + 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], f_cur, -m_run));
      pb[kb][h][i % 8] = static_cast<__bf16>(p);
    }
  };
  // Probabilities are formed in chunks of 8 per lane, chunk e holding block
  // e / 2, half e % 2: A forms chunks 0 .. A_CHUNKS-1, B the rest.
  constexpr int A_CHUNKS = 2;
  // Reference value m_run: as in the bf16 kernel, the first tile's row max,
  // raised only when a later tile's row max passes it by more than RAISE.
  constexpr float RAISE = 20.0f;
  auto s_max = [&]() {
    float mx4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx4[i & 3] = fmaxf(mx4[i & 3], s[kb][i]);
    return pair_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
  };

  // Schedule: the bf16 kernel's four half-phases per kept tile t, the two
  // groups two half-phases apart:
  //   A: scores(t) to fp32, mask, row max and the rare raise, probabilities
  //      of keys 0..31; K(t+1) loads spread through it
  //   B: probabilities of keys 32..127
  //   C: P(t) V(t) and the row sums; the row ids of tile t+1 loaded first
  //   D: S(t+1) = K(t+1) Q^T in int8, V(t+1) loads spread through it
  // Every load is issued unconditionally (past the end of the list the last
  // tile again), so the barriers wait with exact counts. In issue order:
  // K(t+1) (NK, in A), row ids of t+1 (NL, in C), V(t+1) (NL, in D), K(t+2)
  // (next A), ... The end of B waits for V(t) with K(t+1) allowed in
  // flight, the end of C for K(t+1) with the row ids allowed in flight.
  if (n_t > 0) {
  {
    const int32_t j0 = list_at(0);
#pragma unroll
    for (int i = 0; i < C::NK; ++i) dma_k(j0, i);
    asm volatile("" ::: "memory");
    const Rows R0 = rows_of(j0);
#pragma unroll
    for (int i = 0; i < C::NL; ++i) dma_v(R0.r[i], i);
  }
  if constexpr (GROUP == 0) {
    barrier_vm<0>();
    scores();
    barrier_lds();
  } else {
    barrier_lds();
    barrier_lds();
    barrier_vm<0>();
    scores();
    barrier_lds();
  }
  int32_t vc_cur = vcount[list_at(0)];
  float sk_cur = sk_of[list_at(0)];
  int32_t j1 = list_at(1);   // tile t+1

  for (int t = 0; t < n_t; ++t) {
    const int32_t j2 = list_at(t + 2);
    const int32_t vc_next = vcount[j1];
    const float sk_next = sk_of[j1];
    __builtin_amdgcn_s_setprio(0);   // vector half-phases yield to the other group's MFMAs
    // ---- A
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = float(si[kb][i]);
    if (vc_cur < VEDA_TILE) {
      asm volatile("" ::: "memory");
      const int g4 = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5) * 4;
      const int thr = vc_cur - g4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i / 4) + (i % 4) >= thr) s[kb][i] = -INFINITY;
    }
    f_cur = fmaxf(qlog2 * sk_cur, 1e-30f);
    {
      const float xm = s_max() * f_cur;   // this tile's row max, log2 units
      if (t == 0) {
        m_run = xm;
      } else if (__builtin_amdgcn_ballot_w64(xm > m_run + RAISE) != 0) {   // rare
        const float d = fmaxf(0.0f, xm - m_run);
        const float alpha = __builtin_amdgcn_exp2f(-d);
        m_run += d;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) racc[i] *= alpha;
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int i = c * C::NK / 2; i < (c + 1) * C::NK / 2; ++i) dma_k(j1, i);
      __builtin_amdgcn_sched_barrier(0);
      exps8(0, c);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 2; e < A_CHUNKS; ++e) exps8(e / 2, e % 2);
    barrier_lds();
    // ---- B
#pragma unroll
    for (int e = A_CHUNKS; e < 8; ++e) exps8(e / 2, e % 2);
    barrier_vm<C::NK>();   // V(t) landed in every wave (K(t+1) may not)
    const Rows Rv = rows_of(j1);
    __builtin_amdgcn_s_setprio(1);   // MFMA half-phases issue first
    // ---- C
    {
      constexpr int NM = 8 * C::DB;
      constexpr int LA_PV = 4;
      s16x4 Vf[LA_PV + 1][2];
      auto read_v1 = [&](int j, s16x4 (&dst)[2]) {
        const int kstep = j / C::DB, db = j % C::DB;
        const int kb = kstep >> 1, e = kstep & 1;
        const unsigned char *p0 = Vb + v_off[db] + (kb * 32 + e * 16) * C::ROW;
        dst[0] = ds_read_tr(p0);
        dst[1] = ds_read_tr(p0 + 8 * C::ROW);
      };
#pragma unroll
      for (int j = 0; j < LA_PV; ++j) read_v1(j, Vf[j]);
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        if (j + LA_PV < NM) read_v1(j + LA_PV, Vf[(j + LA_PV) % (LA_PV + 1)]);
        const int kstep = j / C::DB, db = j % C::DB;
        const int kb = kstep >> 1, e = kstep & 1;
        const s16x4 lo = Vf[j % (LA_PV + 1)][0], hi4 = Vf[j % (LA_PV + 1)][1];
        const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3],
                                                              hi4[0], hi4[1], hi4[2], hi4[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8),
                                                       pb[kb][e], o[db], 0, 0, 0);
        if (db == C::DB - 1) {
          const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            racc[jj] = __builtin_amdgcn_fdot2_f32_bf16(
                bf16x2{pb[kb][e][2 * jj], pb[kb][e][2 * jj + 1]}, one, racc[jj], false);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA_PV, 0);
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        if (j + LA_PV < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        // the row sums' dot products in two runs of 16, half-way through
        // and at the end of the MFMAs, rather than 4 after every k step:
        // fewer switches between MFMA and vector issue (1-3% faster than
        // runs of 4 or 8; one per MFMA is 6% slower)
        if (j % (4 * C::DB) == 4 * C::DB - 1) __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
      }
    }
    barrier_vm<C::NL>();   // K(t+1) landed; every wave is done with V(t)
    // ---- D
    __builtin_amdgcn_sched_barrier(0);
    scores_with_v(Rv);
    barrier_lds();     // every wave is done with K(t+1)
    vc_cur = vc_next;
    sk_cur = sk_next;
    j1 = j2;
  }
  if constexpr (GROUP == 0) {
    barrier_lds();
    barrier_lds();
  }
  // the loads past the end of the list must land before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  const float l_run = pair_sum((racc[0] + racc[1]) + (racc[2] + racc[3]));
  if (qrow < 0 || shadow) return;
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  uint16_t *ob = static_cast<uint16_t *>(a.out) + int64_t(qrow) * a.out_stride_s +
                 int64_t(heads.h[hi]) * a.out_stride_h;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
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

template <int D>
__global__ void __launch_bounds__(512, 1) attend_i8_kernel(AttendArgs a, HeadList heads,
                                                           const signed char *kq,
                                                           const float *kscale) {
  const int32_t n_pairs = (a.n_heads + 1) / 2;
  const BlockMap bm = map_block(a, n_pairs, blockIdx.x);
  if (!bm.live) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  if (wave >= 4)
    attend_i8_group<D, 0>(a, heads, kq, kscale, bm.hi, bm.tile, wave - 4);
  else
    attend_i8_group<D, 1>(a, heads, kq, kscale, bm.hi, bm.tile, wave);
}

hipError_t launch_attend_i8(const AttendArgs &a, const HeadList &heads, int head_dim,
                            const signed char *kq, const float *kscale, hipStream_t s) {
  const dim3 grid(grid_blocks(a, (a.n_heads + 1) / 2));
  if (head_dim == 128)
    hipLaunchKernelGGL(attend_i8_kernel<128>, grid, dim3(512), 0, s, a, heads, kq, kscale);
  else
    hipLaunchKernelGGL(attend_i8_kernel<64>, grid, dim3(512), 0, s, a, heads, kq, kscale);
  return hipGetLastError();
}

}  // namespace veda
