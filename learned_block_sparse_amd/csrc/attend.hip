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
#include <hip/hip_runtime.h>

#include "attend_common.hpp"

namespace veda {

// --------------------------------------------------------------- bf16 MFMA --
// One workgroup of 8 wavefronts per CU, in two groups of 4 that take the same
// query tile for a pair of heads (the tile lists of every head have the same
// length, so both groups run the same number of steps). Within a group, wave
// w takes query rows 32w .. 32w+31 and all 128 keys of every kept tile, so it
// owns its rows' softmax state outright. Waves w and w+4 share a SIMD; the
// groups run the same four half-phases per tile two half-phases apart, so on
// every SIMD one group's MFMAs (S and P V) meet the other's vector work (the
// softmax). Workgroup barriers close the half-phases and keep that offset.
//
// K and V tiles arrive in LDS by direct buffer-to-LDS loads (no register
// staging) into one K and one V array per group. Such a load writes 64
// lanes x 16 bytes contiguously, so rows are stored unpadded and each
// 16-byte chunk c of row r sits at chunk position c ^ swz(r), which keeps
// both read patterns free of bank conflicts (64 banks):
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
// padding slot is fetched as the row one past the last, outside the
// descriptor's range, which the hardware returns as zeros (the page's
// tile-ordered copies hold zeros in padding slots).
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

// One group (4 waves) of the ping-pong workgroup; GROUP selects its LDS
// buffers and its place in the schedule.
template <int D, int GROUP>
__device__ __attribute__((always_inline)) inline void attend_group(const AttendArgs &a,
                                                                   const HeadList &heads,
                                                                   int32_t pair, int32_t tile,
                                                                   int wave) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char Kb[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char Vb[C::TILE_BYTES];

  // The second group of the last pair of an odd head count repeats the first
  // group's head (it keeps the schedule) and writes nothing.
  const int32_t hi_raw = 2 * pair + GROUP;
  const bool shadow = hi_raw >= a.n_heads;
  const int32_t hi = shadow ? hi_raw - 1 : hi_raw;
  const int64_t hoff = int64_t(heads.h[hi]) * a.stride_h;
  const uint16_t *qb = static_cast<const uint16_t *>(a.q) + hoff;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(static_cast<const uint16_t *>(a.k) + hoff), 0, int(a.kv_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(static_cast<const uint16_t *>(a.v) + hoff), 0, int(a.kv_bytes), 0x00020000);
  const uint32_t row_bytes = uint32_t(a.stride_s) * 2u;

  const int lane = threadIdx.x % 64;
  const int g = lane / 32, l32 = lane % 32;

  // Q fragment (B operand of S^T = K Q^T): q[row][16*ks + 8*g .. +8]
  const int32_t vc_q = a.valid_count[tile];
  const int qi = wave * 32 + l32;
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
  float m_run = -INFINITY;
  // Row sums add, in fp32, exactly the bf16-rounded probabilities the P V
  // product uses (v_dot2_f32_bf16 of each packed pair with (1, 1)), so the
  // numerator and the denominator of the softmax agree: a probability's
  // rounding then moves both alike. They are accumulated in the P V
  // half-phase, four partial sums per lane over this lane's keys; lanes l and
  // l + 32 hold the two halves of query l % 32's keys.
  float racc[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  const int32_t t_begin = a.row_offsets[tile], t_end = a.row_offsets[tile + 1];
  const const_i32 *list = as_const(a.cols + int64_t(hi) * a.entries_per_head);
  const const_i32 *vcount = as_const(a.valid_count);
  const int n_t = t_end - t_begin;

  // Load mapping: wave w fills rows 32w .. 32w+31 of a tile with NL direct
  // loads per tensor; load i lands at bytes (32w + R*i)*ROW + 16*lane
  // (R = rows per load), i.e. row 32w + R*i + lane/CHUNKS, chunk position
  // lane%CHUNKS, which holds global chunk position ^ swz(row).
  constexpr int NL = 2 * C::LOADS;
  const int ld_row = lane / C::CHUNKS, ld_pos = lane % C::CHUNKS;
  uint32_t k_chunk[NL], v_chunk[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int row = 32 * wave + C::ROWS_PER_LOAD * i + ld_row;
    k_chunk[i] = 16u * uint32_t(ld_pos ^ swz_k<D>(row));
    v_chunk[i] = 16u * uint32_t(ld_pos ^ swz_v<D>(row));
  }
  struct Rows {
    int32_t r[NL];
  };
  auto list_at = [&](int idx) -> int32_t { return list[t_begin + min(idx, n_t - 1)]; };
  auto rows_of = [&](int32_t j) {
    Rows out;
    const int32_t *pj = a.perm + int64_t(j) * VEDA_TILE + 32 * wave + ld_row;
#pragma unroll
    for (int i = 0; i < NL; ++i) out.r[i] = pj[C::ROWS_PER_LOAD * i];
    return out;
  };
  // A padding row (id -1) is clamped to seq_len, one row past the end: its
  // offset is past the descriptor's range (the host keeps seq_len and the
  // row pitch below 2^24, so the 24-bit product is exact), so it reads as
  // zeros.
  auto dma1 = [&](const __amdgpu_buffer_rsrc_t &rsrc, unsigned char *dst, int32_t row, int i,
                  uint32_t chunk) {
    const uint32_t r = min(uint32_t(row), a.pad_row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (lds_void *)(dst + (32 * wave + C::ROWS_PER_LOAD * i) * C::ROW), 16,
        __umul24(r, row_bytes) + chunk, 0, 0, 0);
  };

  // Compute-side read offsets (per lane; swizzled positions).
  const uint32_t k_sw = uint32_t(swz_k<D>(l32));
  // chunk (2ks + g) ^ k_sw = 2 (ks ^ (k_sw >> 1)) + (g ^ (k_sw & 1)): one
  // xor-add per k step instead of KS live registers
  const uint32_t k_base = uint32_t(l32 * C::ROW) + 16u * (uint32_t(g) ^ (k_sw & 1u));
  const uint32_t k_h32 = 32u * (k_sw >> 1);
  auto k_off = [&](int ks) -> uint32_t { return k_base + ((32u * uint32_t(ks)) ^ k_h32); };
  const int G = lane >> 4, s16 = lane & 15;
  const int vrow = 4 * (G >> 1) + (s16 >> 2);
  const int vcol = 16 * (G & 1) + 4 * (s16 & 3);
  uint32_t v_off[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int d = db * 32 + vcol;
    v_off[db] = uint32_t(vrow * C::ROW) + 16u * uint32_t((d >> 3) ^ swz_v<D>(vrow)) + 8u * ((d >> 2) & 1);
  }

  f32x16 s[4];
  bf16x8 pb[4][2];
  // S^T = K Q^T for the key tile in Kb, the reads of each k step issued one
  // step ahead of its MFMAs; the V loads of `rows` (NL of them) are spread
  // over the k steps, between the MFMAs, so no wave waits on the address
  // unit's queue.
  auto scores_with_v = [&](const Rows &rows) {
    bf16x8 A[2][4];
    auto read_k = [&](int ks, bf16x8 (&dst)[4]) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        dst[kb] = *reinterpret_cast<const bf16x8 *>(Kb + k_off(ks) + kb * 32 * C::ROW);
    };
    read_k(0, A[0]);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (ks + 1 < C::KS) read_k(ks + 1, A[(ks + 1) & 1]);
      if (ks % (C::KS / NL) == 0) {
        const int i = ks / (C::KS / NL);
        dma1(rv, Vb, rows.r[i], i, v_chunk[i]);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ks & 1][kb], qf[ks], ks == 0 ? f32x16{} : s[kb],
                                                        0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (ks + 1 < C::KS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      if (ks % (C::KS / NL) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };
  auto scores = [&]() {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 A = *reinterpret_cast<const bf16x8 *>(Kb + k_off(ks) + kb * 32 * C::ROW);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[ks], s[kb], 0, 0, 0);
      }
  };
  // probabilities of keys 8h .. 8h+7 of block kb (in the S^T layout)
  auto exps8 = [&](int kb, int h) {
#pragma unroll
    for (int i = 8 * h; i < 8 * h + 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.scale_log2, -m_run));
      pb[kb][h][i % 8] = static_cast<__bf16>(p);
    }
  };
  // The row's reference value m_run (log2 units) is any value the
  // probabilities exp2(scale s - m_run) stay finite against: softmax is the
  // same for every choice, and bf16 and fp32 keep their relative precision at
  // any magnitude. It is set to the first tile's row max and raised only when
  // a later tile's row max passes it by more than RAISE (then O and the row
  // sums are scaled down to the new value before that tile's probabilities
  // are formed). So every probability stays <= 2^RAISE and O and the row sums
  // stay far inside fp32 range.
  constexpr float RAISE = 20.0f;
  auto s_max = [&]() {
    float mx4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx4[i & 3] = fmaxf(mx4[i & 3], s[kb][i]);
    return pair_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
  };

  // Schedule. Each group's work per kept tile t is cut into four
  // half-phases, each closed by a workgroup barrier:
  //   A: softmax(t) first part (mask, row max and the rare raise of the
  //      reference value, probabilities of keys 0..31), loads of K(t+1)
  //      spread through it
  //   B: softmax(t) rest (probabilities of keys 32..127)
  //   C: P(t) V(t) and the row sums, each MFMA's transposing V reads issued
  //      four MFMAs ahead
  //   D: S(t+1) = K(t+1) Q^T, reads one k step ahead, loads of V(t+1) spread
  //      through it
  // The two groups run two half-phases apart (the group on waves 0-3 behind),
  // so A and B of one group meet C and D of the other. K(t+1) has B and C
  // to land, V(t+1) has A and B. Every load is issued unconditionally (past
  // the end of the list the last tile is fetched again), so the barriers can
  // wait with exact counts: in issue order come the row ids of tile t+1
  // (in D), V(t) (in D), K(t+1) (in A), the row ids of tile t+1 again (in C),
  // NL loads each; V(t) is waited for at the end of B with K(t+1) still
  // allowed in flight, K(t+1) at the end of C with those row ids in flight.
  // The prologue keeps the same order (row ids of tile 1 before V(0)), so the
  // compiler's own waits for the row ids agree on the first and later tiles.
  // Both groups see the same list length (the same tile): an empty list,
  // which veda_select never produces, skips the loop in both alike and
  // leaves zeros.
  if (n_t > 0) {
  Rows Rk;
  {
    const Rows R0 = rows_of(list_at(0));
#pragma unroll
    for (int i = 0; i < NL; ++i) dma1(rk, Kb, R0.r[i], i, k_chunk[i]);
    asm volatile("" ::: "memory");
    Rk = rows_of(list_at(1));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NL; ++i) dma1(rv, Vb, R0.r[i], i, v_chunk[i]);
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
  int32_t j1 = list_at(1);   // tile t+1

  for (int t = 0; t < n_t; ++t) {
    // Scalar loads for the next tiles, issued here a half-phase or more
    // before their first use (the barrier closing A waits for them).
    const int32_t j2 = list_at(t + 2);
    const int32_t vc_next = vcount[j1];
    __builtin_amdgcn_s_setprio(0);   // vector half-phases yield to the other group's MFMAs
    // ---- A
    if (vc_cur < VEDA_TILE) {
      asm volatile("" ::: "memory");
      // lane group from the lane id, recomputed here rather than kept live
      const int g4 = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5) * 4;
      const int thr = vc_cur - g4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i / 4) + (i % 4) >= thr) s[kb][i] = -INFINITY;
    }
    {
      const float xm = s_max() * a.scale_log2;   // this tile's row max, log2 units
      if (t == 0) {
        m_run = xm;   // O and the row sums are still zero
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
    // K(t+1) streams in between chunks of probabilities, a few loads at a
    // time, so no wave waits on the address unit's queue.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int i = c * NL / 2; i < (c + 1) * NL / 2; ++i) dma1(rk, Kb, Rk.r[i], i, k_chunk[i]);
      __builtin_amdgcn_sched_barrier(0);
      exps8(0, c);
      __builtin_amdgcn_sched_barrier(0);
    }
    barrier_lds();
    // ---- B
    exps8(1, 0);
    exps8(1, 1);
    exps8(2, 0);
    exps8(2, 1);
    exps8(3, 0);
    exps8(3, 1);
    barrier_vm<NL>();   // V(t) landed in every wave (K(t+1) may not)
    const Rows Rv = rows_of(j1);
    __builtin_amdgcn_s_setprio(1);   // MFMA half-phases issue first
    // ---- C
    // P(t) V(t) as 8 k steps x DB MFMAs. The transposing LDS reads have a
    // long latency, so each MFMA's two reads are issued LA_PV MFMAs ahead
    // (2 LA_PV reads in flight, within the 15 that lgkmcnt can count).
    {
      constexpr int NM = 8 * C::DB;   // MFMAs of the P V half-phase
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
        if (db == C::DB - 1) {   // the k step's probabilities into the row sums
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
    barrier_vm<NL>();   // K(t+1) landed; every wave is done with V(t)
    // ---- D
    Rk = rows_of(j2);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    scores_with_v(Rv);
    barrier_lds();     // every wave is done with K(t+1)
    vc_cur = vc_next;
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
__global__ void __launch_bounds__(512, 1) attend_bf16_kernel(AttendArgs a, HeadList heads) {
  const int32_t n_pairs = (a.n_heads + 1) / 2;
  const BlockMap bm = map_block(a, n_pairs, blockIdx.x);
  if (!bm.live) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);   // scalar
  // the leading schedule on waves 4-7 measured faster than on waves 0-3
  if (wave >= 4)
    attend_group<D, 0>(a, heads, bm.hi, bm.tile, wave - 4);
  else
    attend_group<D, 1>(a, heads, bm.hi, bm.tile, wave);
}

hipError_t launch_attend_bf16(const AttendArgs &a, const HeadList &heads, int head_dim,
                              hipStream_t s) {
  const dim3 grid(grid_blocks(a, (a.n_heads + 1) / 2));
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
  const BlockMap bm = map_block(a, a.n_heads, blockIdx.x);
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
  const dim3 grid(grid_blocks(a, a.n_heads));
  if (head_dim == 128)
    hipLaunchKernelGGL(attend_f32_kernel<128>, grid, dim3(256), 0, s, a, heads);
  else
    hipLaunchKernelGGL(attend_f32_kernel<64>, grid, dim3(256), 0, s, a, heads);
  return hipGetLastError();
}

}  // namespace veda
