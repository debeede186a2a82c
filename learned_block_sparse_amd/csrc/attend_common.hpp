// Pieces shared by the attend kernels (attend.hip: bf16 Q.K^T; attend_i8.hip:
// int8 Q.K^T): the workgroup -> (head, query tile) map, lane exchanges and
// the barriers of the ping-pong schedule.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace veda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Dispatch order: the heavy global query tiles (they see every tile) first,
// then the video tiles. Video tiles are remapped so that each of the 8 XCDs
// (which take workgroups round-robin) works through a contiguous range of
// (head, query tile): neighbouring query tiles share most key tiles, and the
// shared tiles then stay in that XCD's L2.
struct BlockMap {
  int32_t hi, tile;
  bool live;
};

__device__ inline BlockMap map_block(const AttendArgs &a, int32_t n_units, uint32_t b) {
  BlockMap m{0, 0, false};
  const uint32_t G = uint32_t(n_units) * uint32_t(a.n_tiles - a.n_video);
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
  const uint32_t NV = uint32_t(n_units) * uint32_t(a.n_video);
  const uint32_t per = (NV + 7u) / 8u;
  const uint32_t logical = (bv % 8u) * per + bv / 8u;
  if (logical >= NV) return m;
  m.hi = int32_t(logical / uint32_t(a.n_video));
  m.tile = int32_t(logical % uint32_t(a.n_video));
  m.live = true;
  return m;
}

__host__ inline uint32_t grid_blocks(const AttendArgs &a, int32_t n_units) {
  const uint32_t G = uint32_t(n_units) * uint32_t(a.n_tiles - a.n_video);
  const uint32_t Gp = (G + 7u) & ~7u;
  const uint32_t NV = uint32_t(n_units) * uint32_t(a.n_video);
  return Gp + 8u * ((NV + 7u) / 8u);
}

// one 16-byte global read
__device__ inline uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
// Tile lists and valid counts are read with uniform indices and never written
// by this kernel: reading them through the constant address space gives
// scalar loads, which do not count against the vector-memory counter that
// the load pipeline's waits rely on.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ inline const_i32 *as_const(const int32_t *p) { return (const_i32 *)(p); }

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

template <int N>
__device__ inline void barrier_vm() {
  // this wave's loads older than the newest N have landed, its LDS reads have
  // returned; then the workgroup barrier
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ inline void barrier_lds() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace veda
