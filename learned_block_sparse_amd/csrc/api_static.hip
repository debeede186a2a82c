// veda_select_static: veda_select for callers that cannot allocate device
// memory or hand in a workspace (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc). Its scratch is one fixed device
// array per GPU, VEDA_STATIC_SCRATCH_BYTES, held until the process ends; the
// heads of a call go through it in chunks that fit. Allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "select_call.hpp"

namespace veda {
namespace {

// The host-side name of this array is a stand-in, not a device address:
// only the address that hipGetSymbolAddress returns for the current device
// may reach a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[VEDA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
unsigned char *g_scratch[kMaxDevices];   // device address of `scratch`, per device

// The device address of the scratch on the current device, looked up on the
// first call made with that device current and kept for the process.
veda_status scratch_address(unsigned char **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VEDA_ERR_UNSUPPORTED, "device index " + std::to_string(dev) + " beyond 63");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress of the static scratch");
    if (!p) return fail(VEDA_ERR_DEVICE, "the static scratch has no device address");
    g_scratch[dev] = static_cast<unsigned char *>(p);
  }
  *out = g_scratch[dev];
  return VEDA_OK;
}

}  // namespace
}  // namespace veda

using namespace veda;

extern "C" veda_status veda_select_static(const veda_plan_info *info,
                                          const veda_select_info *sel, const int32_t *perm,
                                          const int32_t *valid_count, const void *q,
                                          const void *k, veda_dtype dtype, int64_t stride_s,
                                          int64_t stride_h, int32_t n_heads_total,
                                          const int32_t *heads, const float *proj_q,
                                          const float *proj_k, int32_t *row_offsets,
                                          int32_t *cols, hipStream_t stream) {
  SelectCall c;
  veda_status st = select_check(info, sel, perm, valid_count, q, k, dtype, stride_s, stride_h,
                                n_heads_total, heads, proj_q, proj_k, row_offsets, cols, nullptr,
                                0, &c);
  if (st != VEDA_OK) return st;
  if (!c.scoring) return select_range(c, 0, sel->n_heads, nullptr, stream);   // keeps all
  // the most heads whose pooled features, projections and logits fit
  int32_t chunk = 0;
  for (int32_t nh = sel->n_heads; nh >= 1 && chunk == 0; --nh)
    if (select_workspace(info, sel->head_dim, nh).total <= VEDA_STATIC_SCRATCH_BYTES) chunk = nh;
  if (chunk == 0)
    return fail(VEDA_ERR_UNSUPPORTED,
                "one head's selection needs " +
                    std::to_string(select_workspace(info, sel->head_dim, 1).total) +
                    " bytes of scratch; the static scratch holds " +
                    std::to_string(VEDA_STATIC_SCRATCH_BYTES) +
                    " (use veda_select with a workspace)");
  unsigned char *w = nullptr;
  if ((st = scratch_address(&w)) != VEDA_OK) return st;
  for (int32_t h0 = 0; h0 < sel->n_heads; h0 += chunk) {
    st = select_range(c, h0, std::min(chunk, sel->n_heads - h0), w, stream);
    if (st != VEDA_OK) return st;
  }
  return VEDA_OK;
}
