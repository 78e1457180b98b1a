// ls_replay_attn_fwd_noalloc: the replay forward with the library's own
// device scratch in place of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array (each GPU the library runs on
// holds its own copy until the process ends).  In host code the array's name
// is only a host-side stand-in, so its device address is looked up once per
// device with hipGetSymbolAddress and only that address is ever passed on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ls_internal.hpp"

namespace {

__device__ __align__(256) unsigned char scratch[LS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`.
ls_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LS_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LS_OK;
}

}  // namespace

extern "C" ls_status ls_replay_attn_fwd_noalloc(const ls_attn_shape* sh, const ls_page_table* pt,
                                                const void* q, const void* k_pool,
                                                const void* v_pool, const void* k_resp,
                                                const void* v_resp, float* part_o, float* part_m,
                                                float* part_l, hipStream_t stream) {
  constexpr size_t kBytes = LS_NOALLOC_SCRATCH_BYTES;
  // every check before the first HIP call
  ls_status st =
      ls::fwd_check_args(sh, pt, q, k_pool, v_pool, k_resp, v_resp, part_o, part_m, part_l);
  if (st != LS_OK) return st;
  const size_t phys = ls::ws_phys_bytes(*pt);
  if (phys > kBytes) return LS_ERR_WORKSPACE;  // the resolved page list alone does not fit
  const size_t part_cap = kBytes - phys;      // chunk partials limited to what is left
  if (ls::fwd_ws_need(*sh, *pt, part_cap) > kBytes) return LS_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != LS_OK) return st;
  return ls::fwd_launch(sh, pt, 1, nullptr, q, k_pool, v_pool, k_resp, v_resp, part_o, part_m,
                        part_l, ws, kBytes, part_cap, stream);
}
