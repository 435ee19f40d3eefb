// moe_forward_static: the whole-layer forward with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate device memory (code under graph capture, serving loops, harnesses
// that forbid allocation).
//
// The array lives in this library's code object: every GPU the library runs on
// holds its own copy, at its own address, from the first use until the process
// ends.  Its device address is fetched once per device with
// hipGetSymbolAddress (the array's host-side name is only a stand-in, not a
// device address) and kept; the kernels receive that address as their
// workspace, exactly as moe_forward receives a caller's.
//
// moe_forward writes every workspace byte it reads before reading it, so the
// array needs no clearing between calls.  Every call on one GPU uses the same
// array: calls that overlap on one GPU (other streams, other threads) race.
#include <stdio.h>

#include <mutex>

#include "common.hpp"

constexpr size_t kStaticScratchBytes = 64ull << 20;   // 64 MiB per GPU

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

std::mutex g_mu;
void *g_scratch_ptr[moe::kMaxDevices] = {};

}  // namespace

extern "C" {

moe_status moe_forward_static(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                              void *out, int32_t *topk_idx, float *topk_w, void *stream) {
  size_t need = 0;
  const moe_status s = moe_workspace_size(cfg, T, &need);
  if (s != MOE_OK) return s;
  if (need > kStaticScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "moe_forward_static: the layer needs %zu bytes of workspace, more than the %zu-byte static "
             "scratch; call moe_forward with a caller workspace instead",
             need, kStaticScratchBytes);
    return moe::set_error(MOE_ERR_WORKSPACE, msg);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= moe::kMaxDevices)
    return moe::set_error(MOE_ERR_DEVICE, "moe_forward_static: no usable current device");
  void *ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    ptr = g_scratch_ptr[dev];
    if (ptr == nullptr) {
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || ptr == nullptr) {
        char msg[256];
        snprintf(msg, sizeof(msg), "moe_forward_static: hipGetSymbolAddress: %s", hipGetErrorString(e));
        return moe::set_error(MOE_ERR_DEVICE, msg);
      }
      g_scratch_ptr[dev] = ptr;
    }
  }
  return moe_forward(cfg, T, x, w, out, topk_idx, topk_w, ptr, kStaticScratchBytes, stream);
}

}  // extern "C"
