// vdit_attn_fwd_noalloc: the forward pass with its workspace regions in a fixed
// device array of this library instead of caller memory, for callers that cannot
// allocate. One copy of the array exists per GPU (the code object's global), so
// every call on a GPU shares it; the kernels receive its device address exactly as
// they receive a caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "entry.hpp"
#include "vdit_attn.h"

namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;  // 256 MiB per GPU
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of the current device's copy of `scratch`, looked up once per
// device with that device current (the host-side name `scratch` is only a
// stand-in and is never passed to a kernel or a copy); nullptr on failure.
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" vdit_status_t vdit_attn_fwd_noalloc(vdit_attn_t h, const void* q, const void* k, const void* v,
                                               int32_t key_len, void* out, void* hip_stream) {
  size_t need = 0;
  int plan_dev = -1;
  vdit_status_t st = vdit::plan_workspace(h, &need, &plan_dev);
  if (st != VDIT_OK) return st;
  if (need > kScratchBytes) return VDIT_ERR_UNSUPPORTED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan_dev) return VDIT_ERR_DEVICE;
  void* ws = scratch_address(dev);
  if (!ws) return VDIT_ERR_DEVICE;
  return vdit::fwd_into_workspace(h, q, k, v, key_len, out, ws, kScratchBytes, hip_stream);
}
