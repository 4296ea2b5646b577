// moe_layer_decode_static: the one-call decode layer for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// hosts that forbid hipMalloc).  Its scratch -- the router's float64 partial
// sums and the FFN's intermediate h, which moe_layer_decode takes as a
// workspace argument -- lives in a file-scope device array instead.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (each
// GPU holds its own copy of the array) and only that address is ever passed
// to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "moe_int4_static.h"

namespace {

constexpr size_t kScratchBytes = 4u << 20;  // covers every shape moe_layer_decode takes
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device), or null on failure.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t moe_layer_decode_static_max_bytes(void) { return kScratchBytes; }

moe_status moe_layer_decode_static(const moe_shape* shape, int32_t T, const void* x,
                                   moe_dtype x_dt, const float* w_router, const float* bias,
                                   const uint8_t* experts, const uint8_t* shared,
                                   int32_t* topk_idx, float* topk_w, int32_t* counts,
                                   int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                   int32_t* active, int32_t* n_active, void* y, void* y_shared,
                                   void* out, moe_dtype out_dt, void* stream) {
  // every argument is checked before the array is looked at; sizes beyond
  // the array are refused
  const moe_status st = moe::layer_decode_check(shape, T, x, x_dt, w_router, bias, experts,
                                                shared, topk_idx, topk_w, counts, offsets, perm,
                                                inv_perm, active, n_active, y, y_shared, out,
                                                out_dt);
  if (st != MOE_OK) return st;
  if (moe_layer_decode_workspace_bytes(shape, T) > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (T > 0) {
    ws = scratch_of_current_device();
    if (!ws) return MOE_ERR_HIP;
  }
  // the same kernels as moe_layer_decode, with the array as the workspace
  return moe_layer_decode(shape, T, x, x_dt, w_router, bias, experts, shared, topk_idx, topk_w,
                          counts, offsets, perm, inv_perm, active, n_active, y, y_shared, out,
                          out_dt, ws, kScratchBytes, stream);
}

}  // extern "C"
