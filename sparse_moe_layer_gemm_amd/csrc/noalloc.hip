// moe_forward_noalloc: the whole layer for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). The workspace moe_forward takes as an argument is
// here a file-scope device array that the library holds on every device it
// runs on until the process ends.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on a device comes from hipGetSymbolAddress, called once
// per device with that device current, and only that pointer is handed to the
// kernels. Calls on one device share the array, so calls that overlap on one
// device race. No kernel of the layer needs its workspace cleared first (no
// counters, atomics or flags live there: every byte a kernel reads was written
// earlier in the same call), so nothing is cleared here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // the array's address on each device, once looked up

// The device that `stream` runs on (the current device for the null stream).
moe_status stream_device(hipStream_t stream, int* dev) {
  if (stream == nullptr) return hipGetDevice(dev) == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
  return hipStreamGetDevice(stream, dev) == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// Address of the scratch array on device `dev`, looked up on first use with
// that device current (the caller's current device is restored).
moe_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_LAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_ERR_LAUNCH;
    if (e != hipSuccess || p == nullptr) return MOE_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const void* x, int32_t x_dtype, int64_t T, int32_t H,
                                          int32_t I, int32_t E, int32_t k, const float* w_router,
                                          const float* bias, const moe_expert_weights* w,
                                          int32_t out_dtype, void* out, float* out_f32,
                                          int32_t logits_dtype, void* logits, int32_t* topk_ids,
                                          float* topk_w, void* stream) {
  moe_status s = moe::check_forward(x, x_dtype, T, H, I, E, k, w_router, bias, w, out_dtype, out,
                                    out_f32, logits_dtype, logits, topk_ids, topk_w);
  if (s != MOE_OK || T == 0) return s;
  const size_t need = moe_forward_workspace_size(T, H, I, E, k, w);
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = -1;
  s = stream_device(st, &dev);
  if (s != MOE_OK) return s;
  void* ws = nullptr;
  s = scratch_on(dev, &ws);
  if (s != MOE_OK) return s;
  return moe::enqueue_forward(x, x_dtype, T, H, I, E, k, w_router, bias, w, out_dtype, out, out_f32,
                              logits_dtype, logits, topk_ids, topk_w, ws, kScratchBytes, stream);
}
