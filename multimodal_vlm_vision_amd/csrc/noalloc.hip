// vit_encode for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the forward's workspace is a
// file-scope device array of fixed size instead of a caller buffer.
//
// The array lives in the library's code object, so each GPU the library runs on holds its
// own copy, at its own address, until the process ends.  Host code never passes the array's
// name to a kernel (on the host that name is only a stand-in, not a device address): on the
// first call on a device, with that device current, hipGetSymbolAddress resolves the
// device's copy, and that pointer is kept per device and handed to the unchanged forward
// (vit_encode) as its workspace.  The forward clears what must start at zero itself (the
// V^T pad columns, by a kernel, every call) and writes every other region before reading
// it, so the previous call's contents never matter.  Every call on a GPU shares that GPU's
// array: calls that overlap in time on one GPU race (issue them on one stream or order
// them).
#include <hip/hip_runtime.h>

#include <mutex>

#include "vit_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)VIT_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of each device's `scratch`, once resolved

// The calling thread's current device's copy of `scratch` (resolved once per device).
vit_status scratch_for_current_device(int* device, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    vitmi::set_error("vit_encode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return VIT_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    vitmi::set_error("vit_encode_noalloc: device %d out of range", dev);
    return VIT_E_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      vitmi::set_error("vit_encode_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                       hipGetErrorString(e));
      return VIT_E_HIP;
    }
    g_scratch[dev] = p;
  }
  *device = dev;
  *out = g_scratch[dev];
  return VIT_OK;
}

}  // namespace

extern "C" vit_status vit_encode_noalloc(const vit_ctx* ctx, const vit_plan* plan, const uint8_t* pixels_u8,
                                         float* out, void* stream) {
  if (!ctx || !plan) {
    vitmi::set_error("ctx and plan must not be NULL");
    return VIT_E_ARG;
  }
  if (plan->ws_bytes > kScratchBytes) {
    vitmi::set_error("vit_encode_noalloc: the batch needs a %zu-byte workspace; the static scratch holds %zu "
                     "bytes (use vit_encode with a caller workspace)",
                     plan->ws_bytes, kScratchBytes);
    return VIT_E_WORKSPACE;
  }
  if (plan->n_rows == 0) return VIT_OK;
  int dev = -1;
  void* ws = nullptr;
  const vit_status s = scratch_for_current_device(&dev, &ws);
  if (s != VIT_OK) return s;
  if (ctx->finalized && dev != ctx->device) {
    vitmi::set_error("vit_encode_noalloc: current device %d, but the weights live on device %d", dev,
                     ctx->device);
    return VIT_E_STATE;
  }
  return vit_encode(ctx, plan, pixels_u8, ws, kScratchBytes, out, stream);
}
