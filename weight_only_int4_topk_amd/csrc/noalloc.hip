// fused_moe_wna16_noalloc: the fused layer for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its workspace
// is a file-scope device array, so the call allocates nothing: the array exists once per GPU the
// library runs on, from the module's load until the process ends.
//
// In host code the array's name is only a host-side stand-in, not a device address; its device
// address is looked up once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever handed to kernels.  Every call on one GPU shares the array and leaves its
// contents behind: the layer writes every workspace element it later reads, so nothing needs
// clearing, but two calls that overlap in time on one GPU (two streams, two threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "moe_wna16.h"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the current device (looked up on first use there).
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::api_fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return moe::api_fail(MOE_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return moe::api_fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                           hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int fused_moe_wna16_noalloc(const void* x, const float* router_logits, int M, int H,
                                       int I, int E, int topk, const moe_routing_t* routing,
                                       const void* w13, const void* w13_scales,
                                       const void* w13_zeros, const void* w2,
                                       const void* w2_scales, const void* w2_zeros,
                                       const moe_quant_t* quant, int dtype, int block_m, void* out,
                                       float* topk_weights_out, int32_t* topk_ids_out,
                                       void* stream) {
  if (M > 0 && H > 0 && I > 0 && E > 0 && topk > 0 && quant) {
    const size_t need = fused_moe_wna16_workspace_size(M, H, I, E, topk, quant, dtype, block_m);
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
      return moe::api_fail(MOE_ERR_WORKSPACE,
                           "fused_moe_wna16_noalloc: this batch needs %zu bytes of scratch; the "
                           "static scratch holds %zu (use fused_moe_wna16 with a workspace)",
                           need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  }
  if (stream) {
    // the scratch address is per device: the stream must belong to the current device
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) == hipSuccess && hipStreamGetDevice((hipStream_t)stream, &sdev) == hipSuccess &&
        cur != sdev)
      return moe::api_fail(MOE_ERR_INVALID_ARG,
                           "stream belongs to device %d but device %d is current", sdev, cur);
  }
  void* ws = nullptr;
  if (M > 0) {
    if (int rc = scratch_on_current_device(&ws)) return rc;
  }
  return moe::fused_wna16(x, router_logits, M, H, I, E, topk, routing, w13, w13_scales, w13_zeros,
                          w2, w2_scales, w2_zeros, quant, dtype, block_m, ws,
                          (size_t)MOE_NOALLOC_SCRATCH_BYTES, out, topk_weights_out, topk_ids_out,
                          stream);
}
