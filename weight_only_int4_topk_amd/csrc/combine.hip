// Top-k weighted combine on gfx950: out[m, h] = sum_j w[m,j] * sum_z partial[z, m*topk + j, h].
//
// The second grouped GEMM leaves one float32 row per token-slot (split over K into `split`
// partials); each token's topk slots are adjacent rows, so this is a short streaming reduction in a
// fixed order (z ascending, then j ascending), which keeps the layer bitwise deterministic.  The
// pages do not describe this step; it is the weighted sum that closes every top-k MoE layer.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

template <int DT>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ partial, int split,
                                                      size_t split_stride,
                                                      const float* __restrict__ topk_w, int M,
                                                      int topk, int H, uint16_t* __restrict__ out) {
  const int h4 = H / 4;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)M * h4) return;
  const int m = (int)(idx / h4);
  const int c = (int)(idx - (size_t)m * h4) * 4;
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const size_t slot = (size_t)m * topk + j;
    const float* src = partial + slot * H + c;
    floatx4_t v = *(const floatx4_t*)src;
    for (int zz = 1; zz < split; ++zz) v += *(const floatx4_t*)(src + zz * split_stride);
    acc += topk_w[slot] * v;
  }
  const uint32_t lo = DT == 0 ? f32x2_to_f16x2(acc[0], acc[1]) : f32x2_to_bf16x2(acc[0], acc[1]);
  const uint32_t hi = DT == 0 ? f32x2_to_f16x2(acc[2], acc[3]) : f32x2_to_bf16x2(acc[2], acc[3]);
  *(uint2*)(out + (size_t)m * H + c) = make_uint2(lo, hi);
}

}  // namespace

hipError_t launch_combine(const float* partial, int split, const float* topk_w, int M, int topk,
                          int H, int dtype, void* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const size_t total = (size_t)M * (H / 4);
  const unsigned grid = (unsigned)((total + 255) / 256);
  const size_t stride = (size_t)M * topk * H;
  if (dtype == 0)
    hipLaunchKernelGGL(combine_kernel<0>, dim3(grid), dim3(256), 0, stream, partial, split, stride,
                       topk_w, M, topk, H, (uint16_t*)out);
  else
    hipLaunchKernelGGL(combine_kernel<1>, dim3(grid), dim3(256), 0, stream, partial, split, stride,
                       topk_w, M, topk, H, (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace moe
