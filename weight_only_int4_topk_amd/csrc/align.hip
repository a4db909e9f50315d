// moe_align_block_size on gfx950: one workgroup, deterministic and stable, graph-capturable.
//
// The bodies (scheme and layout) are in align_body.h, shared with the small-batch routing + align
// kernels: up to 64 slots one wavefront aligns alone, beyond that a workgroup of 8 or 16.
#include "align_body.h"
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__global__ void __launch_bounds__(1024) align_kernel(const int32_t* __restrict__ ids, int numel,
                                                     int E, int bm, int nbits,
                                                     int32_t* __restrict__ sorted_ids,
                                                     int32_t* __restrict__ expert_ids,
                                                     int32_t* __restrict__ num_post,
                                                     int64_t capacity) {
  extern __shared__ int smem[];
  __shared__ int s_total;
  align_body(ids, numel, E, bm, nbits, sorted_ids, expert_ids, num_post, capacity, smem, &s_total);
}

// At most 64 slots: one wavefront, no workgroup barriers (align_one_wave).
__global__ void __launch_bounds__(64) align_small_kernel(const int32_t* __restrict__ ids, int numel,
                                                         int E, int bm, int nbits,
                                                         int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ expert_ids,
                                                         int32_t* __restrict__ num_post,
                                                         int64_t capacity) {
  extern __shared__ int smem[];  // pad[E]
  align_one_wave(ids, numel, E, bm, nbits, sorted_ids, expert_ids, num_post, capacity, smem);
}

}  // namespace

hipError_t launch_align(const int32_t* topk_ids, int numel, int E, int block_m,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post,
                        int64_t capacity, hipStream_t stream) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (numel <= kWave) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kWave), (size_t)E * sizeof(int), stream,
                       topk_ids, numel, E, block_m, nbits, sorted_ids, expert_ids, num_post,
                       capacity);
    return hipGetLastError();
  }
  const int nw = E <= 512 ? 16 : 8;
  const size_t lds = (size_t)(nw + 2) * E * sizeof(int);
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(nw * kWave), lds, stream, topk_ids, numel, E,
                     block_m, nbits, sorted_ids, expert_ids, num_post, capacity);
  return hipGetLastError();
}

}  // namespace moe
