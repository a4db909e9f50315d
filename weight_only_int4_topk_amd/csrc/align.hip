// moe_align_block_size on gfx950: one workgroup, deterministic and stable, graph-capturable.
//
// The body (scheme and layout) is in align_body.h, shared with the small-batch routing + align
// kernel.
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

}  // namespace

hipError_t launch_align(const int32_t* topk_ids, int numel, int E, int block_m,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post,
                        int64_t capacity, hipStream_t stream) {
  const int nw = E <= 512 ? 16 : 8;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const size_t lds = (size_t)(nw + 2) * E * sizeof(int);
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(nw * kWave), lds, stream, topk_ids, numel, E,
                     block_m, nbits, sorted_ids, expert_ids, num_post, capacity);
  return hipGetLastError();
}

}  // namespace moe
