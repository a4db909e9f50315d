// Top-k routing on gfx950: one 64-lane wavefront per token, four tokens per workgroup, or (64 to 256
// experts, up to 1024 tokens) one workgroup per token ranking 64-bit order keys (the per-token
// rules are in route_body.h).
#include "align_body.h"
#include "common.h"
#include "launch.h"
#include "route_body.h"

namespace moe {
namespace {

constexpr int kTokensPerWG = 4;
constexpr int kRouteAlignWaves = 16;  // route_align_kernel: tokens per launch = wavefronts
constexpr int kMaxEPL = 16;  // experts per lane: E <= 1024

template <int EPL>
__global__ void __launch_bounds__(256) routing_kernel(const float* __restrict__ logits, int M, int E,
                                                      int topk, RoutingParams p,
                                                      float* __restrict__ out_w,
                                                      int32_t* __restrict__ out_ids) {
  __shared__ float s_score[kTokensPerWG][EPL * kWave];
  const int wid = threadIdx.x / kWave;
  const int token = blockIdx.x * kTokensPerWG + wid;
  if (token >= M) return;
  route_token<EPL>(logits + (size_t)token * E, E, topk, p, s_score[wid],
                   out_w + (size_t)token * topk, out_ids + (size_t)token * topk, nullptr);
}

// One token per workgroup of 256 threads (E <= 256, topk <= 32, at most 64 groups): route_single's
// ranking (each candidate's place from 64-bit order keys, within its wavefront and then among the
// wavefronts' survivors) instead of topk rounds of a wavefront-wide arg-best; same ids and weights.
__global__ void __launch_bounds__(256) routing_rank_kernel(const float* __restrict__ logits, int E,
                                                           int topk, RoutingParams p,
                                                           float* __restrict__ out_w,
                                                           int32_t* __restrict__ out_ids) {
  __shared__ RouteLds r;
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  const float v = t < E ? logits[(size_t)m * E + t] : 0.0f;
  const float w = route_single(v, E, topk, p, r);
  if (t < topk) {
    out_ids[(size_t)m * topk + t] = r.wid[t];
    out_w[(size_t)m * topk + t] = w;
  }
}

// Small batches (M <= 4 tokens, E <= 256): routing and align in one workgroup of 16 wavefronts,
// one token per wavefront, the ids passed to align through LDS (one launch instead of two).
template <int EPL>
__global__ void __launch_bounds__(1024) route_align_kernel(
    const float* __restrict__ logits, int M, int E, int topk, RoutingParams p,
    float* __restrict__ out_w, int32_t* __restrict__ out_ids, int bm, int nbits,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_post, int64_t capacity) {
  extern __shared__ int smem[];  // align counters, then the ids
  __shared__ float s_score[kRouteAlignWaves][EPL * kWave];
  __shared__ int s_total;
  const int nw = kRouteAlignWaves;
  int32_t* s_ids = smem + (nw + 2) * E;
  const int wid = threadIdx.x / kWave;
  if (wid < M)
    route_token<EPL>(logits + (size_t)wid * E, E, topk, p, s_score[wid],
                     out_w + (size_t)wid * topk, out_ids + (size_t)wid * topk,
                     s_ids + wid * topk);
  __syncthreads();
  align_body(s_ids, M * topk, E, bm, nbits, sorted_ids, expert_ids, num_post, capacity, smem,
             &s_total);
}

// Small batches with at most 64 token-slots (M <= 4): one wavefront per token routes it, then the
// first wavefront aligns all slots alone (align_one_wave), after one barrier of M wavefronts.
template <int EPL>
__global__ void __launch_bounds__(256) route_align_small_kernel(
    const float* __restrict__ logits, int M, int E, int topk, RoutingParams p,
    float* __restrict__ out_w, int32_t* __restrict__ out_ids, int bm, int nbits,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_post, int64_t capacity) {
  extern __shared__ int smem[];  // pad[E], then the ids
  __shared__ float s_score[4][EPL * kWave];
  int32_t* s_ids = smem + E;
  const int wid = threadIdx.x / kWave;
  route_token<EPL>(logits + (size_t)wid * E, E, topk, p, s_score[wid],
                   out_w + (size_t)wid * topk, out_ids + (size_t)wid * topk, s_ids + wid * topk);
  __syncthreads();
  if (wid == 0)
    align_one_wave(s_ids, M * topk, E, bm, nbits, sorted_ids, expert_ids, num_post, capacity, smem);
}

template <int EPL>
hipError_t launch_epl(const float* logits, int M, int E, int topk, const RoutingParams& p,
                      float* w, int32_t* ids, hipStream_t stream) {
  const int grid = (M + kTokensPerWG - 1) / kTokensPerWG;
  hipLaunchKernelGGL(routing_kernel<EPL>, dim3(grid), dim3(kTokensPerWG * kWave), 0, stream, logits,
                     M, E, topk, p, w, ids);
  return hipGetLastError();
}

template <int EPL>
hipError_t launch_ra(const float* logits, int M, int E, int topk, const RoutingParams& p, float* w,
                     int32_t* ids, int block_m, int32_t* sorted_ids, int32_t* expert_ids,
                     int32_t* num_post, int64_t capacity, hipStream_t stream) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (M <= 4 && M * topk <= kWave) {
    const size_t lds_small = ((size_t)E + (size_t)M * topk) * sizeof(int);
    hipLaunchKernelGGL(route_align_small_kernel<EPL>, dim3(1), dim3(M * kWave), lds_small, stream,
                       logits, M, E, topk, p, w, ids, block_m, nbits, sorted_ids, expert_ids,
                       num_post, capacity);
    return hipGetLastError();
  }
  const size_t lds = ((size_t)(kRouteAlignWaves + 2) * E + (size_t)M * topk) * sizeof(int);
  hipLaunchKernelGGL(route_align_kernel<EPL>, dim3(1), dim3(kRouteAlignWaves * kWave), lds, stream,
                     logits, M, E, topk, p, w, ids, block_m, nbits, sorted_ids, expert_ids,
                     num_post, capacity);
  return hipGetLastError();
}

}  // namespace

// Measured: one launch saves about 1 us per layer at M = 1; from M = 16 the routing of all tokens
// in one workgroup costs more than the second launch.
bool route_align_fits(int M, int E) { return M >= 1 && M <= 4 && E <= 256; }

hipError_t launch_route_align(const float* logits, int M, int E, int topk, const RoutingParams& p,
                              float* topk_w, int32_t* topk_ids, int block_m, int32_t* sorted_ids,
                              int32_t* expert_ids, int32_t* num_post, int64_t capacity,
                              hipStream_t stream) {
  if (!route_align_fits(M, E)) return hipErrorInvalidValue;
  if (E <= 64)
    return launch_ra<1>(logits, M, E, topk, p, topk_w, topk_ids, block_m, sorted_ids, expert_ids,
                        num_post, capacity, stream);
  if (E <= 128)
    return launch_ra<2>(logits, M, E, topk, p, topk_w, topk_ids, block_m, sorted_ids, expert_ids,
                        num_post, capacity, stream);
  return launch_ra<4>(logits, M, E, topk, p, topk_w, topk_ids, block_m, sorted_ids, expert_ids,
                      num_post, capacity, stream);
}

// The ranking launch where it measured faster (routing alone, graph replays): 256 experts top-8
// grouped sigmoid 6.0 -> 4.0 us at M = 1, 6.4 -> 4.2 at 16, 6.9 -> 5.7 at 1024, but 11.2 -> 12.9
// at 4096; 64 experts top-8 3.6 -> 2.7 at M = 1, 4.3 -> 3.4 at 1024, 6.1 -> 6.3 at 4096; 8 experts
// top-2 slower at every M (1.9 -> 2.4 us at M = 1).
bool routing_rank_pays(int M, int E, int topk, const RoutingParams& p) {
  return E >= 64 && E <= 256 && topk <= 32 && p.num_groups <= 64 && M <= 1024;
}

hipError_t launch_routing(const float* logits, int M, int E, int topk, const RoutingParams& p,
                          float* topk_w, int32_t* topk_ids, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (routing_rank_pays(M, E, topk, p)) {
    hipLaunchKernelGGL(routing_rank_kernel, dim3(M), dim3(256), 0, stream, logits, E, topk, p,
                       topk_w, topk_ids);
    return hipGetLastError();
  }
  if (E <= 64) return launch_epl<1>(logits, M, E, topk, p, topk_w, topk_ids, stream);
  if (E <= 128) return launch_epl<2>(logits, M, E, topk, p, topk_w, topk_ids, stream);
  if (E <= 256) return launch_epl<4>(logits, M, E, topk, p, topk_w, topk_ids, stream);
  if (E <= 512) return launch_epl<8>(logits, M, E, topk, p, topk_w, topk_ids, stream);
  return launch_epl<kMaxEPL>(logits, M, E, topk, p, topk_w, topk_ids, stream);
}

}  // namespace moe
