// moe_align_block_size on gfx950: deterministic and stable, graph-capturable.
//
// The bodies (scheme and layout) are in align_body.h, shared with the small-batch routing + align
// kernels: up to 64 slots one wavefront aligns alone, beyond that a workgroup of 8 or 16.  Inside
// the fused layers, from kAlignMultiMin slots on, two launches over many workgroups produce the
// same output (their per-chunk counts live in the layer's workspace).
#include <algorithm>

#include "align_body.h"
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kAlignMultiMin = 8192;    // slots from which the many-workgroup form runs
constexpr int kMultiChunkMin = 512;     // slots per workgroup of the many-workgroup form, at least
constexpr int kMultiBlocksMax = 128;    // and workgroups, at most

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

// ---- many slots: two launches over many workgroups (the same output as align_body)
//   count:   workgroup b counts the experts of its contiguous chunk of slots (LDS atomics);
//   scatter: workgroup b sums every chunk's counts per expert (all chunks: the expert totals; the
//            chunks before b: its base inside each expert), scans the padded totals into expert
//            offsets, and places its chunk's slots stably (per-wave counts and prefix, then the
//            ballot match-any ranks of align_body); workgroup 0 also writes the padding, the block
//            expert ids, the tail past T and T.
constexpr int kMultiThreads = 256;

__global__ void __launch_bounds__(kMultiThreads) align_count_kernel(const int32_t* __restrict__ ids,
                                                                    int numel, int E, int chunk,
                                                                    int32_t* __restrict__ counts) {
  extern __shared__ int cnt[];  // [E]
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kMultiThreads) cnt[e] = 0;
  __syncthreads();
  const int beg = b * chunk;
  const int end = min(numel, beg + chunk);
  for (int s = beg + (int)threadIdx.x; s < end; s += kMultiThreads) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kMultiThreads) counts[(size_t)b * E + e] = cnt[e];
}

__global__ void __launch_bounds__(kMultiThreads) align_scatter_kernel(
    const int32_t* __restrict__ ids, int numel, int E, int bm, int chunk, int nbits, int nb,
    const int32_t* __restrict__ counts, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ num_post, int64_t capacity) {
  extern __shared__ int sm[];  // tot[E], off[E], start[E], cnt[nw][E]
  __shared__ int s_total;
  constexpr int nw = kMultiThreads / kWave;
  int* tot = sm;             // slots of expert e
  int* off = sm + E;         // this chunk's base inside expert e, then its first position
  int* start = sm + 2 * E;   // first position of expert e
  int* cnt = sm + 3 * E;     // per-wave counts, then running positions
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // every chunk's counts: the expert totals, and this chunk's base inside each expert (16 chunks'
  // counts loaded before any is used)
  for (int i = tid; i < nw * E; i += kMultiThreads) cnt[i] = 0;
  for (int e = tid; e < E; e += kMultiThreads) {
    int all = 0, before = 0;
    for (int c0 = 0; c0 < nb; c0 += 16) {
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = c0 + i < nb ? counts[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        before += c0 + i < b ? c[i] : 0;
        all += c[i];
      }
    }
    tot[e] = all;
    off[e] = before;  // for now: the chunk's base
  }
  __syncthreads();

  // this chunk's slots: per-wave counts over contiguous sub-chunks
  const int beg0 = b * chunk;
  const int end0 = min(numel, beg0 + chunk);
  const int sub = (end0 - beg0 + nw - 1) / nw;
  const int beg = min(end0, beg0 + wave * sub);
  const int end = min(end0, beg + sub);
  for (int s = beg + lane; s < end; s += kWave) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[wave * E + e], 1);
  }
  // wave 0: exclusive scan of the padded totals over experts (a lane owns a contiguous run);
  // each expert's start plus the chunk's base
  if (wave == 0) {
    const int per = (E + kWave - 1) / kWave;
    const int e0 = min(E, lane * per);
    const int e1 = min(E, e0 + per);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += (tot[e] + bm - 1) / bm * bm;
    int inc = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += o;
    }
    int run = inc - local;
    for (int e = e0; e < e1; ++e) {
      start[e] = run;
      off[e] += run;
      run += (tot[e] + bm - 1) / bm * bm;
    }
    if (lane == kWave - 1) s_total = inc;
  }
  __syncthreads();
  // per expert: each wave's start
  for (int e = tid; e < E; e += kMultiThreads) {
    int run = off[e];
    for (int w = 0; w < nw; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int base = beg; base < end; base += kWave) {
    const int s = base + lane;
    const int e = s < end ? ids[s] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = valid && ((e >> bit) & 1);
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & lanemask_lt(lane));
      const int n = __popcll(peers);
      int* run = &cnt[wave * E + e];
      sorted_ids[*run + rank] = s;
      if (rank == n - 1) *run += n;
    }
  }
  if (b != 0) return;
  // workgroup 0: padding of each expert group, block expert ids, the tail past T, and T
  const int T = s_total;
  for (int e = tid; e < E; e += kMultiThreads) {
    const int c = tot[e];
    const int padded = (c + bm - 1) / bm * bm;
    const int o = start[e];
    for (int p = o + c; p < o + padded; ++p) sorted_ids[p] = numel;
    for (int q = o / bm; q < (o + padded) / bm; ++q) expert_ids[q] = e;
  }
  for (int64_t p = T + tid; p < capacity; p += kMultiThreads) sorted_ids[p] = numel;
  const int64_t nblk = (capacity + bm - 1) / bm;
  for (int64_t q = T / bm + tid; q < nblk; q += kMultiThreads) expert_ids[q] = -1;
  if (tid == 0) num_post[0] = T;
}

int multi_chunk(int numel) { return std::max(kMultiChunkMin, (numel + kMultiBlocksMax - 1) / kMultiBlocksMax); }

}  // namespace

size_t align_multi_scratch_bytes(int numel, int E) {
  const int chunk = multi_chunk(numel);
  const int nb = (numel + chunk - 1) / chunk;
  return (size_t)nb * E * 4;
}

bool align_multi_pays(int numel) { return numel >= kAlignMultiMin; }

hipError_t launch_align_multi(const int32_t* topk_ids, int numel, int E, int block_m,
                              int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post,
                              int64_t capacity, int32_t* scratch, hipStream_t stream) {
  if (numel <= 0) return launch_align(topk_ids, numel, E, block_m, sorted_ids, expert_ids,
                                      num_post, capacity, stream);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int chunk = multi_chunk(numel);
  const int nb = (numel + chunk - 1) / chunk;
  int32_t* counts = scratch;  // [nb][E]
  hipLaunchKernelGGL(align_count_kernel, dim3(nb), dim3(kMultiThreads), (size_t)E * sizeof(int),
                     stream, topk_ids, numel, E, chunk, counts);
  if (hipError_t e = hipGetLastError()) return e;
  const size_t lds = (size_t)(3 + kMultiThreads / kWave) * E * sizeof(int);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nb), dim3(kMultiThreads), lds, stream, topk_ids,
                     numel, E, block_m, chunk, nbits, nb, counts, sorted_ids, expert_ids, num_post,
                     capacity);
  return hipGetLastError();
}

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
