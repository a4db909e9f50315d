// moe_align_block_size body for one workgroup (nw = blockDim / 64 wavefronts), shared by the
// align kernel and the small-batch routing + align kernel.
//
// Groups the token-slots by expert (ascending slot order inside an expert) and pads every expert's
// group to a multiple of block_m with a sentinel, writing the per-block expert id and the padded
// total on the device.  "[Kernel] add triton fused moe kernel for gptq/awq" (PR notes) names this
// step and its shared-memory form for large expert counts (DeepSeek-V3, 256 experts) that can be
// captured in a graph; the output layout is the plainest reading of that operation.
//
// Scheme (no order-dependent atomics, so the result never varies between runs):
//   1. each wave counts experts over its own contiguous chunk of slots (LDS atomics: order-free);
//   2. per expert, an exclusive prefix over waves gives each wave's base inside the expert;
//      wave 0 scans the padded per-expert totals into expert offsets;
//   3. each wave walks its chunk 64 slots at a time: lanes holding the same expert find each other
//      with one ballot per expert-id bit (a match-any), rank = number of equal lanes below; the
//      slot goes to offset[e] + base[wave][e] + rank, and the highest-ranked lane advances the base;
//   4. padding positions and blocks get the sentinel / expert ids; the tail past T gets sentinels.
// ids may live in global memory or in LDS; smem holds (nw + 2) * E ints; s_total is an LDS int.
#pragma once

#include "common.h"

namespace moe {

__device__ inline void align_body(const int32_t* __restrict__ ids, int numel, int E, int bm,
                                  int nbits, int32_t* __restrict__ sorted_ids,
                                  int32_t* __restrict__ expert_ids, int32_t* __restrict__ num_post,
                                  int64_t capacity, int* smem, int* s_total) {
  const int nw = blockDim.x / kWave;
  int* cnt = smem;            // [nw][E]: counts, then running base of each wave inside an expert
  int* off = cnt + nw * E;    // [E]: start of expert e in sorted_ids
  int* tot = off + E;         // [E]: number of slots of expert e

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int chunk = (numel + nw - 1) / nw;
  const int beg = min(numel, wave * chunk);
  const int end = min(numel, beg + chunk);

  for (int i = tid; i < nw * E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  // 1. per-wave expert counts
  for (int s = beg + lane; s < end; s += kWave) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[wave * E + e], 1);
  }
  __syncthreads();

  // 2a. per expert: exclusive prefix over waves
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
    tot[e] = run;
  }
  __syncthreads();

  // 2b. wave 0: exclusive scan of padded totals over experts (lane owns a contiguous run)
  if (wave == 0) {
    const int per = (E + kWave - 1) / kWave;
    const int e0 = min(E, lane * per);
    const int e1 = min(E, e0 + per);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += (tot[e] + bm - 1) / bm * bm;
    // inclusive wave scan
    int inc = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += o;
    }
    int run = inc - local;
    for (int e = e0; e < e1; ++e) {
      off[e] = run;
      run += (tot[e] + bm - 1) / bm * bm;
    }
    if (lane == kWave - 1) {
      *s_total = inc;
      num_post[0] = inc;
    }
  }
  __syncthreads();

  // 3. stable scatter
  for (int base = beg; base < end; base += kWave) {
    const int s = base + lane;
    int e = s < end ? ids[s] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & lanemask_lt(lane));
      const int n = __popcll(peers);
      int* run = &cnt[wave * E + e];
      const int pos = off[e] + *run + rank;
      sorted_ids[pos] = s;
      if (rank == n - 1) *run += n;
    }
  }

  // 4. padding of each expert group, block expert ids, and the tail past T
  const int T = *s_total;
  for (int e = tid; e < E; e += blockDim.x) {
    const int c = tot[e];
    const int padded = (c + bm - 1) / bm * bm;
    const int o = off[e];
    for (int p = o + c; p < o + padded; ++p) sorted_ids[p] = numel;
    for (int b = o / bm; b < (o + padded) / bm; ++b) expert_ids[b] = e;
  }
  for (int64_t p = T + tid; p < capacity; p += blockDim.x) sorted_ids[p] = numel;
  const int64_t nblk = (capacity + bm - 1) / bm;
  for (int64_t b = T / bm + tid; b < nblk; b += blockDim.x) expert_ids[b] = -1;
}


// The same operation for at most 64 slots by one wavefront (lane s holds slot s): no per-wave count
// arrays and no workgroup barriers.  Lanes holding the same expert find each other with one ballot
// per expert-id bit (a match-any): a lane's rank among them is its position in ascending slot
// order, their number is the group size.  The lowest lane of each group writes the group's padded
// size into pad[e] (LDS, E ints), one exclusive scan over the experts turns pad into offsets, and
// every lane places its slot; the group's lowest lane also writes its padding and block expert ids.
// Output identical to align_body.  ids may live in LDS or global memory.
__device__ inline void align_one_wave(const int32_t* ids, int numel, int E, int bm, int nbits,
                                      int32_t* __restrict__ sorted_ids,
                                      int32_t* __restrict__ expert_ids,
                                      int32_t* __restrict__ num_post, int64_t capacity, int* pad) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int e = lane; e < E; e += kWave) pad[e] = 0;
  const int e = lane < numel ? ids[lane] : -1;
  const bool valid = (unsigned)e < (unsigned)E;
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  const int rank = valid ? __popcll(peers & lanemask_lt(lane)) : 0;
  const int cnt = valid ? __popcll(peers) : 0;
  const int padded = (cnt + bm - 1) / bm * bm;
  __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in program order
  if (valid && rank == 0) pad[e] = padded;
  __builtin_amdgcn_wave_barrier();

  // exclusive scan of the padded sizes over experts (lane owns a contiguous run of experts)
  const int per = (E + kWave - 1) / kWave;
  const int e0 = min(E, lane * per);
  const int e1 = min(E, e0 + per);
  int local = 0;
  for (int x = e0; x < e1; ++x) local += pad[x];
  int inc = local;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  int run = inc - local;
  for (int x = e0; x < e1; ++x) {
    const int sz = pad[x];
    pad[x] = run;
    run += sz;
  }
  const int T = __shfl(inc, kWave - 1, kWave);
  __builtin_amdgcn_wave_barrier();

  if (valid) {
    const int off = pad[e];
    sorted_ids[off + rank] = lane;
    if (rank == 0) {
      for (int q = off + cnt; q < off + padded; ++q) sorted_ids[q] = numel;
      for (int b = off / bm; b < (off + padded) / bm; ++b) expert_ids[b] = e;
    }
  }
  for (int64_t q = T + lane; q < capacity; q += kWave) sorted_ids[q] = numel;
  const int64_t nblk = (capacity + bm - 1) / bm;
  for (int64_t b = T / bm + lane; b < nblk; b += kWave) expert_ids[b] = -1;
  if (lane == 0) num_post[0] = T;
}

}  // namespace moe
