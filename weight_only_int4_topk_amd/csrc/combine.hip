// Top-k weighted combine on gfx950: out[m, h] = sum_j w[m,j] * sum_z partial[z, m*topk + j, h];
// and, when the first GEMM is split over K, the sum of its partials followed by SiLU(gate) * up.
//
// The second grouped GEMM leaves one float32 row per token-slot (split over K into `split`
// partials); each token's topk slots are adjacent rows, so this is a short streaming reduction in a
// fixed order (z ascending, then j ascending), which keeps the layer bitwise deterministic.  The
// pages do not describe this step; it is the weighted sum that closes every top-k MoE layer.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// Streaming sums over float32 partials, issued in batches of kBatch independent 16-byte loads so
// that a long reduction costs a few memory round trips instead of one per term.  Terms are added in
// a fixed order, so results do not depend on the batching.
constexpr int kBatch = 16;

// sum_z src[z * stride .. + 3], z ascending
__device__ __forceinline__ floatx4_t sum_splits(const float* src, int split, size_t stride) {
  floatx4_t v = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < split; z0 += kBatch) {
    floatx4_t t[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (z0 + q < split) t[q] = *(const floatx4_t*)(src + (size_t)(z0 + q) * stride);
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (z0 + q < split) v = (z0 + q == 0) ? t[q] : v + t[q];
  }
  return v;
}

// sum_j w[j] * (sum_z src[j * H + z * stride .. + 3]) with z ascending inside j ascending; the
// (j, z) terms are loaded kBatch at a time across slot boundaries
__device__ __forceinline__ floatx4_t sum_weighted_slots(const float* src, const float* w, int topk,
                                                        int split, int H, size_t stride) {
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  floatx4_t v = {0.f, 0.f, 0.f, 0.f};
  const int n = topk * split;
  for (int t0 = 0; t0 < n; t0 += kBatch) {
    floatx4_t t[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int k = t0 + q;
      if (k < n) {
        const int j = k / split;
        t[q] = *(const floatx4_t*)(src + (size_t)j * H + (size_t)(k - j * split) * stride);
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int k = t0 + q;
      if (k < n) {
        const int j = k / split;
        const int zz = k - j * split;
        v = zz == 0 ? t[q] : v + t[q];
        if (zz == split - 1) acc += w[j] * v;
      }
    }
  }
  return acc;
}

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
  const size_t slot0 = (size_t)m * topk;
  const floatx4_t acc = sum_weighted_slots(partial + slot0 * H + c, topk_w + slot0, topk, split, H,
                                           split_stride);
  const uint32_t lo = DT == 0 ? f32x2_to_f16x2(acc[0], acc[1]) : f32x2_to_bf16x2(acc[0], acc[1]);
  const uint32_t hi = DT == 0 ? f32x2_to_f16x2(acc[2], acc[3]) : f32x2_to_bf16x2(acc[2], acc[3]);
  *(uint2*)(out + (size_t)m * H + c) = make_uint2(lo, hi);
}

// Few tokens with many partial terms (k * split >= 16, as at M = 1 where the second GEMM is split
// 5-16 ways): the plain kernel leaves most lanes idle and walks the terms in dependent batches.
// Here four wavefronts cover 256 columns of one token, wavefront q summing the q-th quarter of the
// (slot, split) terms (slot-major, each term times its slot's routing weight) in one batch of
// loads, and the quarters are added in LDS in wavefront order: ((q0 + q1) + q2) + q3.  A fixed
// order, so the layer stays bitwise deterministic.
template <int DT>
__global__ void __launch_bounds__(256) combine_quarters_kernel(const float* __restrict__ partial,
                                                               int split, size_t split_stride,
                                                               const float* __restrict__ topk_w,
                                                               int topk, int H,
                                                               uint16_t* __restrict__ out) {
  __shared__ floatx4_t s_q[3][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int q = threadIdx.x / kWave;
  const int cpb = H / 256;
  const int m = blockIdx.x / cpb;
  const int c = (blockIdx.x - m * cpb) * 256 + lane * 4;
  const int n = topk * split;
  const int t0 = q * n / 4, t1 = (q + 1) * n / 4;
  const size_t slot0 = (size_t)m * topk;
  const float* src = partial + slot0 * H + c;
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int b = t0; b < t1; b += kBatch) {
    floatx4_t t[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int k = b + i;
      if (k < t1) {
        const int j = k / split;
        t[i] = *(const floatx4_t*)(src + (size_t)j * H + (size_t)(k - j * split) * split_stride);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int k = b + i;
      if (k < t1) acc += topk_w[slot0 + k / split] * t[i];
    }
  }
  if (q > 0) s_q[q - 1][lane] = acc;
  __syncthreads();
  if (q == 0) {
    acc = ((acc + s_q[0][lane]) + s_q[1][lane]) + s_q[2][lane];
    store4<DT>(out + (size_t)m * H + c, acc);
  }
}

// The second GEMM unsplit, its rows already weighted and rounded to the activation dtype: out[m] =
// sum_j y[m * topk + j] in float32, j ascending, rounded once.  Half the bytes of the float32 rows
// (DeepSeek-V3 prefill at 4096 tokens: 470 MB instead of 940 MB written and read back).  Each
// thread sums 8 columns of one token, the topk rows loaded kBatch at a time.
template <int DT>
__global__ void __launch_bounds__(256) combine_rows_kernel(const uint16_t* __restrict__ y, int M,
                                                           int topk, int H,
                                                           uint16_t* __restrict__ out) {
  const int h8 = H / 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)M * h8) return;
  const int m = (int)(idx / h8);
  const int c = (int)(idx - (size_t)m * h8) * 8;
  const uint16_t* src = y + (size_t)m * topk * H + c;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < topk; j0 += kBatch) {
    u32x4_t t[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (j0 + q < topk) t[q] = *(const u32x4_t*)(src + (size_t)(j0 + q) * H);
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (j0 + q < topk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = t[q][i];
          acc[2 * i] += bits_to_float<DT>((uint16_t)(w & 0xFFFFu));
          acc[2 * i + 1] += bits_to_float<DT>((uint16_t)(w >> 16));
        }
      }
    }
  }
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = DT == 0 ? f32x2_to_f16x2(acc[2 * i], acc[2 * i + 1])
                   : f32x2_to_bf16x2(acc[2 * i], acc[2 * i + 1]);
  *(u32x4_t*)(out + (size_t)m * H + c) = o;
}

// First GEMM split over K: inter[s, i] = SiLU(g) * u with g = sum_z partial[z, s, i] and
// u = sum_z partial[z, s, I + i] (z ascending), rounded to dtype; four columns per thread.
template <int DT>
__global__ void __launch_bounds__(256) act_combine_kernel(const float* __restrict__ partial,
                                                          int split, size_t split_stride, int slots,
                                                          int I, uint16_t* __restrict__ inter) {
  const int i4 = I / 4;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)slots * i4) return;
  const int s = (int)(idx / i4);
  const int c = (int)(idx - (size_t)s * i4) * 4;
  const float* src = partial + (size_t)s * 2 * I + c;
  floatx4_t g, u;
  if (split <= kBatch) {
    // gate and up partials in one batch of loads (one memory round trip instead of two), summed
    // in the order of sum_splits (z ascending), so the result is unchanged
    floatx4_t tg[kBatch], tu[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (q < split) {
        tg[q] = *(const floatx4_t*)(src + (size_t)q * split_stride);
        tu[q] = *(const floatx4_t*)(src + I + (size_t)q * split_stride);
      }
    }
    g = tg[0];
    u = tu[0];
#pragma unroll
    for (int q = 1; q < kBatch; ++q) {
      if (q < split) {
        g = g + tg[q];
        u = u + tu[q];
      }
    }
  } else {
    g = sum_splits(src, split, split_stride);
    u = sum_splits(src + I, split, split_stride);
  }
  floatx4_t a;
#pragma unroll
  for (int q = 0; q < 4; ++q) a[q] = g[q] / (1.0f + __expf(-g[q])) * u[q];
  const uint32_t lo = DT == 0 ? f32x2_to_f16x2(a[0], a[1]) : f32x2_to_bf16x2(a[0], a[1]);
  const uint32_t hi = DT == 0 ? f32x2_to_f16x2(a[2], a[3]) : f32x2_to_bf16x2(a[2], a[3]);
  *(uint2*)(inter + (size_t)s * I + c) = make_uint2(lo, hi);
}

// Dense GEMM split over K: out[r, c] = sum_z partial[z, r, c], z ascending; four columns per thread.
template <int DT>
__global__ void __launch_bounds__(256) split_reduce_kernel(const float* __restrict__ partial,
                                                           int split, size_t split_stride,
                                                           size_t total4, uint16_t* __restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total4) return;
  store4<DT>(out + idx * 4, sum_splits(partial + idx * 4, split, split_stride));
}

// Act-order experts: slot s's activation row through its expert's input-column permutation,
// out[s, j] = in[s / div, perm[ids[s], j]]; eight columns (one 16-byte store) per thread.  Entries
// that would index outside the row or the permutation table give zero instead.
__global__ void __launch_bounds__(256) gather_cols_kernel(const uint16_t* __restrict__ in, int div,
                                                          const int32_t* __restrict__ ids, int E,
                                                          const int32_t* __restrict__ perm, int K,
                                                          int slots, uint16_t* __restrict__ out) {
  const int k8 = K / 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)slots * k8) return;
  const int s = (int)(idx / k8);
  const int j0 = (int)(idx - (size_t)s * k8) * 8;
  const int e = ids[s];
  const uint16_t* row = in + (size_t)(s / div) * K;
  uint32_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t pair = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int pj = (unsigned)e < (unsigned)E ? perm[(size_t)e * K + j0 + 2 * i + h] : -1;
      const uint32_t val = (unsigned)pj < (unsigned)K ? row[pj] : 0u;
      pair |= val << (16 * h);
    }
    v[i] = pair;
  }
  *(u32x4_t*)(out + (size_t)s * K + j0) = u32x4_t{v[0], v[1], v[2], v[3]};
}

}  // namespace

hipError_t launch_gather_cols(const void* in, int div, const int32_t* ids, int E,
                              const int32_t* perm, int K, int slots, int dtype, void* out,
                              hipStream_t stream) {
  (void)dtype;  // 2-byte elements either way
  const size_t total = (size_t)slots * (K / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_cols_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, (const uint16_t*)in, div, ids, E, perm, K, slots, (uint16_t*)out);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const float* partial, int split, int rows, int cols, int dtype,
                               void* out, hipStream_t stream) {
  const size_t total4 = (size_t)rows * cols / 4;
  if (total4 == 0) return hipSuccess;
  const unsigned grid = (unsigned)((total4 + 255) / 256);
  const size_t stride = (size_t)rows * cols;
  if (dtype == 0)
    hipLaunchKernelGGL(split_reduce_kernel<0>, dim3(grid), dim3(256), 0, stream, partial, split,
                       stride, total4, (uint16_t*)out);
  else
    hipLaunchKernelGGL(split_reduce_kernel<1>, dim3(grid), dim3(256), 0, stream, partial, split,
                       stride, total4, (uint16_t*)out);
  return hipGetLastError();
}

hipError_t launch_act_combine(const float* partial, int split, int slots, int I, int dtype,
                              void* inter, hipStream_t stream) {
  if (slots == 0) return hipSuccess;
  const size_t total = (size_t)slots * (I / 4);
  const unsigned grid = (unsigned)((total + 255) / 256);
  const size_t stride = (size_t)slots * 2 * I;
  if (dtype == 0)
    hipLaunchKernelGGL(act_combine_kernel<0>, dim3(grid), dim3(256), 0, stream, partial, split,
                       stride, slots, I, (uint16_t*)inter);
  else
    hipLaunchKernelGGL(act_combine_kernel<1>, dim3(grid), dim3(256), 0, stream, partial, split,
                       stride, slots, I, (uint16_t*)inter);
  return hipGetLastError();
}

hipError_t launch_combine(const float* partial, int split, const float* topk_w, int M, int topk,
                          int H, int dtype, void* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (topk * split >= 16 && H % 256 == 0 && (int64_t)M * (H / 256) <= 1024) {
    const unsigned grid = (unsigned)(M * (H / 256));
    const size_t stride = (size_t)M * topk * H;
    if (dtype == 0)
      hipLaunchKernelGGL(combine_quarters_kernel<0>, dim3(grid), dim3(256), 0, stream, partial,
                         split, stride, topk_w, topk, H, (uint16_t*)out);
    else
      hipLaunchKernelGGL(combine_quarters_kernel<1>, dim3(grid), dim3(256), 0, stream, partial,
                         split, stride, topk_w, topk, H, (uint16_t*)out);
    return hipGetLastError();
  }
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

namespace moe {

hipError_t launch_combine_rows(const void* y, int M, int topk, int H, int dtype, void* out,
                               hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const size_t total = (size_t)M * (H / 8);
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (dtype == 0)
    hipLaunchKernelGGL(combine_rows_kernel<0>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)y, M, topk, H, (uint16_t*)out);
  else
    hipLaunchKernelGGL(combine_rows_kernel<1>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)y, M, topk, H, (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace moe
