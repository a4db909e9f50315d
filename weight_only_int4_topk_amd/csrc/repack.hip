// GPTQ / AWQ checkpoint storage -> the canonical uint4 storage of this library, on the device.
//
// "[Kernel] add triton fused moe kernel for gptq/awq" (review thread) asks for a weight format that
// accepts GPTQ and AWQ checkpoints; the small-n GEMM of "[Kernel] optimize performance of gptq
// marlin kernel when n is small" takes GPTQ's g_idx and sort_indices.  The pages print neither
// checkpoint's packing; the layouts read here are the ones those checkpoint families ship, per
// expert (codes q, zero points z, scales s; decoded weight (q - z) * s):
//   GPTQ: qweight int32 [K/8, N], code (k, n) in bits 4 (k % 8) of word [k / 8, n];
//         qzeros int32 [K/128, N/8], zero (g, n) in bits 4 (n % 8) of word [g, n / 8];
//         scales [K/128, N]; optional g_idx int32 [K] (act-order: group of input column k).
//   AWQ:  qweight int32 [K, N/8], code (k, n) in nibble j of word [k, n / 8] with n % 8 =
//         (0, 2, 4, 6, 1, 3, 5, 7)[j]; qzeros int32 [K/128, N/8] packed the same way.
// Canonical: B uint8 [N, K/2] (byte j = k 2j low, 2j + 1 high), scales [N, K/128], zeros uint8
// [N, K/256] (byte j = group 2j low, 2j + 1 high).  With g_idx the columns are stored in the order
// of perm = stable argsort(g_idx) (each group contiguous), the act-order layer's sorted storage.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// column c of an AWQ word sits in nibble kAwqPos[c]
__constant__ int kAwqPos[8] = {0, 4, 1, 5, 2, 6, 3, 7};

// perm[e, 128 g + r] = the r-th input column (ascending) whose g_idx is g; a group with fewer than
// 128 columns is padded with K (a column no activation row has, read as zero by the act-order
// layer); columns past a full group, or with g_idx outside [0, K/128), are left out.  Both count
// in *invalid.  One workgroup per expert: the group ids go to LDS, then thread g scans them.
__global__ void __launch_bounds__(256) repack_perm_kernel(const int32_t* __restrict__ g_idx, int K,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ invalid) {
  extern __shared__ uint16_t s_g[];
  const int e = blockIdx.x;
  const int G = K / 128;
  const int32_t* gi = g_idx + (size_t)e * K;
  int bad = 0;
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    const int g = gi[k];
    const bool ok = g >= 0 && g < G;
    s_g[k] = ok ? (uint16_t)g : (uint16_t)0xFFFF;
    bad += ok ? 0 : 1;
  }
  __syncthreads();
  int32_t* pe = perm + (size_t)e * K;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    int cnt = 0;
    for (int k = 0; k < K; ++k) {
      if (s_g[k] == g) {
        if (cnt < 128) pe[128 * g + cnt] = k;
        ++cnt;
      }
    }
    for (int r = cnt; r < 128; ++r) pe[128 * g + r] = K;
    bad += cnt > 128 ? cnt - 128 : 128 - cnt;
  }
  if (invalid && bad) atomicAdd(invalid, bad);
}

// Codes: one 32-bit word of canonical storage = 8 codes of row n at columns 8 j8 .. 8 j8 + 7 (of
// the stored order).  A workgroup covers 64 rows x 64 words: it gathers the codes with consecutive
// threads on consecutive n (the checkpoint's fast axis), transposes through LDS, and writes with
// consecutive threads on consecutive words (the canonical fast axis).
template <int FMT, int PERM>
__global__ void __launch_bounds__(256) repack_codes_kernel(const uint32_t* __restrict__ qweight,
                                                           const int32_t* __restrict__ perm, int N,
                                                           int K, uint32_t* __restrict__ out) {
  __shared__ uint32_t tile[64][65];
  const int e = blockIdx.z;
  const int n0 = blockIdx.y * 64;
  const int w0 = blockIdx.x * 64;
  const int KW = K / 8;  // words per canonical row
  const uint32_t* qw = qweight + (size_t)e * K * N / 8;
  const int32_t* pe = PERM ? perm + (size_t)e * K : nullptr;
  const int tn = threadIdx.x & 63;
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {
    const int j8 = w0 + r;
    const int n = n0 + tn;
    uint32_t word = 0;
    if (j8 < KW && n < N) {
      if (FMT == 0 && !PERM) {
        word = qw[(size_t)j8 * N + n];  // a GPTQ word already holds k = 8 j8 + i in nibble i
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = PERM ? pe[8 * j8 + i] : 8 * j8 + i;
          uint32_t q = 0;
          if (k >= 0 && k < K) {
            if (FMT == 0) q = (qw[(size_t)(k >> 3) * N + n] >> (4 * (k & 7))) & 0xFu;
            else q = (qw[(size_t)k * (N / 8) + (n >> 3)] >> (4 * kAwqPos[n & 7])) & 0xFu;
          }
          word |= q << (4 * i);
        }
      }
    }
    tile[r][tn] = word;
  }
  __syncthreads();
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {
    const int n = n0 + r;
    const int j8 = w0 + tn;
    if (n < N && j8 < KW) out[((size_t)e * N + n) * KW + j8] = tile[tn][r];
  }
}

// Scales and zero points: thread (e, n, j) writes scales of groups 2j, 2j + 1 and zero byte j of
// row n (consecutive threads on consecutive n read consecutive checkpoint entries).
template <int FMT>
__global__ void __launch_bounds__(256) repack_meta_kernel(const uint16_t* __restrict__ scales,
                                                          const uint32_t* __restrict__ qzeros, int N,
                                                          int G, uint16_t* __restrict__ s_out,
                                                          uint8_t* __restrict__ z_out) {
  const int e = blockIdx.z;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int j = blockIdx.y;
  if (n >= N) return;
  const uint16_t* se = scales + (size_t)e * G * N;
  const uint32_t* ze = qzeros + (size_t)e * G * (N / 8);
  const int pos = FMT == 0 ? (n & 7) : kAwqPos[n & 7];
  uint32_t zz = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = 2 * j + h;
    s_out[((size_t)e * N + n) * G + g] = se[(size_t)g * N + n];
    zz |= ((ze[(size_t)g * (N / 8) + (n >> 3)] >> (4 * pos)) & 0xFu) << (4 * h);
  }
  z_out[((size_t)e * N + n) * (G / 2) + j] = (uint8_t)zz;
}

}  // namespace

hipError_t launch_repack_uint4(int format, const int32_t* qweight, const int32_t* qzeros,
                               const void* scales, const int32_t* g_idx, int E, int N, int K,
                               uint8_t* B, void* scales_out, uint8_t* zeros_out, int32_t* perm_out,
                               int32_t* invalid, hipStream_t stream) {
  const int G = K / 128;
  if (g_idx) {
    hipLaunchKernelGGL(repack_perm_kernel, dim3(E), dim3(256), (size_t)K * sizeof(uint16_t), stream,
                       g_idx, K, perm_out, invalid);
    if (hipError_t err = hipGetLastError()) return err;
  }
  const dim3 gc((unsigned)((K / 8 + 63) / 64), (unsigned)((N + 63) / 64), (unsigned)E);
  const uint32_t* qw = (const uint32_t*)qweight;
  uint32_t* out = (uint32_t*)B;
  if (format == 0) {
    if (g_idx)
      hipLaunchKernelGGL((repack_codes_kernel<0, 1>), gc, dim3(256), 0, stream, qw, perm_out, N, K, out);
    else
      hipLaunchKernelGGL((repack_codes_kernel<0, 0>), gc, dim3(256), 0, stream, qw, perm_out, N, K, out);
  } else {
    hipLaunchKernelGGL((repack_codes_kernel<1, 0>), gc, dim3(256), 0, stream, qw, perm_out, N, K, out);
  }
  if (hipError_t err = hipGetLastError()) return err;
  const dim3 gm((unsigned)((N + 255) / 256), (unsigned)(G / 2), (unsigned)E);
  if (format == 0)
    hipLaunchKernelGGL((repack_meta_kernel<0>), gm, dim3(256), 0, stream, (const uint16_t*)scales,
                       (const uint32_t*)qzeros, N, G, (uint16_t*)scales_out, zeros_out);
  else
    hipLaunchKernelGGL((repack_meta_kernel<1>), gm, dim3(256), 0, stream, (const uint16_t*)scales,
                       (const uint32_t*)qzeros, N, G, (uint16_t*)scales_out, zeros_out);
  return hipGetLastError();
}

}  // namespace moe
