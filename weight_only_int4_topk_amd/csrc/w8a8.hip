// w8a8 on gfx950: int8 activations quantised per token at run time, int8 weights with one
// symmetric scale per output channel, products on the integer matrix cores.
//
// The int8 MoE backend listing pairs int8 weights (kInt8StaticChannelSym) with activations
// quantised per token (kInt8DynamicTokenSym; int8_w8a8_moe_quant_config with per_act_token_quant).
// The pages print no formula; the quantisation is the plain symmetric one, decided in float32:
// s = max|x_row| / 127, q = clamp(rint(x / s), -127, 127), rint = round half to even.
//
// GEMM: v_mfma_i32_16x16x64_i8 takes 16 int8 of A and 16 int8 of B per lane.  A lane's B operand is
// its own 16-byte load of one weight row (bytes 16 * (lane / 16) .. of a 64-byte k-block), so the
// weights reach the matrix cores exactly as stored: no decode.  The activation tile is read from
// LDS at the same k offsets, so A and B agree on the k order.  Integer accumulation is exact; the
// epilogue scales by the row's activation scale and the column's weight scale in float32.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcW3 = 0x00020000;  // gfx9-family buffer descriptor: 32-bit data format

// one wavefront per row, four rows per workgroup; K % 512 == 0 is not required (K % 256 == 0)
template <int DT>
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* __restrict__ x, int rows,
                                                         int K, int8_t* __restrict__ q,
                                                         float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * 4 + (int)(threadIdx.x / kWave);
  if (row >= rows) return;
  const uint16_t* xr = x + (size_t)row * K;
  float amax = 0.0f;
  for (int k = lane * 8; k < K; k += kWave * 8) {
    const u32x4_t v = *(const u32x4_t*)(xr + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      amax = fmaxf(amax, fabsf(bits_to_float<DT>((uint16_t)(w & 0xFFFFu))));
      amax = fmaxf(amax, fabsf(bits_to_float<DT>((uint16_t)(w >> 16))));
    }
  }
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, kWave));
  const float s = amax / 127.0f;  // correctly rounded float32 division
  for (int k = lane * 8; k < K; k += kWave * 8) {
    const u32x4_t v = *(const u32x4_t*)(xr + k);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = v[i / 2];
      const float f = bits_to_float<DT>((uint16_t)(i & 1 ? w >> 16 : w & 0xFFFFu));
      const float r = s > 0.0f ? fminf(fmaxf(__builtin_rintf(f / s), -127.0f), 127.0f) : 0.0f;
      packed[i / 4] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (i % 4));
    }
    *(uint2*)(q + (size_t)row * K + k) = make_uint2(packed[0], packed[1]);
  }
  if (lane == 0) scales[row] = s;
}

template <int DT, int MT, int ACT, int OUTF32, int NTW>
__global__ void __launch_bounds__(256) w8a8_gemm_kernel(W8A8Params p) {
  // NTW column tiles of 16 per wavefront: each activation fragment read from LDS feeds NTW MFMAs
  constexpr int BM = 16 * MT;
  constexpr int KC = 256;                    // k per activation chunk: 4 k-blocks of 64
  constexpr int KBC = KC / 64;
  constexpr int LDA = KC + 16;               // LDS row pitch in bytes (16 rows -> distinct banks)
  constexpr int VPR = KC / 16;               // 16-byte vectors per row chunk
  constexpr int AV = BM * VPR / 256;         // per thread
  static_assert(AV >= 1 && BM * VPR % 256 == 0, "whole vectors per thread");
  constexpr int NOUT = ACT ? NTW / 2 : NTW;
  constexpr int WG_COLS = 4 * NOUT * 16;
  __shared__ __attribute__((aligned(16))) uint8_t s_a0[BM * LDA];
  __shared__ __attribute__((aligned(16))) uint8_t s_a1[BM * LDA];
  __shared__ int s_slot[BM];
  __shared__ float s_as[BM];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int rsub = lane & 15;
  const int grp = lane >> 4;
  const int N = p.N, K = p.K;
  const int n_out = ACT ? N / 2 : N;
  const int n_chunks = n_out / WG_COLS;
  const int nc = blockIdx.x % n_chunks;
  const int blk = blockIdx.x / n_chunks;
  if (blk * BM >= p.num_post[0]) return;
  const int e = p.expert_ids[blk];
  if ((unsigned)e >= (unsigned)p.E) return;
  if (tid < BM) {
    const int s = p.sorted_ids[blk * BM + tid];
    const bool ok = (unsigned)s < (unsigned)p.num_slots;
    s_slot[tid] = ok ? s : -1;
    s_as[tid] = ok ? p.a_scales[s / p.a_row_div] : 0.0f;
  }

  int col[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    if constexpr (ACT) {
      const int g0 = nc * WG_COLS + wave * NOUT * 16;
      col[t] = t < NOUT ? g0 + t * 16 : N / 2 + g0 + (t - NOUT) * 16;
    } else {
      col[t] = nc * WG_COLS + wave * NTW * 16 + t * 16;
    }
  }
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + (size_t)e * N * K), (short)0, (int)((size_t)N * K), kRsrcW3);
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.A, (short)0, (int)((size_t)p.num_a_rows * K), kRsrcW3);
  uint32_t vw[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) vw[t] = (uint32_t)(col[t] + rsub) * K + grp * 16;

  // activation vectors of this thread: row r of the block, 16 bytes at column c16 * 16 of a chunk;
  // rows without a slot read past the end of the buffer, which loads zeros
  uint32_t arow[AV], acol[AV], aoff[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int idx = tid + i * 256;
    const int r = idx / VPR;
    const int c16 = idx - r * VPR;
    const int sl = p.sorted_ids[blk * BM + r];
    const int row = (unsigned)sl < (unsigned)p.num_slots ? sl / p.a_row_div : -1;
    arow[i] = row >= 0 ? (uint32_t)row * K : 0x80000000u;
    acol[i] = c16 * 16;
    aoff[i] = r * LDA + c16 * 16;
  }
  u32x4_t areg[AV];
  auto load_a = [&](int c) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const uint32_t off = arow[i] < 0x80000000u ? arow[i] + c * KC + acol[i] : 0x80000000u;
      areg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_a, off, 0, 0));
    }
  };
  auto store_a = [&](uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < AV; ++i) *(u32x4_t*)(buf + aoff[i]) = areg[i];
  };
  auto load_w = [&](u32x4_t (&w)[NTW], int kb) {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      w[t] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_w, vw[t], kb * 64, 0));
  };

  i32x4_t acc[MT][NTW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[m][t] = i32x4_t{0, 0, 0, 0};

  const int nkb = K / 64;
  const int nchunk = K / KC;
  u32x4_t wcur[NTW], wnext[NTW];
  load_w(wcur, 0);
  load_a(0);
  store_a(s_a0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const bool more = c + 1 < nchunk;
    if (more) load_a(c + 1);
    const uint8_t* abuf = (c & 1) ? s_a1 : s_a0;
#pragma unroll
    for (int j = 0; j < KBC; ++j) {
      const int kb = c * KBC + j;
      load_w(wnext, min(kb + 1, nkb - 1));
      u32x4_t af[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
        af[m] = *(const u32x4_t*)(abuf + (m * 16 + rsub) * LDA + j * 64 + grp * 16);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          acc[m][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, af[m]),
                                                            __builtin_bit_cast(i32x4_t, wcur[t]),
                                                            acc[m][t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NTW; ++t) wcur[t] = wnext[t];
    }
    // the other buffer was last read in chunk c - 1, before the barrier that ended it
    if (more) store_a((c & 1) ? s_a0 : s_a1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4 * (lane / 16) + i of each 16-row tile, column lane % 16
  const uint16_t* wsc = (const uint16_t*)p.w_scales + (size_t)e * N;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m * 16 + grp * 4 + i;
      const int slot = s_slot[r];
      if (slot < 0) continue;
      const float sa = s_as[r];
      const float wscale = p.topk_w ? p.topk_w[slot] : 1.0f;
#pragma unroll
      for (int t = 0; t < NOUT; ++t) {
        const int cc = col[t] + rsub;
        if constexpr (ACT) {
          const float g = (float)acc[m][t][i] * sa * bits_to_float<DT>(wsc[cc]);
          const float u = (float)acc[m][t + NOUT][i] * sa * bits_to_float<DT>(wsc[N / 2 + cc]);
          ((uint16_t*)p.C)[(size_t)slot * (N / 2) + cc] =
              float_to_bits<DT>(g / (1.0f + __expf(-g)) * u * wscale);
        } else if constexpr (OUTF32) {
          const float v = (float)acc[m][t][i] * sa * bits_to_float<DT>(wsc[cc]);
          ((float*)p.C)[(size_t)slot * N + cc] = v * wscale;
        } else {
          const float v = (float)acc[m][t][i] * sa * bits_to_float<DT>(wsc[cc]);
          ((uint16_t*)p.C)[(size_t)slot * N + cc] = float_to_bits<DT>(v * wscale);
        }
      }
    }
  }
}

template <int DT, int MT, int NTW>
hipError_t launch_w8a8_ntw(const W8A8Params& p, int act, int out_f32, hipStream_t stream) {
  const int n_out = act ? p.N / 2 : p.N;
  const int wg_cols = 4 * (act ? NTW / 2 : NTW) * 16;
  const long long grid = (long long)(n_out / wg_cols) * p.num_blocks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (act)
    hipLaunchKernelGGL((w8a8_gemm_kernel<DT, MT, 1, 0, NTW>), dim3((unsigned)grid), dim3(256), 0,
                       stream, p);
  else if (out_f32)
    hipLaunchKernelGGL((w8a8_gemm_kernel<DT, MT, 0, 1, NTW>), dim3((unsigned)grid), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((w8a8_gemm_kernel<DT, MT, 0, 0, NTW>), dim3((unsigned)grid), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

// The SiLU GEMM takes four column tiles per wavefront where its gate columns divide the wider
// workgroup (each activation fragment then feeds four MFMAs instead of two: DeepSeek-V3 int8
// experts with 64-row blocks at M = 4096, 3012 -> 2852 us; at M = 1024, where the weight stream
// bounds it, the two are equal); the plain GEMM keeps two (with four, H = 7168 gives half as many
// workgroups and the M = 1024 layer measured 4 % slower).  128-row blocks keep two: eight row
// tiles already reuse each fragment, and registers are the limit.
template <int DT, int MT>
hipError_t launch_w8a8_mt(const W8A8Params& p, int act, int out_f32, hipStream_t stream) {
  if constexpr (MT <= 4) {
    if (act && (p.N / 2) % 128 == 0) return launch_w8a8_ntw<DT, MT, 4>(p, act, out_f32, stream);
  }
  return launch_w8a8_ntw<DT, MT, 2>(p, act, out_f32, stream);
}

template <int DT>
hipError_t launch_w8a8_dt(const W8A8Params& p, int block_m, int act, int out_f32,
                          hipStream_t stream) {
  switch (block_m) {
    case 16: return launch_w8a8_mt<DT, 1>(p, act, out_f32, stream);
    case 32: return launch_w8a8_mt<DT, 2>(p, act, out_f32, stream);
    case 64: return launch_w8a8_mt<DT, 4>(p, act, out_f32, stream);
    case 128: return launch_w8a8_mt<DT, 8>(p, act, out_f32, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_quant_rows(const void* x, int rows, int K, int dtype, int8_t* q, float* scales,
                             hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (dtype == 0)
    hipLaunchKernelGGL(quant_rows_kernel<0>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)x, rows, K, q, scales);
  else
    hipLaunchKernelGGL(quant_rows_kernel<1>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)x, rows, K, q, scales);
  return hipGetLastError();
}

hipError_t launch_w8a8_gemm(const W8A8Params& p, int block_m, int act, int dtype,
                            hipStream_t stream, int out_f32) {
  if (w8a8_mma32_fits(block_m, act, p.N))
    return launch_w8a8_mma32(p, block_m, act, dtype, out_f32, stream);
  return dtype == 0 ? launch_w8a8_dt<0>(p, block_m, act, out_f32, stream)
                    : launch_w8a8_dt<1>(p, block_m, act, out_f32, stream);
}

}  // namespace moe
