// Grouped GEMM over all experts in one launch, weights decoded in registers, for gfx950.
//
// The one-launch grouped GEMM over every expert is the method of "[Kernel] add triton fused moe
// kernel for gptq/awq" (PR description: one launch instead of one per expert); the weight storage
// is the GPTQ/AWQ-compatible uint4 g128 with integer zero points (same PR, review thread; benchmark
// script of "[Kernel] optimize performance of gptq marlin kernel when n is small") or int8 with one
// symmetric scale per output channel (int8 MoE backend listing, w8a16 quant config).  The K step
// of the kernel is always one quantisation group, the invariant whose violation "[Model] Add
// Support for GPTQ Fused MOE" reports as wrong results (bug report in the review thread).
//
// Work decomposition (all sizes in elements):
//   workgroup = 4 wavefronts = one block of BM = 16*MT slots (one expert) x one column chunk
//               x one K split; the block's activation rows are gathered into LDS, KC columns at a time
//   wavefront = NTW column tiles of 16 (with the SiLU epilogue: NTW/2 gate tiles and the matching
//               up tiles, so gate and up of one output sit in the same lane)
//   k-block   = 64 bytes of one weight row: 128 k of uint4 (one quantisation group) or 64 k of
//               int8.  Lane l loads 16 bytes of row (tile column + l % 16) at byte 16*(l / 16):
//               each row is read as a contiguous 64-byte run; the stream is prefetched PF k-blocks
//               ahead in registers.
// MFMA v_mfma_f32_16x16x32_{f16,bf16}: A = 16 activation rows x 32 k, B = 32 k x 16 weight columns.
// A dot product does not depend on the order of k, as long as A and B agree on it; each lane's
// B operand is the 8 weights it decodes itself from one dword of its own 16-byte load (nibble i
// holds k = i), paired (k0,k4) (k1,k5) (k2,k6) (k3,k7) because that pairing is what the shift-and-
// mask decode yields.  The activation tile is stored in LDS with each run of 8 values permuted the
// same way, so no weight ever moves between lanes.
//
// Decoding is exact: the MFMA sees the correctly rounded dtype value of (q - z) * s (fp16: the
// subtraction of two exact half-precision integers 1024+q and 1024+z, then one rounded multiply;
// bf16: an exact float32 fma of 128+q against s and -(128+z)*s, then one rounding to bf16).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

template <int DT>
struct Mfma;
template <>
struct Mfma<0> {
  static __device__ __forceinline__ floatx4_t run(u32x4_t a, u32x4_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<1> {
  static __device__ __forceinline__ floatx4_t run(u32x4_t a, u32x4_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

// Per-lane, per-tile decode constants of one k-block.
struct DecodeK {
  uint32_t s2;   // fp16: scale in both halves
  uint32_t zn2;  // fp16: -(1024 + z) in both halves
  float sf;      // bf16: scale as float
  float cf;      // bf16: -(magic + z) * scale (exact)
};

template <int DT, int BITS>
__device__ __forceinline__ DecodeK make_decode(uint32_t sbits, uint32_t z) {
  DecodeK d;
  if constexpr (DT == 0) {
    d.s2 = sbits | (sbits << 16);
    if constexpr (BITS == 4) {
      const uint32_t zb = __builtin_bit_cast(uint16_t, (_Float16)(-(1024.0f + (float)z)));
      d.zn2 = zb | (zb << 16);
    } else {
      const uint32_t zb = __builtin_bit_cast(uint16_t, (_Float16)(-1152.0f));
      d.zn2 = zb | (zb << 16);
    }
    d.sf = 0.0f;
    d.cf = 0.0f;
  } else {
    d.sf = __uint_as_float(sbits << 16);
    d.cf = (BITS == 4) ? -(128.0f + (float)z) * d.sf : -128.0f * d.sf;
    d.s2 = 0;
    d.zn2 = 0;
  }
  return d;
}

__device__ __forceinline__ uint32_t h2_sub_mul(uint32_t t, uint32_t zn2, uint32_t s2) {
  const half2_t r = (__builtin_bit_cast(half2_t, t) + __builtin_bit_cast(half2_t, zn2)) *
                    __builtin_bit_cast(half2_t, s2);
  return __builtin_bit_cast(uint32_t, r);
}

// uint4: 8 nibbles of one dword (nibble i = k offset i) -> B operand, pairs (0,4)(1,5)(2,6)(3,7)
template <int DT>
__device__ __forceinline__ u32x4_t decode_u4(uint32_t w, const DecodeK& d) {
  u32x4_t b;
  if constexpr (DT == 0) {
    const uint32_t M = 0x64006400u;  // fp16 1024 in both halves
    b[0] = h2_sub_mul((w & 0x000F000Fu) | M, d.zn2, d.s2);
    b[1] = h2_sub_mul(((w >> 4) & 0x000F000Fu) | M, d.zn2, d.s2);
    b[2] = h2_sub_mul(((w >> 8) & 0x000F000Fu) | M, d.zn2, d.s2);
    b[3] = h2_sub_mul(((w >> 12) & 0x000F000Fu) | M, d.zn2, d.s2);
  } else {
    const uint32_t M = 0x43000000u;  // float 128; nibble at bits 16..19 adds q
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(((w << (16 - 4 * i)) & 0x000F0000u) | M);
      const float hi = __uint_as_float(((w >> (4 * i)) & 0x000F0000u) | M);
      b[i] = f32x2_to_bf16x2(__builtin_fmaf(lo, d.sf, d.cf), __builtin_fmaf(hi, d.sf, d.cf));
    }
  }
  return b;
}

// int8: two dwords (bytes = k offsets 0..7) -> B operand in natural order
template <int DT>
__device__ __forceinline__ u32x4_t decode_s8(uint32_t lo, uint32_t hi, const DecodeK& d) {
  u32x4_t b;
  const uint32_t ulo = lo ^ 0x80808080u;  // q + 128, unsigned
  const uint32_t uhi = hi ^ 0x80808080u;
  if constexpr (DT == 0) {
    const uint32_t C = 0x64646464u;  // high byte of fp16 1024 + u
    b[0] = h2_sub_mul(__builtin_amdgcn_perm(C, ulo, 0x04010400u), d.zn2, d.s2);
    b[1] = h2_sub_mul(__builtin_amdgcn_perm(C, ulo, 0x04030402u), d.zn2, d.s2);
    b[2] = h2_sub_mul(__builtin_amdgcn_perm(C, uhi, 0x04010400u), d.zn2, d.s2);
    b[3] = h2_sub_mul(__builtin_amdgcn_perm(C, uhi, 0x04030402u), d.zn2, d.s2);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t u = i == 0 ? ulo : uhi;
      const float f0 = (float)(u & 0xFFu);
      const float f1 = (float)((u >> 8) & 0xFFu);
      const float f2 = (float)((u >> 16) & 0xFFu);
      const float f3 = (float)(u >> 24);
      b[2 * i] = f32x2_to_bf16x2(__builtin_fmaf(f0, d.sf, d.cf), __builtin_fmaf(f1, d.sf, d.cf));
      b[2 * i + 1] = f32x2_to_bf16x2(__builtin_fmaf(f2, d.sf, d.cf), __builtin_fmaf(f3, d.sf, d.cf));
    }
  }
  return b;
}

template <int MT>
struct Shape {
  static constexpr int BM = 16 * MT;
  static constexpr int KC = MT == 1 ? 1024 : (MT == 2 ? 512 : (MT == 4 ? 256 : 128));
  static constexpr int LDA = KC + 8;  // LDS row stride in 16-bit elements (16-byte pad)
  static constexpr int PF = MT <= 2 ? 4 : 2;
};

template <int DT, int BITS, int MT, int NTW, int ACT, int OUTF32>
__global__ void __launch_bounds__(kThreads) wna16_gemm_kernel(GemmParams p) {
  using S = Shape<MT>;
  constexpr int BM = S::BM;
  constexpr int KC = S::KC;
  constexpr int LDA = S::LDA;
  constexpr int PF = S::PF;
  constexpr int KB = BITS == 4 ? 128 : 64;        // k per k-block (64 bytes of a weight row)
  constexpr int STEPS = KB / 32;                    // MFMAs per k-block
  constexpr int KBC = KC / KB;                      // k-blocks per LDS chunk
  constexpr int NOUT = ACT ? NTW / 2 : NTW;         // output tiles per wave
  constexpr int WG_COLS = kWaves * NOUT * 16;

  __shared__ __attribute__((aligned(16))) uint16_t s_a[BM * LDA];
  __shared__ int s_slot[BM];
  __shared__ int s_row[BM];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int N = p.N;
  const int K = p.K;
  const int n_out = ACT ? N / 2 : N;
  const int n_chunks = n_out / WG_COLS;
  const int split = p.split_k;

  int bid = blockIdx.x;
  const int z = bid % split;
  bid /= split;
  const int nc = bid % n_chunks;
  const int blk = bid / n_chunks;
  if (blk * BM >= p.num_post[0]) return;
  const int e = p.expert_ids[blk];
  if ((unsigned)e >= (unsigned)p.E) return;

  if (tid < BM) {
    const int s = p.sorted_ids[blk * BM + tid];
    const bool ok = (unsigned)s < (unsigned)p.num_slots;
    s_slot[tid] = ok ? s : -1;
    s_row[tid] = ok ? s / p.a_row_div : -1;
  }
  __syncthreads();

  // K range of this split, in k-blocks
  const int kb_total = K / KB;
  const int kb_per = (kb_total + split - 1) / split;
  const int kb_beg = z * kb_per;
  const int kb_end = min(kb_total, kb_beg + kb_per);

  // this lane's weight rows
  const int rsub = lane & 15;
  const int grp = lane >> 4;  // 16-byte slice of the 64-byte k-block
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
  const size_t row_bytes = BITS == 4 ? (size_t)K / 2 : (size_t)K;
  const uint8_t* wrow[NTW];
  const uint16_t* srow[NTW];
  const uint8_t* zrow[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const size_t n = (size_t)e * N + col[t] + rsub;
    wrow[t] = p.B + n * row_bytes + grp * 16;
    if constexpr (BITS == 4) {
      srow[t] = (const uint16_t*)p.scales + n * (K / 128);
      zrow[t] = p.zeros + n * (K / 256);
    } else {
      srow[t] = (const uint16_t*)p.scales + n;
      zrow[t] = nullptr;
    }
  }

  u32x4_t wq[PF][NTW];
  uint32_t sq[PF][NTW];
  uint32_t zq[PF][NTW];
  auto load_kb = [&](int slot, int kb) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      wq[slot][t] = *(const u32x4_t*)(wrow[t] + (size_t)kb * 64);
      if constexpr (BITS == 4) {
        sq[slot][t] = srow[t][kb];
        zq[slot][t] = zrow[t][kb >> 1];
      }
    }
  };

  DecodeK dk8[NTW];
  if constexpr (BITS == 8) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) dk8[t] = make_decode<DT, 8>(srow[t][0], 0);
  }

  floatx4_t acc[MT][NTW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (kb_beg + u < kb_end) load_kb(u, kb_beg + u);

  for (int kb0 = kb_beg; kb0 < kb_end; kb0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kb = kb0 + u;
      if (kb >= kb_end) break;
      const int kbl = (kb - kb_beg) % KBC;
      if (kbl == 0) {
        // gather the block's activation rows for the next KC columns into LDS
        __syncthreads();
        const int k0 = kb * KB;
        const int kc_len = min(KC, (kb_end - kb) * KB);
        const int vec_per_row = kc_len / 8;
        for (int i = tid; i < BM * vec_per_row; i += kThreads) {
          const int r = i / vec_per_row;
          const int c8 = i - r * vec_per_row;
          const int row = s_row[r];
          u32x4_t v = {0u, 0u, 0u, 0u};
          if (row >= 0)
            v = *(const u32x4_t*)((const uint16_t*)p.A + (size_t)row * K + k0 + c8 * 8);
          if constexpr (BITS == 4) {
            // (x0..x7) -> (x0,x4,x1,x5,x2,x6,x3,x7), the decode's k pairing
            const u32x4_t o = {__builtin_amdgcn_perm(v[2], v[0], 0x05040100u),
                               __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
                               __builtin_amdgcn_perm(v[3], v[1], 0x05040100u),
                               __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
            v = o;
          }
          *(u32x4_t*)&s_a[r * LDA + c8 * 8] = v;
        }
        __syncthreads();
      }

      DecodeK dk[NTW];
      if constexpr (BITS == 4) {
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          dk[t] = make_decode<DT, 4>(sq[u][t], (zq[u][t] >> ((kb & 1) * 4)) & 0xFu);
      }
      const uint16_t* abase = &s_a[rsub * LDA + kbl * KB + grp * (KB / 4)];
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        u32x4_t a[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) a[m] = *(const u32x4_t*)(abase + m * 16 * LDA + s * 8);
        u32x4_t b[NTW];
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          if constexpr (BITS == 4)
            b[t] = decode_u4<DT>(wq[u][t][s], dk[t]);
          else
            b[t] = decode_s8<DT>(wq[u][t][2 * s], wq[u][t][2 * s + 1], dk8[t]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int t = 0; t < NTW; ++t) acc[m][t] = Mfma<DT>::run(a[m], b[t], acc[m][t]);
      }
      if (kb + PF < kb_end) load_kb(u, kb + PF);
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+i of each 16-row tile, column lane%16
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m * 16 + grp * 4 + i;
      const int slot = s_slot[r];
      if (slot < 0) continue;
      const float wscale = p.topk_w ? p.topk_w[slot] : 1.0f;
#pragma unroll
      for (int t = 0; t < NOUT; ++t) {
        const int c = col[t] + rsub;
        if constexpr (ACT) {
          const float g = acc[m][t][i];
          const float up = acc[m][t + NOUT][i];
          const float v = g / (1.0f + __expf(-g)) * up * wscale;
          ((uint16_t*)p.C)[(size_t)slot * (N / 2) + c] = float_to_bits<DT>(v);
        } else if constexpr (OUTF32) {
          ((float*)p.C)[((size_t)z * p.num_slots + slot) * N + c] = acc[m][t][i] * wscale;
        } else {
          ((uint16_t*)p.C)[(size_t)slot * N + c] = float_to_bits<DT>(acc[m][t][i] * wscale);
        }
      }
    }
  }
}

constexpr int kNTW = 2;

template <int DT, int BITS, int MT>
hipError_t launch_mt(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
  const int n_out = c.act ? p.N / 2 : p.N;
  const int n_chunks = n_out / gemm_wg_cols(c);
  const long long grid = (long long)n_chunks * p.num_blocks * p.split_k;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (c.act)
    hipLaunchKernelGGL((wna16_gemm_kernel<DT, BITS, MT, kNTW, 1, 0>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, p);
  else if (c.out_f32)
    hipLaunchKernelGGL((wna16_gemm_kernel<DT, BITS, MT, kNTW, 0, 1>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((wna16_gemm_kernel<DT, BITS, MT, kNTW, 0, 0>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int DT, int BITS>
hipError_t launch_bits(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
  switch (c.block_m) {
    case 16: return launch_mt<DT, BITS, 1>(p, c, stream);
    case 32: return launch_mt<DT, BITS, 2>(p, c, stream);
    case 64: return launch_mt<DT, BITS, 4>(p, c, stream);
    case 128: return launch_mt<DT, BITS, 8>(p, c, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_wg_cols(const GemmConfig& c) { return kWaves * (c.act ? kNTW / 2 : kNTW) * 16; }

hipError_t launch_gemm(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
  if (c.dtype == 0)
    return c.bits == 4 ? launch_bits<0, 4>(p, c, stream) : launch_bits<0, 8>(p, c, stream);
  return c.bits == 4 ? launch_bits<1, 4>(p, c, stream) : launch_bits<1, 8>(p, c, stream);
}

}  // namespace moe
