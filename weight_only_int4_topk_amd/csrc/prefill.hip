// Grouped GEMM over all experts for the prefill regime (block_m 128 and 256) on the 32 x 32 matrix
// cores of gfx950.
//
// The same operation as wna16_gemm_kernel (one launch over every expert, "[Kernel] add triton
// fused moe kernel for gptq/awq", PR description; uint4 g128 with integer zero points or int8 with
// one scale per output channel; the K step is one quantisation group), tiled for large blocks:
// here the matrix cores bound the kernel, and on gfx950 v_mfma_f32_32x32x16_{f16,bf16} retires
// twice the flops per cycle of the 16 x 16 x 32 form (measured: 2.40 against 1.35 PFLOP/s for a
// stream of independent bf16 MFMAs on all 256 compute units).
//
// Work decomposition:
//   workgroup = WAVES wavefronts = one block of BM = 32 MT slots (one expert) x one column chunk x
//               one K split.  The block's activation rows go from memory straight into LDS, one k-block
//               at a time, double-buffered.
//   wavefront = NT column tiles of 32 weight rows (with the SiLU epilogue: a gate tile and the
//               matching up tile, or at NT = 1 one mixed tile of 16 gate rows and the 16 matching
//               up rows), every row tile of the block.
//   k-block   = 64 bytes of a weight row: 128 k of uint4 (one group) or 64 k of int8.  Lane l of a
//               column tile loads 32 bytes of row (l % 32) at byte 32 (l / 32), so lane half h
//               covers k in [64 h, 64 h + 64) (int8: [32 h, 32 h + 32)) of the k-block.
// MFMA step s of a k-block (16 k): lane half h supplies k = 64 h + 8 s + (0..7) (int8: 32 h + 8 s +
// (0..7)) of its weight column (B) and of its activation row (A), in natural order.  Matrix-core
// operand layout (gfx950, 32x32x16): A lane l = row l % 32, k 8 (l / 32) .. + 7 of the step; B lane
// l = column l % 32, same k; result register i of lane l = row 8 (i / 4) + 4 (l / 32) + i % 4,
// column l % 32.
//
// Decoding: each lane turns the 8 nibbles (or bytes) of one dword of its own load into the dtype
// values (q - z) * s in natural k order: a byte-to-float conversion per weight, one exact float32
// fma against s and -z * s (4- or 8-bit codes times an 8- or 11-bit scale), one rounding to the
// dtype, so the matrix cores see the correctly rounded decoded weight for fp16 and bf16 alike.  A
// decoded column tile serves every row tile of the block (MT of them), which is what keeps the
// decode's vector instructions below the matrix-core time once the block is full.
//
// Row tiles past the block's last listed slot (the tail of an expert's last block) are skipped.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kRsrc3 = 0x00020000;  // gfx9-family buffer descriptor: 32-bit data format

typedef float floatx16_t __attribute__((ext_vector_type(16)));

template <int DT>
struct Mfma32;
template <>
struct Mfma32<0> {
  static __device__ __forceinline__ floatx16_t run(u32x4_t a, u32x4_t b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma32<1> {
  static __device__ __forceinline__ floatx16_t run(u32x4_t a, u32x4_t b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return DT == 0 ? f32x2_to_f16x2(lo, hi) : f32x2_to_bf16x2(lo, hi);
}

// uint4: the 8 nibbles of w (nibble i = k offset i) as 4 dtype pairs (k0,k1) (k2,k3) (k4,k5)
// (k6,k7); sf = s, cf = -z * s.  The masks go through v_bitop3_b32 so that every nibble sits in a
// byte of its own and converts with one v_cvt_f32_ubyte.
template <int DT>
__device__ __forceinline__ u32x4_t decode_nat_u4(uint32_t w, float sf, float cf) {
  const uint32_t even = __builtin_amdgcn_bitop3_b32(w, 0x0F0F0F0Fu, 0u, 0xC0);       // w & m
  const uint32_t odd = __builtin_amdgcn_bitop3_b32(w >> 4, 0x0F0F0F0Fu, 0u, 0xC0);  // (w >> 4) & m
  u32x4_t b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float q0 = (float)((even >> (8 * i)) & 0xFFu);
    const float q1 = (float)((odd >> (8 * i)) & 0xFFu);
    b[i] = pack2<DT>(__builtin_fmaf(q0, sf, cf), __builtin_fmaf(q1, sf, cf));
  }
  return b;
}

// int8: two dwords (byte i = k offset i) as 4 dtype pairs in natural order; codes are read as
// q + 128 (unsigned bytes) and cf = -128 * s.
template <int DT>
__device__ __forceinline__ u32x4_t decode_nat_s8(uint32_t lo, uint32_t hi, float sf, float cf) {
  const uint32_t u[2] = {lo ^ 0x80808080u, hi ^ 0x80808080u};
  u32x4_t b;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float f0 = (float)(u[i] & 0xFFu);
    const float f1 = (float)((u[i] >> 8) & 0xFFu);
    const float f2 = (float)((u[i] >> 16) & 0xFFu);
    const float f3 = (float)(u[i] >> 24);
    b[2 * i] = pack2<DT>(__builtin_fmaf(f0, sf, cf), __builtin_fmaf(f1, sf, cf));
    b[2 * i + 1] = pack2<DT>(__builtin_fmaf(f2, sf, cf), __builtin_fmaf(f3, sf, cf));
  }
  return b;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_p() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS-only workgroup barrier: global loads in flight stay in flight across it
__device__ __forceinline__ void barrier_lds_p() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int DT, int BITS, int MT, int NT, int WAVES, int NBUF, int ACT, int OUTF32>
__global__ void __launch_bounds__(WAVES * 64, 2) prefill_gemm_kernel(GemmParams p) {
  constexpr int THREADS = WAVES * kWave;
  constexpr int BM = 32 * MT;
  constexpr int KB = BITS == 4 ? 128 : 64;        // k per k-block: 64 bytes of a weight row
  constexpr int STEPS = KB / 16;                  // 32x32x16 MFMAs per k-block and tile pair
  constexpr int VPR = KB / 8;                     // 16-byte chunks of an activation row per k-block
  constexpr int AV = BM * VPR / THREADS;          // direct-to-LDS loads per thread per k-block
  static_assert(AV >= 1 && BM * VPR % THREADS == 0, "whole activation chunks per thread");
  // SiLU epilogue: gate and up tiles in pairs, or (one tile per wavefront) a mixed tile whose
  // lanes 0-15 hold 16 gate rows and lanes 16-31 the matching up rows
  static_assert(!ACT || NT % 2 == 0 || NT == 1, "SiLU epilogue: paired or mixed tiles");
  constexpr bool MIXED = ACT && NT == 1;
  constexpr int NOUT = ACT ? (MIXED ? 1 : NT / 2) : NT;
  constexpr int TCOLS = MIXED ? 16 : 32;          // output columns of a column tile
  constexpr int WG_COLS = WAVES * NOUT * TCOLS;   // output columns of a workgroup
  static_assert(NBUF == 2 || NBUF == 3, "two or three activation buffers");
  // k-blocks per unrolled iteration: every buffer and weight slot index a compile-time constant
  constexpr int U = NBUF == 3 ? 6 : 2;
  // loads per lane and k-block issued with the weights: 2 per column tile (32 bytes), and for uint4
  // the tile's scale and zero-point byte
  constexpr int LPK = BITS == 4 ? 4 * NT : 2 * NT;

  // the two activation buffers are separate variables, so the compiler can tell a direct load into
  // one from fragment reads of the other (with one array it waits for every load in flight first);
  // every access names its buffer at compile time (two k-blocks per unrolled iteration)
  __shared__ __attribute__((aligned(16))) uint16_t s_a0[BM * KB];
  __shared__ __attribute__((aligned(16))) uint16_t s_a1[BM * KB];
  __shared__ __attribute__((aligned(16))) uint16_t s_a2[NBUF == 3 ? BM * KB : 8];
  auto abuf_of = [&](int b) -> uint16_t* { return b == 0 ? s_a0 : (b == 1 ? s_a1 : s_a2); };
  __shared__ int s_slot[BM];
  // 16-byte chunk j of activation row r sits at chunk j ^ swz(r): the 16 rows of a fragment read
  // (same logical chunk) land on 16 different bank groups
  auto swz = [](int r) -> int { return VPR == 16 ? (r & 15) : ((r >> 1) & 7); };

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
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
  int e, n_valid_b = 0, brow0 = 0;
  if (p.batched) {
    e = blk / p.bpe;
    const int j = blk - e * p.bpe;
    n_valid_b = min(p.expert_counts[e], p.max_tokens) - j * BM;
    if (n_valid_b <= 0) return;
    brow0 = e * p.max_tokens + j * BM;
  } else {
    if (blk * BM >= (p.dense ? p.num_slots : p.num_post[0])) return;
    e = p.dense ? 0 : p.expert_ids[blk];
  }
  if ((unsigned)e >= (unsigned)p.E) return;
  auto slot_at = [&](int i) -> int {
    if (p.batched) {
      const int r = i - blk * BM;
      return r < n_valid_b ? brow0 + r : -1;
    }
    return p.dense ? (i < p.num_slots ? i : -1) : p.sorted_ids[i];
  };
  if (tid < BM) {
    const int s = slot_at(blk * BM + tid);
    s_slot[tid] = (unsigned)s < (unsigned)p.num_slots ? s : -1;
  }

  const int kb_total = K / KB;
  const int kb_per = (kb_total + split - 1) / split;
  const int kb_beg = z * kb_per;
  const int kb_end = min(kb_total, kb_beg + kb_per);
  const int kb_last = min(max(kb_beg, kb_end - 1), kb_total - 1);

  const int c32 = lane & 31;
  const int h = lane >> 5;
  // col[t]: first output column of tile t (of the gate half with the SiLU epilogue); wrow[t]: the
  // weight row lane l streams for tile t
  auto col_of = [&](int t) -> int {
    if constexpr (MIXED) {
      return nc * WG_COLS + wave * 16;
    } else if constexpr (ACT) {
      const int g0 = nc * WG_COLS + wave * NOUT * 32;
      return t < NOUT ? g0 + t * 32 : N / 2 + g0 + (t - NOUT) * 32;
    } else {
      return nc * WG_COLS + (wave * NT + t) * 32;
    }
  };
  int col[NT], wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    col[t] = col_of(t);
    if constexpr (MIXED) wrow[t] = c32 < 16 ? col[t] + c32 : N / 2 + col[t] + (c32 - 16);
    else wrow[t] = col[t] + c32;
  }

  const uint32_t row_bytes = BITS == 4 ? (uint32_t)K / 2 : (uint32_t)K;
  const uint32_t srow_bytes = BITS == 4 ? (uint32_t)(K / 128) * 2 : 2u;
  const uint32_t zrow_bytes = (uint32_t)(K / 256);
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + (size_t)e * N * row_bytes), (short)0, (int)(N * row_bytes), kRsrc3);
  const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)p.scales + (size_t)e * N * srow_bytes), (short)0,
      (int)(N * srow_bytes), kRsrc3);
  const __amdgpu_buffer_rsrc_t rs_z = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(BITS == 4 ? p.zeros + (size_t)e * N * zrow_bytes : p.zeros), (short)0,
      BITS == 4 ? (int)(N * zrow_bytes) : 0, kRsrc3);
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.A, (short)0, (int)((size_t)p.num_a_rows * K * 2), kRsrc3);
  uint32_t vw[NT], vs[NT], vz[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t n = (uint32_t)wrow[t];
    vw[t] = n * row_bytes + h * 32;
    vs[t] = n * srow_bytes;
    vz[t] = n * zrow_bytes;
  }

  // ---- activation k-block c straight into LDS buffer b.  Lane l of wave w writes the 16 bytes of
  // slot idx = w * 64 + l + i * THREADS of the unpadded tile, i.e. (row idx / VPR, physical chunk
  // idx % VPR), which holds logical chunk (idx % VPR) ^ swz(row).  Padding rows and k past this
  // split's range read past the end of the buffer, which loads zeros.
  // slot idx = tid + i * THREADS: row tid / VPR + i * THREADS / VPR, physical chunk tid % VPR;
  // swz of that row depends on row % 16 only (or row / 2 % 8), the same for every i, so one
  // column offset serves all of the thread's loads
  static_assert((THREADS / VPR) % 16 == 0, "every load of a thread has the same row swizzle");
  uint32_t arow[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int r = (tid + i * THREADS) / VPR;
    const int sl = slot_at(blk * BM + r);
    const int row = (unsigned)sl < (unsigned)p.num_slots ? (p.a_row_div == 1 ? sl : sl / p.a_row_div) : -1;
    arow[i] = row >= 0 ? (uint32_t)row * K * 2 : 0x80000000u;
  }
  const uint32_t acol = (uint32_t)((tid % VPR) ^ swz(tid / VPR)) * 8;
  const uint32_t klim = (uint32_t)(kb_end * KB);
  auto dma_a = [&](int c, uint16_t* buf) {
    const uint32_t kbase = (uint32_t)((kb_beg + c) * KB);
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const uint32_t k = kbase + acol;
      const uint32_t off = (arow[i] < 0x80000000u && k < klim) ? arow[i] + k * 2 : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_a,
          (__attribute__((address_space(3))) void*)((uint8_t*)buf +
                                                    (size_t)(wave * kWave + i * THREADS) * 16),
          16, off, 0, 0, 0);
    }
  };

  // ---- weights (and uint4 metadata) of one k-block, two k-blocks in flight
  u32x4_t wq[2][NT][2];
  uint32_t ms[2][NT], mz[2][NT];
  auto load_kb = [&](int slot, int kb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wq[slot][t][j] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_w, vw[t] + j * 16, kb * 64, 0));
      if constexpr (BITS == 4) {
        ms[slot][t] = __builtin_amdgcn_raw_buffer_load_b16(rs_s, vs[t], kb * 2, 0);
        mz[slot][t] = __builtin_amdgcn_raw_buffer_load_b8(rs_z, vz[t], kb >> 1, 0);
      }
    }
  };
  float sf8[NT], cf8[NT];
  if constexpr (BITS == 8) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sf8[t] = bits_to_float<DT>(
          (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs_s, (uint32_t)wrow[t] * 2, 0, 0));
      cf8[t] = -128.0f * sf8[t];  // exact: 8-bit times the scale's significand
    }
  }

  floatx16_t acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;

  // ---- prologue.  The loads are ordered as in the steady state of the loop, so its waits hold
  // from the first iteration: in iteration i the weights of k-block i + 2 are requested, then
  // (after the barrier) activation k-block i + NBUF.
  const int nkb = kb_end - kb_beg;
  dma_a(0, s_a0);
  load_kb(0, min(kb_beg, kb_last));
  if constexpr (NBUF == 2) {
    load_kb(1, min(kb_beg + 1, kb_last));
    wait_vmcnt_p<2 * LPK>();   // activation k-block 0 has landed
  } else {
    wait_vmcnt_p<LPK>();
  }
  barrier_lds_p();  // publishes s_slot and k-block 0
  // row tiles holding at least one listed slot (listed slots are a prefix of the block)
  int n_valid = 0;
#pragma unroll
  for (int q = 0; q < BM / kWave; ++q)
    n_valid += __builtin_popcountll(__ballot(s_slot[q * kWave + lane] >= 0));
  const int mt_valid = __builtin_amdgcn_readfirstlane((n_valid + 31) / 32);
  dma_a(1, s_a1);
  if constexpr (NBUF == 3) {
    load_kb(1, min(kb_beg + 1, kb_last));
    dma_a(2, s_a2);
  }

  const int n_iter = (nkb + U - 1) / U;
  // the k loop for MA active row tiles (a compile-time count, so the fragment reads of a step are
  // issued together ahead of its MFMAs)
  auto kloop = [&](auto ma_c) {
    constexpr int MA = decltype(ma_c)::value;
    for (int it = 0; it < n_iter; ++it) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int idx = it * U + j;
        const int kb = kb_beg + idx;
        const int ws = j % 2;                  // weight slot
        const uint16_t* abuf = abuf_of(j % NBUF);
        // k-blocks past the range (the unroll's tail) keep their loads and barriers, not their math
        if (idx < nkb) {
          float sf[NT], cf[NT];
          if constexpr (BITS == 4) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              sf[t] = bits_to_float<DT>((uint16_t)(ms[ws][t] & 0xFFFFu));
              const uint32_t zz = (mz[ws][t] >> ((kb & 1) * 4)) & 0xFu;
              cf[t] = -(float)zz * sf[t];  // exact: 4-bit times the scale's significand
            }
          } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              sf[t] = sf8[t];
              cf[t] = cf8[t];
            }
          }
#pragma unroll
          for (int st = 0; st < STEPS; ++st) {
            const int cl = (BITS == 4 ? 8 * h : 4 * h) + st;  // logical 16-byte chunk of the row
            u32x4_t b[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              if constexpr (BITS == 4)
                b[t] = decode_nat_u4<DT>(wq[ws][t][st / 4][st % 4], sf[t], cf[t]);
              else
                b[t] = decode_nat_s8<DT>(wq[ws][t][st / 2][(2 * st) % 4],
                                         wq[ws][t][st / 2][(2 * st) % 4 + 1], sf[t], cf[t]);
            }
#pragma unroll
            for (int m = 0; m < MA; ++m) {
              const int row = m * 32 + c32;
              const u32x4_t a = *(const u32x4_t*)(abuf + row * KB + ((cl ^ swz(row)) * 8));
#pragma unroll
              for (int t = 0; t < NT; ++t) acc[m][t] = Mfma32<DT>::run(a, b[t], acc[m][t]);
            }
          }
        }
        load_kb(ws, min(kb + 2, kb_last));
        // activation k-block idx + 1 must have landed: the loads requested after it are the
        // weights of k-blocks idx + 2 (and, with three buffers, idx + 1 and activation k-block
        // idx + 2); then k-block idx + NBUF goes into the buffer just read
        wait_vmcnt_p<NBUF == 2 ? LPK : 2 * LPK + AV>();
        barrier_lds_p();
        dma_a(idx + NBUF, abuf_of(j % NBUF));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  static_assert(MT == 2 || MT == 4 || MT == 8, "block_m 64, 128 or 256");
  if constexpr (MT == 2) {
    if (mt_valid >= 2) kloop(std::integral_constant<int, 2>{});
    else kloop(std::integral_constant<int, 1>{});
  } else if constexpr (MT == 4) {
    if (mt_valid >= 4) kloop(std::integral_constant<int, 4>{});
    else if (mt_valid == 3) kloop(std::integral_constant<int, 3>{});
    else if (mt_valid == 2) kloop(std::integral_constant<int, 2>{});
    else kloop(std::integral_constant<int, 1>{});
  } else {
    switch (mt_valid) {
      case 8: kloop(std::integral_constant<int, 8>{}); break;
      case 7: kloop(std::integral_constant<int, 7>{}); break;
      case 6: kloop(std::integral_constant<int, 6>{}); break;
      case 5: kloop(std::integral_constant<int, 5>{}); break;
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      default: kloop(std::integral_constant<int, 1>{}); break;
    }
  }
  // direct loads still in flight must land before the workgroup's LDS is handed on
  wait_vmcnt_p<0>();

  if constexpr (MIXED) {
    // lane c (c < 16) of each 32-lane half holds gate column col + c, lane c + 16 the up column:
    // every lane fetches its partner's value, lanes c < 16 write
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= mt_valid) continue;
      float up[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) up[i] = __shfl_xor(acc[m][0][i], 16, kWave);
      if (c32 < 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = m * 32 + 8 * (i / 4) + 4 * h + (i % 4);
          const int slot = s_slot[r];
          if (slot < 0) continue;
          const float wscale = p.topk_w ? p.topk_w[slot] : 1.0f;
          const float g = acc[m][0][i];
          const float v = g / (1.0f + __expf(-g)) * up[i] * wscale;
          ((uint16_t*)p.C)[(size_t)slot * (N / 2) + col[0] + c32] = float_to_bits<DT>(v);
        }
      }
    }
    return;
  }

  // epilogue: register i of lane l holds row 8 (i / 4) + 4 h + i % 4 of each 32-row tile, column
  // l % 32 of each column tile
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= mt_valid) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = m * 32 + 8 * (i / 4) + 4 * h + (i % 4);
      const int slot = s_slot[r];
      if (slot < 0) continue;
      const float wscale = p.topk_w ? p.topk_w[slot] : 1.0f;
#pragma unroll
      for (int t = 0; t < NOUT; ++t) {
        const int cc = col[t] + c32;
        if constexpr (ACT && !MIXED) {
          const float g = acc[m][t][i];
          const float up = acc[m][t + NOUT][i];
          const float v = g / (1.0f + __expf(-g)) * up * wscale;
          ((uint16_t*)p.C)[(size_t)slot * (N / 2) + cc] = float_to_bits<DT>(v);
        } else if constexpr (OUTF32) {
          ((float*)p.C)[((size_t)z * p.num_slots + slot) * N + cc] = acc[m][t][i] * wscale;
        } else {
          ((uint16_t*)p.C)[(size_t)slot * N + cc] = float_to_bits<DT>(acc[m][t][i] * wscale);
        }
      }
    }
  }
}

// Eight wavefronts share one activation tile (half the activation loads per weight byte of four),
// two activation buffers: measured against four wavefronts and against a third buffer (two
// k-blocks of lookahead) on the DeepSeek-V3 prefill layer at 4096 tokens, all within 3 %, eight
// with two buffers fastest (uint4 first GEMM 2.83 ms, int8 layer 4.57 against 4.85 ms)
constexpr int kPrefillWaves = 8;
constexpr int kPrefillBufs = 2;

// ------------------------------------------------------------------------------------------------
// w8a8: int8 activations (one float32 scale per row) x int8 weights (one scale per output column),
// same blocking on v_mfma_i32_32x32x32_i8 (measured 4.35 POP/s on all compute units, against
// 2.7 for the 16x16x64 form).  A k-block is 64 k (64 bytes of a weight row, 64 bytes of an
// activation row); lane half h of a column tile loads bytes [32 h, 32 h + 32) of its weight row, so
// MFMA step s (32 k) takes k = 32 h + 16 s + (0..15) from lane half h: the load's bytes as they are
// (no decode) for B, and the same 16 bytes of the activation row (logical chunk 2 h + s) for A.
// Integer sums are exact; the epilogue scales by the row's and the column's scale in float32.
// ------------------------------------------------------------------------------------------------
typedef int32_t i32x16_t __attribute__((ext_vector_type(16)));
typedef int32_t i32x4v_t __attribute__((ext_vector_type(4)));

// block_m 256 (MT = 8): one column tile per wavefront (eight 32-row accumulator tiles take the
// registers, two wavefronts per SIMD), with the SiLU epilogue a mixed tile of 16 gate rows and the
// 16 matching up rows, as in the 256-row prefill GEMM
template <int DT, int MT, int NT, int WAVES, int ACT, int OUTF32>
__global__ void __launch_bounds__(WAVES * 64, MT == 8 ? 1 : 2) w8a8_mma32_kernel(W8A8Params p) {
  constexpr int THREADS = WAVES * kWave;
  constexpr int BM = 32 * MT;
  constexpr int KB = 64;                          // k (bytes) per k-block
  constexpr int STEPS = 2;                        // 32x32x32 MFMAs per k-block and tile pair
  constexpr int VPR = KB / 16;                    // 16-byte chunks of an activation row per k-block
  constexpr int NCH = BM * VPR;                   // chunks of the tile per k-block
  constexpr int AV = (NCH + THREADS - 1) / THREADS;
  static_assert(NCH % kWave == 0 && (NCH >= THREADS ? NCH % THREADS == 0 : true),
                "whole wavefronts of activation chunks");
  static_assert(!ACT || NT % 2 == 0 || NT == 1, "SiLU epilogue: paired or mixed tiles");
  static_assert(MT != 8 || NT == 1, "256-row blocks: one column tile per wavefront");
  constexpr bool MIXED = ACT && NT == 1;
  constexpr int NOUT = ACT ? (MIXED ? 1 : NT / 2) : NT;
  constexpr int WG_COLS = WAVES * NOUT * (MIXED ? 16 : 32);
  constexpr int LPK = 2 * NT;                     // weight loads per lane and k-block

  __shared__ __attribute__((aligned(16))) uint8_t s_a0[BM * KB];
  __shared__ __attribute__((aligned(16))) uint8_t s_a1[BM * KB];
  __shared__ int s_slot[BM];
  __shared__ float s_as[BM];
  // 64-byte rows: four rows share a 256-byte bank window, so rows r, r + 4, r + 8, r + 12 take
  // distinct chunk positions: a fragment read (same logical chunk, 16 rows) hits 16 bank groups
  auto swz = [](int r) -> int { return (r >> 2) & 3; };

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int N = p.N, K = p.K;
  const int n_out = ACT ? N / 2 : N;
  const int n_chunks = n_out / WG_COLS;
  const int nc = (int)blockIdx.x % n_chunks;
  const int blk = (int)blockIdx.x / n_chunks;
  if (blk * BM >= p.num_post[0]) return;
  const int e = p.expert_ids[blk];
  if ((unsigned)e >= (unsigned)p.E) return;
  if (tid < BM) {
    const int sl = p.sorted_ids[blk * BM + tid];
    const bool ok = (unsigned)sl < (unsigned)p.num_slots;
    s_slot[tid] = ok ? sl : -1;
    s_as[tid] = ok ? p.a_scales[sl / p.a_row_div] : 0.0f;
  }
  const int kb_total = K / KB;
  const int c32 = lane & 31;
  const int h = lane >> 5;
  // col[t]: first output column of tile t (of the gate half with the SiLU epilogue); wrow[t]: the
  // weight row lane l streams for tile t (mixed tile: gate rows in lanes c32 < 16, up rows above)
  int col[NT], wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if constexpr (MIXED) {
      col[t] = nc * WG_COLS + wave * 16;
      wrow[t] = c32 < 16 ? col[t] + c32 : N / 2 + col[t] + (c32 - 16);
    } else if constexpr (ACT) {
      const int g0 = nc * WG_COLS + wave * NOUT * 32;
      col[t] = t < NOUT ? g0 + t * 32 : N / 2 + g0 + (t - NOUT) * 32;
      wrow[t] = col[t] + c32;
    } else {
      col[t] = nc * WG_COLS + (wave * NT + t) * 32;
      wrow[t] = col[t] + c32;
    }
  }
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + (size_t)e * N * K), (short)0, (int)((size_t)N * K), kRsrc3);
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.A, (short)0, (int)((size_t)p.num_a_rows * K), kRsrc3);
  uint32_t vw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) vw[t] = (uint32_t)wrow[t] * (uint32_t)K + h * 32;

  // activation chunks: slot idx = tid + i * THREADS of the unpadded tile (row idx / VPR, physical
  // chunk idx % VPR holding logical chunk (idx % VPR) ^ swz(row)); a wavefront past the tile's
  // chunks loads nothing
  static_assert(NCH < THREADS || (THREADS / VPR) % 16 == 0, "one column offset for all loads");
  uint32_t arow[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int idx = tid + i * THREADS;
    const int r = idx / VPR;
    int sl = -1;
    if (idx < NCH) sl = p.sorted_ids[blk * BM + r];
    const int row = (unsigned)sl < (unsigned)p.num_slots ? sl / p.a_row_div : -1;
    arow[i] = row >= 0 ? (uint32_t)row * (uint32_t)K : 0x80000000u;
  }
  const uint32_t acol = (uint32_t)((tid % VPR) ^ swz(tid / VPR)) * 16;
  auto dma_a = [&](int kb, uint8_t* buf) {
    const uint32_t kbase = (uint32_t)(kb * KB);
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      if (NCH >= THREADS || wave * kWave < NCH) {
        const uint32_t off = (arow[i] < 0x80000000u && kb < kb_total) ? arow[i] + kbase + acol
                                                                       : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs_a,
            (__attribute__((address_space(3))) void*)(buf + (size_t)(wave * kWave + i * THREADS) * 16),
            16, off, 0, 0, 0);
      }
    }
  };
  u32x4_t wq[2][NT][2];
  auto load_kb = [&](int slot, int kb) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wq[slot][t][j] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_w, vw[t] + j * 16, kb * KB, 0));
  };

  i32x16_t acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][t][i] = 0;

  const int kb_last = kb_total - 1;
  dma_a(0, s_a0);
  load_kb(0, 0);
  load_kb(1, min(1, kb_last));
  wait_vmcnt_p<2 * LPK>();
  barrier_lds_p();
  int n_valid = 0;
#pragma unroll
  for (int q = 0; q < BM / kWave; ++q)
    n_valid += __builtin_popcountll(__ballot(s_slot[q * kWave + lane] >= 0));
  const int mt_valid = __builtin_amdgcn_readfirstlane((n_valid + 31) / 32);
  dma_a(1, s_a1);

  const int n_iter = (kb_total + 1) / 2;
  auto kloop = [&](auto ma_c) {
    constexpr int MA = decltype(ma_c)::value;
    for (int it = 0; it < n_iter; ++it) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int kb = it * 2 + j;
        const uint8_t* abuf = j ? s_a1 : s_a0;
        if (kb < kb_total) {
#pragma unroll
          for (int st = 0; st < STEPS; ++st) {
            const int cl = 2 * h + st;
#pragma unroll
            for (int m = 0; m < MA; ++m) {
              const int row = m * 32 + c32;
              const u32x4_t a = *(const u32x4_t*)(abuf + row * KB + ((cl ^ swz(row)) * 16));
#pragma unroll
              for (int t = 0; t < NT; ++t)
                acc[m][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                    __builtin_bit_cast(i32x4v_t, a), __builtin_bit_cast(i32x4v_t, wq[j][t][st]),
                    acc[m][t], 0, 0, 0);
            }
          }
        }
        load_kb(j, min(kb + 2, kb_last));
        wait_vmcnt_p<LPK>();
        barrier_lds_p();
        dma_a(kb + 2, j ? s_a1 : s_a0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  static_assert(MT == 2 || MT == 4 || MT == 8, "block_m 64, 128 or 256");
  if constexpr (MT == 2) {
    if (mt_valid >= 2) kloop(std::integral_constant<int, 2>{});
    else kloop(std::integral_constant<int, 1>{});
  } else if constexpr (MT == 4) {
    if (mt_valid >= 4) kloop(std::integral_constant<int, 4>{});
    else if (mt_valid == 3) kloop(std::integral_constant<int, 3>{});
    else if (mt_valid == 2) kloop(std::integral_constant<int, 2>{});
    else kloop(std::integral_constant<int, 1>{});
  } else {
    switch (mt_valid) {
      case 8: kloop(std::integral_constant<int, 8>{}); break;
      case 7: kloop(std::integral_constant<int, 7>{}); break;
      case 6: kloop(std::integral_constant<int, 6>{}); break;
      case 5: kloop(std::integral_constant<int, 5>{}); break;
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      default: kloop(std::integral_constant<int, 1>{}); break;
    }
  }
  wait_vmcnt_p<0>();

  // epilogue: register i of lane l holds row 8 (i / 4) + 4 h + i % 4 of each 32-row tile
  const uint16_t* wsc = (const uint16_t*)p.w_scales + (size_t)e * N;
  if constexpr (MIXED) {
    // each lane scales its own row's sums (its weight row's scale), then lane c (c < 16) of each
    // 32-lane half takes the up value of lane c + 16 and writes SiLU(gate) * up
    const float ws = bits_to_float<DT>(wsc[wrow[0]]);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= mt_valid) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m * 32 + 8 * (i / 4) + 4 * h + (i % 4);
        const float v = (float)acc[m][0][i] * s_as[r] * ws;
        const float u = __shfl_xor(v, 16, kWave);
        const int slot = s_slot[r];
        if (c32 < 16 && slot >= 0) {
          const float wscale = p.topk_w ? p.topk_w[slot] : 1.0f;
          ((uint16_t*)p.C)[(size_t)slot * (N / 2) + col[0] + c32] =
              float_to_bits<DT>(v / (1.0f + __expf(-v)) * u * wscale);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m >= mt_valid) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = m * 32 + 8 * (i / 4) + 4 * h + (i % 4);
      const int slot = s_slot[r];
      if (slot < 0) continue;
      const float sa = s_as[r];
      const float wscale = p.topk_w ? p.topk_w[slot] : 1.0f;
#pragma unroll
      for (int t = 0; t < NOUT; ++t) {
        const int cc = col[t] + c32;
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

template <int DT, int MT, int NT>
hipError_t launch_w8a8_32(const W8A8Params& p, int act, int out_f32, hipStream_t stream) {
  constexpr int WV = kPrefillWaves;
  const int n_out = act ? p.N / 2 : p.N;
  const int wg_cols = act ? (NT == 1 ? WV * 16 : WV * (NT / 2) * 32) : WV * NT * 32;
  const long long grid = (long long)(n_out / wg_cols) * p.num_blocks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 block(WV * kWave);
  if (act) {
    if constexpr (NT % 2 == 0 || MT == 8)
      hipLaunchKernelGGL((w8a8_mma32_kernel<DT, MT, NT, WV, 1, 0>), dim3((unsigned)grid), block, 0,
                         stream, p);
    else
      return hipErrorInvalidValue;
  } else if (out_f32) {
    hipLaunchKernelGGL((w8a8_mma32_kernel<DT, MT, NT, WV, 0, 1>), dim3((unsigned)grid), block, 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((w8a8_mma32_kernel<DT, MT, NT, WV, 0, 0>), dim3((unsigned)grid), block, 0,
                       stream, p);
  }
  return hipGetLastError();
}

template <int DT, int MT>
hipError_t launch_w8a8_32_nt(const W8A8Params& p, int act, int out_f32, hipStream_t stream) {
  if constexpr (MT == 8) {
    return launch_w8a8_32<DT, MT, 1>(p, act, out_f32, stream);
  } else {
    if (act || p.N % (kPrefillWaves * 64) == 0) return launch_w8a8_32<DT, MT, 2>(p, act, out_f32, stream);
    return launch_w8a8_32<DT, MT, 1>(p, act, out_f32, stream);
  }
}


template <int DT, int BITS, int MT, int NT, int WAVES, int NBUF>
hipError_t launch_nt(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
  const int n_out = c.act ? p.N / 2 : p.N;
  const int n_chunks = n_out / prefill_wg_cols(c, p.N);
  const long long grid = (long long)n_chunks * p.num_blocks * p.split_k;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 block(WAVES * kWave);
  if (c.act) {
    hipLaunchKernelGGL((prefill_gemm_kernel<DT, BITS, MT, NT, WAVES, NBUF, 1, 0>),
                       dim3((unsigned)grid), block, 0, stream, p);
  } else if (c.out_f32) {
    hipLaunchKernelGGL((prefill_gemm_kernel<DT, BITS, MT, NT, WAVES, NBUF, 0, 1>),
                       dim3((unsigned)grid), block, 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_gemm_kernel<DT, BITS, MT, NT, WAVES, NBUF, 0, 0>),
                       dim3((unsigned)grid), block, 0, stream, p);
  }
  return hipGetLastError();
}

template <int DT, int BITS, int MT>
hipError_t launch_mt_p(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
  if constexpr (MT == 8) {
    return launch_nt<DT, BITS, MT, 1, kPrefillWaves, kPrefillBufs>(p, c, stream);
  } else {
    if (prefill_nt(c, p.N) == 2)
      return launch_nt<DT, BITS, MT, 2, kPrefillWaves, kPrefillBufs>(p, c, stream);
    return launch_nt<DT, BITS, MT, 1, kPrefillWaves, kPrefillBufs>(p, c, stream);
  }
}

template <int DT, int BITS>
hipError_t launch_bits_p(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
  if (c.block_m == 256) return launch_mt_p<DT, BITS, 8>(p, c, stream);
  return launch_mt_p<DT, BITS, 4>(p, c, stream);
}

}  // namespace

// Column tiles of 32 per wavefront.  block_m 128: 2 (gate and up with the SiLU epilogue, or 64
// weight rows), or 1 where N holds no whole number of workgroups of 2.  block_m 256: 1 (eight
// 32-row accumulator tiles per column tile take the registers two tiles would need; with the SiLU
// epilogue the tile is mixed: 16 gate rows and the 16 matching up rows).
int prefill_nt(const GemmConfig& c, int N) {
  if (c.block_m == 256) return 1;
  if (c.act) return 2;
  return N % (kPrefillWaves * 64) == 0 ? 2 : 1;
}

int prefill_wg_cols(const GemmConfig& c, int N) {
  if (c.act) return kPrefillWaves * (c.block_m == 256 ? 16 : 32);
  return kPrefillWaves * 32 * prefill_nt(c, N);
}

// block_m 128 and 256 only: at 64 rows (about 32 slots per expert in the DeepSeek-V3 layer at 1024
// tokens, often a single 32-row tile) the exact decode is repeated for too few rows and the 16-row
// kernel with biased codes is faster (measured: first GEMM 1.57 against 1.40 ms)
bool prefill_fits(const GemmConfig& c, int N) {
  if (c.block_m != 128 && c.block_m != 256) return false;
  if (c.act) return (N / 2) % prefill_wg_cols(c, N) == 0;
  return N % prefill_wg_cols(c, N) == 0;
}

size_t prefill_lds_bytes(const GemmConfig& c) {
  const int kb = c.bits == 4 ? 128 : 64;
  return sizeof(uint16_t) * kPrefillBufs * (size_t)c.block_m * kb + sizeof(int) * (size_t)c.block_m;
}

bool w8a8_mma32_fits(int block_m, int act, int N) {
  if (block_m != 64 && block_m != 128 && block_m != 256) return false;
  if (act) return (N / 2) % (kPrefillWaves * (block_m == 256 ? 16 : 32)) == 0;
  return N % (kPrefillWaves * 32) == 0;
}

hipError_t launch_w8a8_mma32(const W8A8Params& p, int block_m, int act, int dtype, int out_f32,
                             hipStream_t stream) {
  if (!w8a8_mma32_fits(block_m, act, p.N)) return hipErrorInvalidValue;
  if (dtype == 0)
    return block_m == 64    ? launch_w8a8_32_nt<0, 2>(p, act, out_f32, stream)
           : block_m == 128 ? launch_w8a8_32_nt<0, 4>(p, act, out_f32, stream)
                            : launch_w8a8_32_nt<0, 8>(p, act, out_f32, stream);
  return block_m == 64    ? launch_w8a8_32_nt<1, 2>(p, act, out_f32, stream)
         : block_m == 128 ? launch_w8a8_32_nt<1, 4>(p, act, out_f32, stream)
                          : launch_w8a8_32_nt<1, 8>(p, act, out_f32, stream);
}

hipError_t launch_prefill(const GemmParams& p_in, const GemmConfig& c, hipStream_t stream) {
  GemmParams p = p_in;
  const int kb_total = p.K / (c.bits == 4 ? 128 : 64);
  if (p.split_k < 1 || p.split_k > kb_total || (p.split_k > 1 && !c.out_f32) ||
      !prefill_fits(c, p.N))
    return hipErrorInvalidValue;
  if (c.dtype == 0)
    return c.bits == 4 ? launch_bits_p<0, 4>(p, c, stream) : launch_bits_p<0, 8>(p, c, stream);
  return c.bits == 4 ? launch_bits_p<1, 4>(p, c, stream) : launch_bits_p<1, 8>(p, c, stream);
}

}  // namespace moe
