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
// fp16 uint4: a nibble in bits 0..3 of a 16-bit half under the exponent of 1024 reads as 1024 + q,
// and one in bits 4..7 reads as 1024 + 16 q; both are exact.  So the pairs (k0,k4) and (k2,k6) are
// masked out of w and w >> 8 in place, and the pairs (k1,k5) and (k3,k7) in place with the high
// nibble mask, scaled by 16.  The activations at those k offsets are stored in LDS divided by 16,
// so every product a * w is unchanged: one shift and four and-or per 8 weights instead of three
// shifts.  bf16 has too few mantissa bits for 1024 + 16 q under any exponent, so its biased codes
// keep the three shifts, and its exact decode converts each nibble from a byte of its own in
// natural k order (no activation permutation then).
//
// What the matrix cores see.  block_m 16 and 32: q - z exactly (magic-biased codes whose bias and
// zero point are removed by a second MFMA or by an exact half-precision subtraction), the group
// scale applied in float32 to each k-block's partial sum.  block_m 64 and 128: the correctly
// rounded dtype value of (q - z) * s (fp16: the exact difference of the half-precision integers
// 1024+q and 1024+z, then one rounded multiply; bf16: an exact float32 fma of q against s and
// -z*s, then one rounding).  Two limits of the fp16 uint4 paths, both from the factor 16:
//   - an activation divided by 16 is exact for |a| >= 2^-10; below that a / 16 is subnormal and
//     loses up to 4 low bits (a relative error up to 2^-7 on such tiny activations);
//   - the block_m >= 64 decode forms 16 (q - z) s in fp16, which overflows to inf for a group
//     scale above 65504 / 240 (about 273, decoded weights beyond about 4000 in magnitude).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family buffer descriptor: 32-bit data format

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
  uint32_t zn2h; // fp16 uint4: -(1024 + 16 z) in both halves (the high-nibble pairs)
  float sf;      // bf16: scale as float
  float cf;      // bf16: -(magic + z) * scale (exact)
};

template <int DT, int BITS>
__device__ __forceinline__ DecodeK make_decode(uint32_t sbits, uint32_t z) {
  DecodeK d;
  if constexpr (DT == 0) {
    d.s2 = (sbits & 0xFFFFu) * 0x10001u;
    if constexpr (BITS == 4) {
      d.zn2 = (0xE400u | z) * 0x10001u;  // fp16 -(1024 + z): sign, exponent of 1024, mantissa z
      d.zn2h = (0xE400u | (z << 4)) * 0x10001u;
    } else {
      const uint32_t zb = __builtin_bit_cast(uint16_t, (_Float16)(-1152.0f));
      d.zn2 = zb | (zb << 16);
      d.zn2h = d.zn2;
    }
    d.sf = 0.0f;
    d.cf = 0.0f;
  } else {
    d.sf = __uint_as_float(sbits << 16);
    d.cf = (BITS == 4) ? -(float)z * d.sf : -128.0f * d.sf;  // exact: 4- or 8-bit times 8-bit
    d.s2 = 0;
    d.zn2 = 0;
    d.zn2h = 0;
  }
  return d;
}

__device__ __forceinline__ uint32_t h2_add(uint32_t x, uint32_t y) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, x) + __builtin_bit_cast(half2_t, y));
}

__device__ __forceinline__ uint32_t h2_sub_mul(uint32_t t, uint32_t zn2, uint32_t s2) {
  const half2_t r = (__builtin_bit_cast(half2_t, t) + __builtin_bit_cast(half2_t, zn2)) *
                    __builtin_bit_cast(half2_t, s2);
  return __builtin_bit_cast(uint32_t, r);
}

// (a & m) | c in one gfx950 v_bitop3_b32 (truth table 0xEA: S0 & S1 | S2).  Left to itself the
// compiler splits this into an and plus an or, because VOP3 encodings take no literal operands.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}

// uint4: 8 nibbles of one dword (nibble i = k offset i) -> B operand.  fp16: pairs (0,4)(1,5)(2,6)
// (3,7), the (1,5) and (3,7) pairs as 16 times the weight (their activations are / 16); bf16:
// natural order.
template <int DT>
__device__ __forceinline__ u32x4_t decode_u4(uint32_t w, const DecodeK& d, uint32_t mlo,
                                             uint32_t mhi, uint32_t magic) {
  u32x4_t b;
  if constexpr (DT == 0) {
    const uint32_t w8 = w >> 8;
    b[0] = h2_sub_mul(and_or(w, mlo, magic), d.zn2, d.s2);
    b[1] = h2_sub_mul(and_or(w, mhi, magic), d.zn2h, d.s2);
    b[2] = h2_sub_mul(and_or(w8, mlo, magic), d.zn2, d.s2);
    b[3] = h2_sub_mul(and_or(w8, mhi, magic), d.zn2h, d.s2);
  } else {
    // bf16, natural k order (k0,k1)(k2,k3)(k4,k5)(k6,k7): every nibble in a byte of its own, one
    // byte-to-float conversion each (v_cvt_f32_ubyte0..3), then (q - z) * s exactly in one float32
    // fma (4-bit times 8-bit operands) and one rounding to bf16.  The masks go through
    // v_bitop3_b32: a plain `&` lets the compiler fold mask and byte select into a 4-bit field
    // extract per nibble (v_bfe_u32 + v_cvt_f32_ubyte0, two instructions instead of one).
    const uint32_t even = __builtin_amdgcn_bitop3_b32(w, 0x0F0F0F0Fu, 0u, 0xC0);       // w & m
    const uint32_t odd = __builtin_amdgcn_bitop3_b32(w >> 4, 0x0F0F0F0Fu, 0u, 0xC0);  // (w >> 4) & m
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q0 = (float)((even >> (8 * i)) & 0xFFu);
      const float q1 = (float)((odd >> (8 * i)) & 0xFFu);
      b[i] = f32x2_to_bf16x2(__builtin_fmaf(q0, d.sf, d.cf), __builtin_fmaf(q1, d.sf, d.cf));
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

// Biased decode for the decode-regime kernels: the MFMA sees magic + q exactly (fp16 1024 + q and
// 1024 + 16 q as in decode_u4, or bf16 128 + q), pairs (k0,k4)(k1,k5)(k2,k6)(k3,k7).  The bias and
// the zero point are removed by a second MFMA against -(magic + z) (fp16: -(1024 + 16 z) on the
// high-nibble pairs) and the group scale is applied to the float32 partial sum of the k-block, so
// per 8 weights the VALU does 1 shift and 4 and-or (bf16: 3 shifts and 4 and-or).
template <int DT>
__device__ __forceinline__ u32x4_t bias_u4(uint32_t w, uint32_t mlo, uint32_t mhi, uint32_t magic) {
  if constexpr (DT == 0) {
    const uint32_t w8 = w >> 8;
    return u32x4_t{and_or(w, mlo, magic), and_or(w, mhi, magic), and_or(w8, mlo, magic),
                   and_or(w8, mhi, magic)};
  } else {
    return u32x4_t{and_or(w, mlo, magic), and_or(w >> 4, mlo, magic), and_or(w >> 8, mlo, magic),
                   and_or(w >> 12, mlo, magic)};
  }
}

// int8 biased decode: u = q + 128 in natural k order; fp16 as 1024 + u, bf16 as u itself (exact).
template <int DT>
__device__ __forceinline__ u32x4_t bias_s8(uint32_t lo, uint32_t hi) {
  const uint32_t ulo = lo ^ 0x80808080u;
  const uint32_t uhi = hi ^ 0x80808080u;
  if constexpr (DT == 0) {
    const uint32_t C = 0x64646464u;
    return u32x4_t{__builtin_amdgcn_perm(C, ulo, 0x04010400u), __builtin_amdgcn_perm(C, ulo, 0x04030402u),
                   __builtin_amdgcn_perm(C, uhi, 0x04010400u), __builtin_amdgcn_perm(C, uhi, 0x04030402u)};
  } else {
    return u32x4_t{f32x2_to_bf16x2((float)(ulo & 0xFFu), (float)((ulo >> 8) & 0xFFu)),
                   f32x2_to_bf16x2((float)((ulo >> 16) & 0xFFu), (float)(ulo >> 24)),
                   f32x2_to_bf16x2((float)(uhi & 0xFFu), (float)((uhi >> 8) & 0xFFu)),
                   f32x2_to_bf16x2((float)((uhi >> 16) & 0xFFu), (float)(uhi >> 24))};
  }
}

// Wait until at most N vector-memory loads of this wave are outstanding (loads complete in issue
// order); the other counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS-only workgroup barrier: waits for this wave's LDS traffic, not for its global loads, so the
// weight prefetch stays in flight across it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

template <int BITS, int MT, int NTW, int THREADS = kThreads>
struct Shape {
  static constexpr int BM = 16 * MT;
  static constexpr int KB = BITS == 4 ? 128 : 64;            // k per k-block
  // activation chunk: four 16-byte vectors per thread, at least one k-block; two for BLOCK_M 16
  // and 32 (256 and 128 columns: a short K, as in a tensor-parallel share with I = 256, is then a
  // whole number of unrolled iterations instead of half of one spent on virtual k-blocks, and the
  // smaller tile and staging registers leave room for four workgroups per compute unit)
  static constexpr int KC0 = (MT <= 2 ? 2 : 4) * 8 * kThreads / BM;
  static constexpr int KC = KC0 < KB ? KB : KC0;
  static constexpr int AV = BM * KC / 8 / THREADS;           // 16-byte vectors per thread
  static_assert(AV >= 1 && BM * KC / 8 % THREADS == 0, "whole activation vectors per thread");
  static constexpr int LDA = KC + 8;                          // LDS row stride (16-byte pad)
  static constexpr int KBC = KC / KB;                         // k-blocks per chunk
  // weight k-blocks in flight per wavefront.  The decode kernels keep 2, not 4: fewer registers
  // per wavefront and more wavefronts per SIMD stream faster than a deeper prefetch (measured on
  // the Mixtral-shaped w13 at M = 64, BM 32: 217 -> 140 registers, two wavefronts per SIMD ->
  // three, 141 -> 127 us)
  static constexpr int PF = MT <= 2 ? 2 : (NTW == 2 ? 2 : 1);
  // activation chunks in flight in registers: a chunk's loads must be issued at least PF k-blocks
  // before it is stored to LDS, or the wait for it (memory counters complete in issue order) also
  // waits for the newest weight prefetches and shortens the weight pipeline at every chunk edge
  static constexpr int AQ0 = (PF + KBC - 1) / KBC;
  static constexpr int AQ = (MT >= 8 && AQ0 > 1) ? 1 : AQ0;   // BM 128: registers are the limit
  static constexpr int UA = KBC * AQ;
  static constexpr int U0 = UA / gcd_c(UA, PF) * PF;          // lcm(KBC * AQ, PF)
  // unroll; BM >= 64 also a multiple of 2 * KBC (each activation buffer once per iteration)
  static constexpr int U = MT >= 4 ? U0 / gcd_c(U0, 2 * KBC) * (2 * KBC) : U0;
};

template <int DT, int BITS, int MT, int NTW, int ACT, int OUTF32, int WAVES, int MULTI = 0>
__global__ void __launch_bounds__(WAVES * kWave) wna16_gemm_kernel(GemmParams p) {
  constexpr int THREADS = WAVES * kWave;
  using S = Shape<BITS, MT, NTW, THREADS>;
  constexpr int BM = S::BM;
  constexpr int KC = S::KC;
  constexpr int PF = S::PF;
  constexpr int KB = S::KB;
  constexpr int AV = S::AV;
  constexpr int KBC = S::KBC;
  constexpr int U = S::U;
  constexpr int AQ = S::AQ;
  constexpr int STEPS = KB / 32;                    // MFMAs per k-block
  constexpr int NOUT = ACT ? NTW / 2 : NTW;         // output tiles per wave
  constexpr int WG_COLS = WAVES * NOUT * 16;
  constexpr int VPR = KC / 8;                       // 16-byte vectors per activation row chunk
  constexpr int R = WAVES * NTW * 16;               // weight rows of the workgroup
  // metadata row pitch in dwords: consecutive staging threads write entries 2 * RP apart, and
  // RP = 2 (mod 32) spreads them over the LDS banks
  constexpr int RP = R + 2;
  // BM >= 64 (one k-block per activation chunk, a workgroup barrier after every k-block): the
  // uint4 metadata goes through a two-slot LDS ring refilled at each barrier from loads issued two
  // k-blocks ahead, instead of the whole K range staged up front.  Its 1 KiB instead of up to
  // 29 KiB (K = 7168) lets 64-row workgroups share a compute unit four at a time.
  constexpr bool RING = BITS == 4 && MT >= 4;
  static_assert(!RING || (S::KBC == 1 && S::U % 2 == 0), "ring: one k-block per chunk, even unroll");
  // decode regime: biased codes with MFMA-side bias removal (fewer VALU ops per weight); prefill:
  // exact decoded weights, no extra MFMAs (the matrix cores are the bottleneck there)
  constexpr bool BIASED = MT <= 2;
  // MULTI: the workgroup streams p.cgroup column chunks in turn against one activation tile (the
  // whole K range of a short K, staged once), writing each chunk's float32 partials as it ends:
  // the start-up of a workgroup (slot ids, activation rows, metadata, the first weight latency) is
  // paid once per cgroup chunks instead of once per chunk
  static_assert(!MULTI || (BIASED && BITS == 4 && MT == 1 && !ACT && OUTF32),
                "column groups: uint4, 16-row blocks, float32 partials");
  // the activation k order in LDS follows the weight decode: permuted for the shift-and-mask
  // decodes (fp16, and bf16 biased codes), natural for the bf16 exact decode and for int8
  constexpr bool PERM_A = BITS == 4 && (DT == 0 || BIASED);
  // BM >= 64 with natural k order: activation chunks go from memory straight into LDS (buffer loads
  // with an LDS destination), an unpadded tile whose row-major order is the threads' load order;
  // no registers or instructions spent staging them
  constexpr bool DIRECT = !PERM_A && MT >= 4;
  constexpr int LDA = DIRECT ? KC : S::LDA;
  // The unpadded tile is swizzled instead: 16-byte chunk j of row r sits at chunk j ^ swz(r), so
  // the 16 rows of a fragment read (same logical chunk) fall on 16 different bank groups
  // (64 banks; 16 or 8 chunks per row).  swz(row) depends only on row % 16 = rsub.
  static_assert(!DIRECT || KC / 8 == 16 || KC / 8 == 8, "swizzle covers 8 or 16 chunks per row");
  auto swz = [](int r) -> int { return KC / 8 == 16 ? (r & 15) : ((r >> 1) & 7); };
  // uint4 scales and zero points of the workgroup's rows, in dynamic LDS as
  // meta[slot][row] = scale | zero << 16.  BM <= 32: the whole K range, staged once before the
  // weight stream starts (slot = kb - kb_beg; the host sizes it (rows + 2) * k-blocks * 4 bytes);
  // consecutive threads read consecutive pairs of k-blocks of one row, so each cache line of scales
  // is touched once.  Per-lane loads of a 2-byte scale and a 1-byte zero point every k-block would
  // triple the memory instructions of the weight stream and cap it near 3.2 TB/s.  BM >= 64: a
  // two-slot ring (slot = k-block & 1), one load pair per row and k-block spread over the threads.
  extern __shared__ uint32_t s_meta[];

  // The two activation buffers are separate LDS variables: with one array the compiler cannot
  // tell that an LDS-destination load into one buffer leaves the other alone, and waits for every
  // outstanding load (weight prefetch included) before reading fragments after it.
  __shared__ __attribute__((aligned(16))) uint16_t s_a0[BM * LDA];
  __shared__ __attribute__((aligned(16))) uint16_t s_a1[BM * LDA];
  auto abuf = [&](int b) -> uint16_t* { return b ? s_a1 : s_a0; };
  // DIRECT: in the unrolled loop the buffer of every chunk is a compile-time constant (an even
  // number of chunks per unrolled iteration), so each access names its variable
  static_assert(!DIRECT || (U / KBC) % 2 == 0, "even number of chunks per unrolled iteration");
  __shared__ int s_slot[BM];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wavefront-uniform (a scalar: the LDS destination of a direct load is a scalar register, and a
  // per-lane value there costs a loop that makes it uniform)
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int N = p.N;
  const int K = p.K;
  const int n_out = ACT ? N / 2 : N;
  const int n_chunks = n_out / WG_COLS;
  const int split = p.split_k;
  const int G = MULTI ? p.cgroup : 1;  // column chunks of this workgroup
  const int n_groups = n_chunks / G;

  int bid = blockIdx.x;
  const int z = bid % split;
  bid /= split;
  const int nc = (bid % n_groups) * G;  // first column chunk
  const int blk = bid / n_groups;
  // Row maps.  Aligned: slots listed by sorted_ids, expert per block from expert_ids.  Dense: rows
  // are slots 0..num_slots-1 in order, one expert.  Batched: block blk covers rows j*BM.. of expert
  // blk / bpe (j = blk % bpe), slot = row index e * max_tokens + j*BM + r, valid below the expert's
  // count (clamped to max_tokens).
  int e, n_valid = 0, brow0 = 0;
  if (p.batched) {
    e = blk / p.bpe;
    const int j = blk - e * p.bpe;
    n_valid = min(p.expert_counts[e], p.max_tokens) - j * BM;
    if (n_valid <= 0) return;
    brow0 = e * p.max_tokens + j * BM;
  } else {
    if (blk * BM >= (p.dense ? p.num_slots : p.num_post[0])) return;
    e = p.dense ? 0 : p.expert_ids[blk];
  }
  if ((unsigned)e >= (unsigned)p.E) return;
  auto slot_at = [&](int i) -> int {
    if (p.batched) {
      const int r = i - blk * BM;
      return r < n_valid ? brow0 + r : -1;
    }
    return p.dense ? (i < p.num_slots ? i : -1) : p.sorted_ids[i];
  };

  // slot of each block row, for the epilogue (published by the prologue's barrier)
  if (tid < BM) {
    const int s = slot_at(blk * BM + tid);
    s_slot[tid] = (unsigned)s < (unsigned)p.num_slots ? s : -1;
  }

  // K range of this split, in k-blocks (a split past the end has an empty range and writes zeros)
  const int kb_total = K / KB;
  const int kb_per = (kb_total + split - 1) / split;
  const int kb_beg = z * kb_per;
  const int kb_end = min(kb_total, kb_beg + kb_per);
  const int kb_last = min(max(kb_beg, kb_end - 1), kb_total - 1);  // always a real k-block
  // staged metadata row pitch (dwords): R + 2, or G * R + 2 for column groups
  const int RPM = MULTI ? G * R + 2 : RP;

  // rows of the workgroup: local row lr = (wave * NTW + t) * 16 + r
  auto col_of = [&](int w, int t) -> int {
    if constexpr (ACT) {
      const int g0 = nc * WG_COLS + w * NOUT * 16;
      return t < NOUT ? g0 + t * 16 : N / 2 + g0 + (t - NOUT) * 16;
    } else {
      return nc * WG_COLS + w * NTW * 16 + t * 16;
    }
  };
  const int rsub = lane & 15;
  const int grp = lane >> 4;  // 16-byte slice of the 64-byte k-block
  int col[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) col[t] = col_of(wave, t);

  // Every global load goes through a buffer descriptor: the expert's base address sits in scalar
  // registers, per-lane offsets are fixed for the whole K loop and the k-block offset is a scalar,
  // so no load needs vector address arithmetic and none is conditional (the compiler can then keep
  // the prefetch in flight with exact vmcnt waits).
  const uint32_t row_bytes = BITS == 4 ? (uint32_t)K / 2 : (uint32_t)K;
  const uint32_t srow_bytes = BITS == 4 ? (uint32_t)(K / 128) * 2 : 2u;
  const uint32_t zrow_bytes = (uint32_t)(K / 256);
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + (size_t)e * N * row_bytes), (short)0, (int)(N * row_bytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)p.scales + (size_t)e * N * srow_bytes), (short)0, (int)(N * srow_bytes),
      kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_z = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(BITS == 4 ? p.zeros + (size_t)e * N * zrow_bytes : p.zeros), (short)0,
      BITS == 4 ? (int)(N * zrow_bytes) : 0, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.A, (short)0, (int)((size_t)p.num_a_rows * K * 2), kRsrcWord3);
  uint32_t vw[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) vw[t] = (uint32_t)(col[t] + rsub) * row_bytes + grp * 16;

  // ---- activation chunk c (KC columns of the block's BM rows): registers, then LDS.  Padding rows
  // and columns past this split's K range read past the end of the buffer, which loads zeros.
  uint32_t arow[AV], acol[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int idx = tid + i * THREADS;
    const int r = idx / VPR;
    // each thread reads the slot ids it needs itself: the activation loads then leave without
    // waiting for a workgroup barrier, under the same memory latency as weights and scales
    const int sl = slot_at(blk * BM + r);
    const int row = (unsigned)sl < (unsigned)p.num_slots ? (p.a_row_div == 1 ? sl : sl / p.a_row_div) : -1;
    arow[i] = row >= 0 ? (uint32_t)row * K * 2 : 0x80000000u;
    // DIRECT: this thread's LDS slot (r, idx % VPR) holds logical chunk (idx % VPR) ^ swz(r)
    acol[i] = (uint32_t)(DIRECT ? ((idx - r * VPR) ^ swz(r)) : (idx - r * VPR)) * 8;
  }
  const uint32_t klim = (uint32_t)(kb_end * KB);
  // chunk c travels in areg[c % AQ] (the index is a compile-time constant at every use)
  u32x4_t areg[DIRECT ? 1 : AQ][DIRECT ? 1 : AV];
  // DIRECT: chunk c into LDS buffer buf; lane l of wave w writes the 16 bytes of thread
  // w * 64 + l + i * THREADS, which in an unpadded tile is that thread's (row, 8-column group)
  auto dma_a = [&](int c, int buf) {
    const uint32_t kbase = (uint32_t)((kb_beg + c * KBC) * KB);
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const uint32_t k = kbase + acol[i];
      const uint32_t off = (arow[i] < 0x80000000u && k < klim) ? arow[i] + k * 2 : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_a,
          (__attribute__((address_space(3))) void*)((uint8_t*)abuf(buf) +
                                                    (size_t)(wave * kWave + i * THREADS) * 16),
          16, off, 0, 0, 0);
    }
  };
  auto load_a = [&](int q, int c) {
    const uint32_t kbase = (uint32_t)((kb_beg + c * KBC) * KB);
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const uint32_t k = kbase + acol[i];
      const uint32_t off = (arow[i] < 0x80000000u && k < klim) ? arow[i] + k * 2 : 0x80000000u;
      areg[q][i] =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_a, off, 0, 0));
    }
  };
  auto store_a = [&](int q, int buf) {
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int idx = tid + i * THREADS;
      const int r = idx / VPR;
      const int c8 = idx - r * VPR;
      u32x4_t v = areg[q][i];
      if constexpr (PERM_A) {
        // (x0..x7) -> (x0,x4,x1,x5,x2,x6,x3,x7), the decode's k pairing
        v = u32x4_t{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u),
                    __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
                    __builtin_amdgcn_perm(v[3], v[1], 0x05040100u),
                    __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
        if constexpr (DT == 0) {
          // the (x1,x5) and (x3,x7) words meet weights decoded as 16 times their value.  The
          // words are copied to scalars first: this compiler's __builtin_bit_cast of a vector
          // element (bit_cast(half2_t, v[1])) reads element 0 whatever the index.
          const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
          const uint32_t w1 = v[1], w3 = v[3];
          v[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, w1) * sixteenth);
          v[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, w3) * sixteenth);
        }
      }
      *(u32x4_t*)&abuf(buf)[r * LDA + c8 * 8] = v;
    }
  };

  // ---- weight stream: PF k-blocks in flight, 16 bytes per lane per tile
  u32x4_t wq[PF][NTW];
  auto load_kb = [&](int slot, int kb) {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      wq[slot][t] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_w, vw[t], kb * 64, 0));
  };

  floatx4_t acc[MT][NTW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[m][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // biased-decode constants (registers: gfx950 VOP3 encodings take no literals)
  const floatx4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t kMask = p.dec_mask;      // 0x000F000F
  const uint32_t kMaskHi = p.dec_mask_hi; // 0x00F000F0 (fp16 uint4) or 0x000F000F
  const uint32_t kMagic = p.dec_magic;  // fp16 1024 (0x6400) or bf16 128 (0x4300) in both halves
  // fp16 -(1024 + z) = 0xE400 | z; bf16 -(128 + z) = 0xC300 | z
  constexpr uint32_t kZeroBase = DT == 0 ? 0xE400u : 0xC300u;
  const uint32_t one2 = DT == 0 ? 0x3C003C00u : 0x3F803F80u;
  const u32x4_t ones = {one2, one2, one2, one2};
  floatx4_t rsum[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) rsum[m] = zero4;
  DecodeK dk8[NTW];
  if constexpr (BITS == 8 && !BIASED) {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      dk8[t] = make_decode<DT, 8>(
          __builtin_amdgcn_raw_buffer_load_b16(rs_s, (uint32_t)(col[t] + rsub) * 2, 0, 0), 0);
  }

  // ---- metadata of one k-block, read from LDS one k-block ahead of its use.  Activation
  // fragments are read where they are used (step s, row tile m: 16 bytes of row m * 16 + rsub at
  // k offset grp * (KB / 4) + s * 8 of the k-block): holding a k-block of them ahead would take
  // 4 * MT * 4 registers, and a wavefront per SIMD more hides their latency better (measured).
  uint32_t mf[NTW];
  // jc = k-block within its chunk, b = buffer of the chunk
  auto frag_base = [&](int jc, int b) -> const uint16_t* {
    return abuf(b) + rsub * LDA + jc * KB + grp * (KB / 4);
  };
  auto load_meta = [&](int idx) {
    if constexpr (BITS == 4) {
      const int mrow = RING ? (idx & 1) : min(kb_beg + idx, kb_last) - kb_beg;
#pragma unroll
      for (int t = 0; t < NTW; ++t) mf[t] = s_meta[mrow * RPM + (wave * NTW + t) * 16 + rsub];
    }
  };
  // RING: thread tid serves workgroup row tid % R for one k-block, in register set X % 2 for
  // k-block X (relative to kb_beg; past the range, the last real k-block).  The first R / 64
  // wavefronts fetch the rows' 2-byte scales, the others the 2-byte words holding their zero
  // points (even-aligned; a zero-point block of N rows is N * K / 256 bytes, even as N is), and
  // each writes its 16-bit half of the LDS entry: one memory instruction per wavefront and k-block
  // (the address unit, not the bytes, is what these loads cost), the same instruction in both
  // roles, so no branch.
  static_assert(!RING || 2 * R == THREADS, "ring: two wavefront roles over the workgroup's rows");
  const uint32_t m_lr = (uint32_t)(tid % R);
  const uint32_t m_n = (uint32_t)(col_of(m_lr / (NTW * 16), (m_lr / 16) % NTW) + (m_lr % 16));
  const int m_zero = wave >= R / kWave ? 1 : 0;
  const __amdgpu_buffer_rsrc_t rs_m = m_zero ? rs_z : rs_s;
  uint32_t m_v[2];
  auto ring_load = [&](int set, int X) {
    const int kb = min(kb_beg + X, kb_last);
    const uint32_t off = m_zero ? ((m_n * zrow_bytes + (kb >> 1)) & ~1u) : m_n * srow_bytes + kb * 2;
    m_v[set] = __builtin_amdgcn_raw_buffer_load_b16(rs_m, off, 0, 0);
  };
  auto ring_store = [&](int set, int X) {
    const int kb = min(kb_beg + X, kb_last);
    const uint32_t zbit = (((m_n * zrow_bytes + (kb >> 1)) & 1u) << 3) | ((kb & 1) << 2);
    const uint32_t v = m_zero ? (m_v[set] >> zbit) & 0xFu : m_v[set] & 0xFFFFu;
    reinterpret_cast<uint16_t*>(s_meta)[2 * ((X & 1) * RP + m_lr) + m_zero] = (uint16_t)v;
  };

  // ---- prologue: chunk 0 in LDS, chunks 1..AQ in flight, PF k-blocks of weights in flight.
  // Prefetch indices past the range are clamped to the last k-block (a redundant, in-bounds load),
  // so the number of loads in flight is the same on every path.
  // The first weight k-blocks, then the first activation chunk (whose addresses wait on the slot
  // ids), are requested before the scales are staged, so one memory latency covers them all (the
  // staging waits for its own loads, issued last).
#pragma unroll
  for (int u = 0; u < PF; ++u) load_kb(u, min(kb_beg + u, kb_last));
  if constexpr (DIRECT) dma_a(0, 0);
  else load_a(0, 0);

  // ---- uint4 metadata.  BM <= 32: the whole K range of this split, fetched in even-aligned pairs
  // of k-blocks (one 4-byte load holds two scales, one byte two zero points); a pair straddling
  // either end of the range writes only its in-range half.  BM >= 64: the ring's first k-blocks.
  if constexpr (RING) {
    // k-block 0 into slot 0 now; k-blocks 1 and 2 in flight
    ring_load(0, 0);
    ring_load(1, 1);
    ring_store(0, 0);
    ring_load(0, 2);
  } else if constexpr (BITS == 4) {
    // MULTI: rows of chunk g at g * R + lr, row pitch G * R + 2
    const int kb0 = kb_beg & ~1;
    const int npair = (kb_end - kb0 + 1) >> 1;
    for (int item = tid; item < G * R * npair; item += THREADS) {
      const int gl = item / npair;
      const int j = item - gl * npair;
      const int g = MULTI ? gl / R : 0;
      const int lr = gl - g * R;
      const uint32_t n =
          (uint32_t)(col_of(lr / (NTW * 16), (lr / 16) % NTW) + g * WG_COLS + (lr % 16));
      const int kb = kb0 + 2 * j;
      const uint32_t sc = __builtin_amdgcn_raw_buffer_load_b32(rs_s, n * srow_bytes + kb * 2, 0, 0);
      const uint32_t zb = __builtin_amdgcn_raw_buffer_load_b8(rs_z, n * zrow_bytes + (kb >> 1), 0, 0);
      if (kb >= kb_beg) s_meta[(kb - kb_beg) * RPM + gl] = (sc & 0xFFFFu) | ((zb & 0xFu) << 16);
      if (kb + 1 < kb_end)
        s_meta[(kb + 1 - kb_beg) * RPM + gl] = (sc >> 16) | (((zb >> 4) & 0xFu) << 16);
    }
  }

  if constexpr (DIRECT) wait_vmcnt<0>();  // chunk 0 has landed (behind the first weights)
  else store_a(0, 0);
  barrier_lds();  // publishes the staged scales and chunk 0
  if constexpr (DIRECT) {
    dma_a(1, 1);
  } else if constexpr (!MULTI) {
#pragma unroll
    for (int q = 1; q <= AQ; ++q) load_a(q % AQ, q);
  }
  load_meta(0);

  // biased uint4 codes of one k-block (weights in wq[slot], metadata meta[t] = scale | zero << 16,
  // fragments from a_s(step, row tile)): the bias and the zero point are removed either by a
  // broadcast MFMA (BM 16: the matrix cores have room) or, for fp16 at BM 32, by one exact
  // half-precision subtraction per two weights ((1024 + q) - (1024 + z) = q - z), which halves the
  // MFMAs where they would otherwise bound the kernel.  The scale is applied per k-block.
  auto biased_u4_kb = [&](auto ma_c, int slot, const uint32_t* meta, auto&& a_s) {
    constexpr int MA = decltype(ma_c)::value;  // row tiles holding listed slots
    constexpr bool SUBZ = DT == 0 && MT == 2;
    floatx4_t accg[MA][NTW];
    u32x4_t bz[NTW];
    float sf[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const uint32_t z = meta[t] >> 16;
      const uint32_t zz = (kZeroBase | z) * 0x10001u;
      const uint32_t zh = DT == 0 ? (kZeroBase | (z << 4)) * 0x10001u : zz;
      bz[t] = u32x4_t{zz, zh, zz, zh};
      sf[t] = bits_to_float<DT>((uint16_t)(meta[t] & 0xFFFFu));
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      u32x4_t b[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        b[t] = bias_u4<DT>(wq[slot][t][st], kMask, kMaskHi, kMagic);
        if constexpr (SUBZ) {
          // element copies first: a bit_cast of a vector element reads element 0
          const uint32_t b0 = b[t][0], b1 = b[t][1], b2 = b[t][2], b3 = b[t][3];
          const uint32_t zlo = bz[t][0], zhi = bz[t][1];
          b[t] = u32x4_t{h2_add(b0, zlo), h2_add(b1, zhi), h2_add(b2, zlo), h2_add(b3, zhi)};
        }
      }
#pragma unroll
      for (int m = 0; m < MA; ++m)
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          accg[m][t] = Mfma<DT>::run(a_s(st, m), b[t], st == 0 ? zero4 : accg[m][t]);
          if constexpr (!SUBZ) accg[m][t] = Mfma<DT>::run(a_s(st, m), bz[t], accg[m][t]);
        }
    }
#pragma unroll
    for (int m = 0; m < MA; ++m)
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][t][i] = __builtin_fmaf(sf[t], accg[m][t][i], acc[m][t][i]);
  };

  // epilogue: lane holds rows 4*(lane/16)+i of each 16-row tile, column lane%16 (plus coff, the
  // column offset of a column group's chunk)
  auto store_out = [&](int coff) {
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
          const int cc = col[t] + rsub + coff;
          if constexpr (ACT) {
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
  };

  if constexpr (MULTI) {
    // Column groups: the whole K range of this split is activation chunk 0 (buffer 0, staged by
    // the prologue); k-block sequence idx = g * kb_n + kbi runs over the G chunks, the weight
    // prefetch running on across chunk edges (chunk g's rows sit g * WG_COLS rows further, a
    // uniform offset); at the end of each chunk its partials are written and the sums cleared.
    const int kb_n = kb_end - kb_beg;  // even (K % 256 == 0, unsplit) and at most one chunk
    const int total = G * kb_n;
    const uint32_t gstep = (uint32_t)WG_COLS * row_bytes;
    for (int it = 0; it < total; it += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int idx = it + j;
        const int g = idx / kb_n;
        const int kbi = idx - g * kb_n;
        const uint16_t* abase = frag_base(kbi, 0);
        auto a_s = [&](int st, int m) -> u32x4_t {
          return *(const u32x4_t*)(abase + m * 16 * LDA + st * 8);
        };
        uint32_t meta[NTW];
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          meta[t] = s_meta[kbi * RPM + g * R + (wave * NTW + t) * 16 + rsub];
        biased_u4_kb(std::integral_constant<int, MT>{}, j, meta, a_s);
        const int nidx = min(idx + PF, total - 1);
        const int ng = nidx / kb_n;
        const uint32_t soff = (uint32_t)ng * gstep + (uint32_t)(kb_beg + nidx - ng * kb_n) * 64;
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          wq[j][t] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_w, vw[t], soff, 0));
        if (kbi == kb_n - 1) {
          store_out(g * WG_COLS);
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int t = 0; t < NTW; ++t) acc[m][t] = zero4;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return;
  }

  // Whole unrolled iterations only: k-blocks past kb_end are virtual (zero activations, weights of
  // the last real k-block), so they add exact zeros.  Any exit inside the unrolled body would merge
  // into the loop header and make the compiler drain the prefetch at the top of every iteration.
  // the k loop for MA row tiles holding listed slots (a compile-time count: tiles past the block's
  // last listed slot, the tail of an expert's last block, are neither read nor multiplied)
  auto main_loop = [&](auto ma_c) {
    constexpr int MA = decltype(ma_c)::value;
    const int n_iter = (kb_end - kb_beg + U - 1) / U;
    for (int it = 0; it < n_iter; ++it) {
  #pragma unroll
      for (int j = 0; j < U; ++j) {
        const int idx = it * U + j;
        const int kb = kb_beg + idx;
        const int slot = j % PF;
        const int jc = j % KBC;
        const int c = idx / KBC;
        // buffer of chunk c: a constant where U / KBC is even (always for DIRECT)
        const int cb = (U / KBC) % 2 == 0 ? (j / KBC) & 1 : c & 1;
        // this k-block's activation fragments
        const uint16_t* abase = frag_base(jc, cb);
        auto a_s = [&](int st, int m) -> u32x4_t {
          if constexpr (DIRECT) {
            const int cl = jc * (KB / 8) + grp * (KB / 32) + st;  // logical chunk within the row
            return *(const u32x4_t*)(abuf(cb) + (m * 16 + rsub) * LDA + ((cl ^ swz(rsub)) * 8));
          }
          else return *(const u32x4_t*)(abase + m * 16 * LDA + st * 8);
        };
        uint32_t meta[NTW];
  #pragma unroll
        for (int t = 0; t < NTW; ++t) meta[t] = mf[t];
        if constexpr (BIASED && BITS == 4) {
          biased_u4_kb(ma_c, slot, meta, a_s);
        } else if constexpr (BIASED) {
          // int8: biased codes accumulate over all of K; row sums (ones MFMA) remove the bias at the end
  #pragma unroll
          for (int st = 0; st < STEPS; ++st) {
  #pragma unroll
            for (int m = 0; m < MA; ++m) rsum[m] = Mfma<DT>::run(a_s(st, m), ones, rsum[m]);
  #pragma unroll
            for (int t = 0; t < NTW; ++t) {
              const u32x4_t bb = bias_s8<DT>(wq[slot][t][2 * st], wq[slot][t][2 * st + 1]);
  #pragma unroll
              for (int m = 0; m < MA; ++m) acc[m][t] = Mfma<DT>::run(a_s(st, m), bb, acc[m][t]);
            }
          }
        } else {
          DecodeK dk[NTW];
          if constexpr (BITS == 4) {
  #pragma unroll
            for (int t = 0; t < NTW; ++t) dk[t] = make_decode<DT, 4>(meta[t] & 0xFFFFu, meta[t] >> 16);
          }
          // fragments of step s + 1 are read while step s decodes and multiplies (where the
          // registers allow: not for fp16 BM 128, whose activation staging needs them)
          constexpr bool STEP_AHEAD = DIRECT || MT <= 4;
          u32x4_t acur[MA];
          if constexpr (STEP_AHEAD) {
  #pragma unroll
            for (int m = 0; m < MA; ++m) acur[m] = a_s(0, m);
          }
  #pragma unroll
          for (int st = 0; st < STEPS; ++st) {
            u32x4_t anext[MA];
            if constexpr (STEP_AHEAD) {
              if (st + 1 < STEPS) {
  #pragma unroll
                for (int m = 0; m < MA; ++m) anext[m] = a_s(st + 1, m);
              }
            }
            u32x4_t b[NTW];
  #pragma unroll
            for (int t = 0; t < NTW; ++t) {
              if constexpr (BITS == 4)
                b[t] = decode_u4<DT>(wq[slot][t][st], dk[t], kMask, kMaskHi, kMagic);
              else
                b[t] = decode_s8<DT>(wq[slot][t][2 * st], wq[slot][t][2 * st + 1], dk8[t]);
            }
  #pragma unroll
            for (int m = 0; m < MA; ++m)
  #pragma unroll
              for (int t = 0; t < NTW; ++t)
                acc[m][t] = Mfma<DT>::run(STEP_AHEAD ? acur[m] : a_s(st, m), b[t], acc[m][t]);
            if constexpr (STEP_AHEAD) {
              if (st + 1 < STEPS) {
  #pragma unroll
                for (int m = 0; m < MA; ++m) acur[m] = anext[m];
              }
            }
          }
        }
        load_kb(slot, min(kb + PF, kb_last));
        if (jc == KBC - 1) {
          if constexpr (DIRECT) {
            // end of chunk c: chunk c+1 was requested before this chunk's KBC weight prefetches, so
            // waiting for all but those leaves it in LDS; then chunk c+2 into the buffer of chunk c
            wait_vmcnt<KBC * NTW>();
            if constexpr (RING) ring_store((j + 1) & 1, idx + 1);
            barrier_lds();
            if constexpr (RING) ring_load((j + 1) & 1, idx + 3);
            dma_a(c + 2, cb);
          } else {
            // end of chunk c: publish chunk c+1 (zeros past the range), then fetch chunk c+1+AQ
            const int q = ((j / KBC) + 1) % AQ;  // == (c + 1) % AQ, as U is a multiple of KBC * AQ
            store_a(q, cb ^ 1);
            if constexpr (RING) ring_store((j + 1) & 1, idx + 1);
            barrier_lds();
            if constexpr (RING) ring_load((j + 1) & 1, idx + 3);
            load_a(q, c + 1 + AQ);
          }
        }
        load_meta(idx + 1);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetches where they are issued
      }
    }
  };
  // 64-row blocks with activations straight into LDS (bf16 uint4, int8) only: with 16 or 32 rows,
  // or activations staged through registers (fp16 uint4), the extra loop copies cost a wavefront
  // per SIMD of registers (BLOCK_M 32: 128 -> 155; fp16 uint4 BLOCK_M 64: 152 -> 216)
  if constexpr (MT == 4 && DIRECT) {
    // listed slots are a prefix of the block (s_slot published by the prologue's barrier)
    const int n_valid = __builtin_popcountll(__ballot(lane < BM && s_slot[lane] >= 0));
    const int mt_valid = __builtin_amdgcn_readfirstlane((n_valid + 15) / 16);
    if (mt_valid >= 4) main_loop(std::integral_constant<int, 4>{});
    else if (mt_valid == 3) main_loop(std::integral_constant<int, 3>{});
    else if (mt_valid == 2) main_loop(std::integral_constant<int, 2>{});
    else main_loop(std::integral_constant<int, 1>{});
  } else {
    main_loop(std::integral_constant<int, MT>{});
  }

  // LDS-destination loads still in flight (chunks past the range) must land before the workgroup's
  // LDS can be handed to another workgroup
  if constexpr (DIRECT) wait_vmcnt<0>();

  if constexpr (BIASED && BITS == 8) {
    // remove the +128 bias (fp16: +1152 with the 1024 magic) and apply the per-channel scale
    const float bias = DT == 0 ? 1152.0f : 128.0f;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const float sc = bits_to_float<DT>(
          (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs_s, (uint32_t)(col[t] + rsub) * 2, 0, 0));
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][t][i] = sc * __builtin_fmaf(-bias, rsum[m][i], acc[m][t][i]);
    }
  }

  store_out(0);
}

template <int DT, int BITS, int MT, int NTW, int WV>
hipError_t launch_ntw(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
  const int n_out = c.act ? p.N / 2 : p.N;
  const int n_chunks = n_out / gemm_wg_cols(c);
  if (c.cgroup < 1 || n_chunks % c.cgroup) return hipErrorInvalidValue;
  const long long grid = (long long)(n_chunks / c.cgroup) * p.num_blocks * p.split_k;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = gemm_meta_lds_bytes(p.K, p.split_k, c);
  if (gemm_lds_bytes(p.K, p.split_k, c) > kGemmLdsLimit) return hipErrorInvalidValue;
  if (c.cgroup > 1) {
    if (!gemm_cgroup_fits(c, p.K, p.split_k)) return hipErrorInvalidValue;
    if constexpr (BITS == 4 && MT == 1) {
      hipLaunchKernelGGL((wna16_gemm_kernel<DT, BITS, MT, NTW, 0, 1, WV, 1>), dim3((unsigned)grid),
                         dim3(WV * kWave), lds, stream, p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (c.act)
    hipLaunchKernelGGL((wna16_gemm_kernel<DT, BITS, MT, NTW, 1, 0, WV>), dim3((unsigned)grid),
                       dim3(WV * kWave), lds, stream, p);
  else if (c.out_f32)
    hipLaunchKernelGGL((wna16_gemm_kernel<DT, BITS, MT, NTW, 0, 1, WV>), dim3((unsigned)grid),
                       dim3(WV * kWave), lds, stream, p);
  else
    hipLaunchKernelGGL((wna16_gemm_kernel<DT, BITS, MT, NTW, 0, 0, WV>), dim3((unsigned)grid),
                       dim3(WV * kWave), lds, stream, p);
  return hipGetLastError();
}

template <int DT, int BITS, int MT>
hipError_t launch_mt(const GemmParams& p, const GemmConfig& c, hipStream_t stream) {
  if (MT == 1 && c.ntw == 4) return launch_ntw<DT, BITS, MT, (MT == 1 ? 4 : 2), 4>(p, c, stream);
  if constexpr (MT >= 2) {
    if (c.waves == 8) return launch_ntw<DT, BITS, MT, 2, 8>(p, c, stream);
  }
  return launch_ntw<DT, BITS, MT, 2, 4>(p, c, stream);
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

// wavefronts per workgroup the launch uses (8 only where the kernel is built with 8: block_m >= 32
// with two column tiles)
static int gemm_waves(const GemmConfig& c) {
  return c.waves == 8 && c.block_m >= 32 ? 8 : 4;
}

size_t gemm_meta_lds_bytes(int K, int split_k, const GemmConfig& c) {
  if (c.bits != 4) return 0;
  const int ntw = (c.ntw == 4 && c.block_m == 16) ? 4 : 2;
  const int waves = gemm_waves(c);
  if (c.block_m >= 64) return (size_t)(waves * ntw * 16 + 2) * 2 * 4;  // two-slot ring
  const int kb_total = K / 128;
  const int kb_per = (kb_total + split_k - 1) / split_k;
  // row pitch R + 2 dwords (column groups: cgroup * R + 2)
  return (size_t)((c.cgroup > 1 ? c.cgroup : 1) * waves * ntw * 16 + 2) * kb_per * 4;
}

bool gemm_cgroup_fits(const GemmConfig& c, int K, int split_k) {
  using S = Shape<4, 1, 4>;
  return c.bits == 4 && c.block_m == 16 && !c.act && c.out_f32 && split_k == 1 && K <= S::KC;
}

template <int BITS, int MT>
constexpr size_t static_lds_bytes() {
  using S = Shape<BITS, MT, 2>;  // the activation tiles do not depend on the column tiles
  return sizeof(uint16_t) * 2 * S::BM * S::LDA + 2 * sizeof(int) * S::BM;
}

size_t gemm_lds_bytes(int K, int split_k, const GemmConfig& c) {
  size_t st = 0;
  const bool b4 = c.bits == 4;
  switch (c.block_m) {
    case 16: st = b4 ? static_lds_bytes<4, 1>() : static_lds_bytes<8, 1>(); break;
    case 32: st = b4 ? static_lds_bytes<4, 2>() : static_lds_bytes<8, 2>(); break;
    case 64: st = b4 ? static_lds_bytes<4, 4>() : static_lds_bytes<8, 4>(); break;
    default: st = b4 ? static_lds_bytes<4, 8>() : static_lds_bytes<8, 8>(); break;
  }
  return st + gemm_meta_lds_bytes(K, split_k, c);
}

int gemm_wg_cols(const GemmConfig& c) {
  const int ntw = (c.ntw == 4 && c.block_m == 16) ? 4 : 2;
  return gemm_waves(c) * (c.act ? ntw / 2 : ntw) * 16;
}

hipError_t launch_gemm(const GemmParams& p_in, const GemmConfig& c, hipStream_t stream) {
  if (prefill_fits(c, p_in.N)) return launch_prefill(p_in, c, stream);
  if (c.block_m > 128) return hipErrorInvalidValue;  // 256-row blocks: the prefill kernel only
  GemmParams p = p_in;
  const int kb_total = p.K / (c.bits == 4 ? 128 : 64);
  if (p.split_k < 1 || p.split_k > kb_total || (p.split_k > 1 && !c.out_f32))
    return hipErrorInvalidValue;
  p.dec_mask = 0x000F000Fu;
  p.dec_mask_hi = (c.dtype == 0 && c.bits == 4) ? 0x00F000F0u : 0x000F000Fu;
  p.dec_magic = c.dtype == 0 ? 0x64006400u : 0x43004300u;
  p.cgroup = c.cgroup;
  if (c.dtype == 0)
    return c.bits == 4 ? launch_bits<0, 4>(p, c, stream) : launch_bits<0, 8>(p, c, stream);
  return c.bits == 4 ? launch_bits<1, 4>(p, c, stream) : launch_bits<1, 8>(p, c, stream);
}

}  // namespace moe
