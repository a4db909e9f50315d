// The layer for one token (M = 1) with uint4 experts in two launches.
//
// The same operation as the grouped GEMMs of the layer ("[Kernel] add triton fused moe kernel for
// gptq/awq", PR description: one launch over all experts; uint4 g128 with integer zero points):
//   up:   inter[j, n] = SiLU(W13[e_j, n, :] . x) * (W13[e_j, I + n, :] . x)      n < I
//   down: out[n]      = sum_j w_j * (W2[e_j, n, :] . inter[j, :])               n < H
// with (e_j, w_j) the token's top-k experts and routing weights.  With one token a block of the
// grouped GEMM holds one listed row of sixteen, and the layer's time goes to start-up and to the
// passes between its launches (routing, align, the split first GEMM's SiLU pass, the combine);
// here each weight row is one dot product, the first launch routes the token itself and the
// second adds the top-k products.
//
// Arithmetic.  Each lane takes whole 128-k quantisation groups of a row.  The 8 nibbles of a
// weight dword become four pairs of the activation dtype, (k0,k4) (k1,k5) (k2,k6) (k3,k7), each
// nibble shifted into the top four mantissa bits of a number with unit last place (fp16 1024,
// bf16 128): the pair value is magic + c q with c = 64 (fp16) or 8 (bf16), one shift and one
// and-or per pair.  v_dot2_f32_{f16,bf16} multiplies the pairs with the matching activation
// pairs (5-bit by 11- or 8-bit significands: exact in float32) into a float32 sum.  Per group,
//   sum_k (q_k - z) a_k = (sum_k (magic + c q_k) a_k - (magic + c z) sum_k a_k) / c,
// times the group scale, with sum_k a_k of every group formed once per workgroup; magic is at
// most twice c times the largest q - z, so the subtraction cancels at most about one bit.  The
// activations sit in LDS permuted per 8-k chunk to (a0,a4,a1,a5,a2,a6,a3,a7), and the 16 chunks
// of a group rotated by the group index, so the lanes of a wavefront, which read the same chunk of
// consecutive groups, hit different banks.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "route_body.h"

namespace moe {
namespace {

constexpr int kSWaves = 8;
constexpr int kSThreads = kSWaves * kWave;
constexpr int kRsrcS = 0x00020000;  // gfx9-family buffer descriptor: 32-bit data format

template <int DT>
__device__ __forceinline__ float dot2(uint32_t w, uint32_t a, float c) {
  if constexpr (DT == 0)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w), __builtin_bit_cast(half2_t, a), c,
                                  false);
  else {
    typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, w),
                                           __builtin_bit_cast(bf162_t, a), c, false);
  }
}

__device__ __forceinline__ uint32_t and_or_s(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);  // (a & m) | c
}

// Sum over aligned groups of L lanes (L a power of two <= 64) in a fixed order, in registers: DPP
// inside rows of 16, then row and half swaps; every lane of a group returns the group's sum.
__device__ __forceinline__ float lane_group_sum(float v, int L) {
  if (L >= 2) v += dpp_f<kDppXor1>(v);
  if (L >= 4) v += dpp_f<kDppXor2>(v);
  if (L >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (L >= 16) v += dpp_f<kDppMirror>(v);
  if (L >= 32) {
    uint32_t a, b;
    swap_pair<false>(__float_as_uint(v), a, b);
    v = __uint_as_float(a) + __uint_as_float(b);
  }
  if (L >= 64) {
    uint32_t a, b;
    swap_pair<true>(__float_as_uint(v), a, b);
    v = __uint_as_float(a) + __uint_as_float(b);
  }
  return v;
}

// LDS dword offset of 8-k chunk c of a staged vector: chunk r of group g sits at slot (r + g) % 16
__device__ __forceinline__ int chunk_pos(int g, int r) { return 4 * (g * 16 + ((r + g) & 15)); }

// Stage nvec activation vectors of length K (dtype, vector v = source row row_of(v) of src) into
// LDS: sx + v * K / 2 dwords in
// the permuted, rotated chunk layout, and ssum[v * G + g] = sum of group g of vector v (float32,
// the 8 values of a chunk in order, then the 16 chunks of a group by a butterfly).  Each thread
// issues the loads of four chunks before it stores any.
struct RowsInOrder {
  __device__ int operator()(int v) const { return v; }
};

template <int DT, typename RowOf = RowsInOrder>
__device__ void stage_vectors(const uint16_t* __restrict__ src, int nvec, int K,
                              uint32_t* __restrict__ sx, float* __restrict__ ssum,
                              RowOf row_of = RowOf()) {
  constexpr int kB = 4;
  const int nch = K / 8;
  const int G = K / 128;
  const int total = nvec * nch;  // a multiple of 16: whole 16-lane groups are in or out together
  for (int t0 = threadIdx.x; t0 < total; t0 += kB * kSThreads) {
    u32x4_t raw[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int t = t0 + b * kSThreads;
      if (t < total) {  // vector t / nch (source row row_of(t / nch)), chunk t % nch
        const int v = t / nch;
        raw[b] = *(const u32x4_t*)(src + (size_t)row_of(v) * K + (size_t)(t - v * nch) * 8);
      }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int t = t0 + b * kSThreads;
      if (t >= total) continue;
      const int v = t / nch;
      const int c = t - v * nch;
      const uint32_t r0 = raw[b][0], r1 = raw[b][1], r2 = raw[b][2], r3 = raw[b][3];
      const u32x4_t pv = {__builtin_amdgcn_perm(r2, r0, 0x05040100u),
                          __builtin_amdgcn_perm(r2, r0, 0x07060302u),
                          __builtin_amdgcn_perm(r3, r1, 0x05040100u),
                          __builtin_amdgcn_perm(r3, r1, 0x07060302u)};
      *(u32x4_t*)(sx + (size_t)v * (K / 2) + chunk_pos(c >> 4, c & 15)) = pv;
      float s = 0.f;
      const uint32_t rr[4] = {r0, r1, r2, r3};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s += bits_to_float<DT>((uint16_t)(rr[i] & 0xFFFFu));
        s += bits_to_float<DT>((uint16_t)(rr[i] >> 16));
      }
      s = lane_group_sum(s, 16);  // the 16 chunks of a group sit in one row of 16 lanes
      if ((c & 15) == 0) ssum[v * G + (c >> 4)] = s;
    }
  }
}

// Nibble pair d of a weight dword (k offsets d and d + 4) moved into the mask bits of its
// 16-bit halves: bits 6-9 (fp16) or 3-6 (bf16), the top four mantissa bits of the magic number.
template <int DT, int D>
__device__ __forceinline__ uint32_t pair_bits(uint32_t w) {
  constexpr int sh = DT == 0 ? 6 - 4 * D : 3 - 4 * D;
  if constexpr (sh >= 0) return w << sh;
  else return w >> (-sh);
}

// sum_k (magic + c q_k) a_k over the 128 k of group g: w = the group's 64 bytes (4 x 16), sv = the
// staged vector; four partial sums added in a fixed order
template <int DT>
__device__ __forceinline__ float group_dot(const u32x4_t (&w)[4], const uint32_t* sv, int g,
                                           uint32_t mask, uint32_t magic) {
  float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4_t a = *(const u32x4_t*)(sv + chunk_pos(g, 4 * q + d));
      const uint32_t a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
      const uint32_t wd = w[q][d];
      p0 = dot2<DT>(and_or_s(pair_bits<DT, 0>(wd), mask, magic), a0, p0);
      p1 = dot2<DT>(and_or_s(pair_bits<DT, 1>(wd), mask, magic), a1, p1);
      p2 = dot2<DT>(and_or_s(pair_bits<DT, 2>(wd), mask, magic), a2, p2);
      p3 = dot2<DT>(and_or_s(pair_bits<DT, 3>(wd), mask, magic), a3, p3);
    }
  }
  return (p0 + p1) + (p2 + p3);
}

// group_dot with the activation reads of one quarter group (4 chunks) at a time: the scheduler may
// not hoist later reads above the previous quarter's products, which bounds the registers
// the reads hold (the few-token kernels loop over slots around it)
template <int DT>
__device__ __forceinline__ float group_dot_lean(const u32x4_t (&w)[4], const uint32_t* sv, int g,
                                                uint32_t mask, uint32_t magic) {
  float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4_t a = *(const u32x4_t*)(sv + chunk_pos(g, 4 * q + d));
      const uint32_t a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
      const uint32_t wd = w[q][d];
      p0 = dot2<DT>(and_or_s(pair_bits<DT, 0>(wd), mask, magic), a0, p0);
      p1 = dot2<DT>(and_or_s(pair_bits<DT, 1>(wd), mask, magic), a1, p1);
      p2 = dot2<DT>(and_or_s(pair_bits<DT, 2>(wd), mask, magic), a2, p2);
      p3 = dot2<DT>(and_or_s(pair_bits<DT, 3>(wd), mask, magic), a3, p3);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return (p0 + p1) + (p2 + p3);
}

// group scale / c and magic + c z of the group's zero point (see the file comment)
template <int DT>
__device__ __forceinline__ void group_terms(uint32_t sbits, uint32_t zbyte, int g, float& sc,
                                            float& off) {
  constexpr float c = DT == 0 ? 64.0f : 8.0f;
  constexpr float magicv = DT == 0 ? 1024.0f : 128.0f;
  sc = bits_to_float<DT>((uint16_t)(sbits & 0xFFFFu)) * (1.0f / c);
  off = magicv + c * (float)((zbyte >> ((g & 1) * 4)) & 0xFu);
}


// ------------------------------------------------------------------------------------------------
// up: the workgroup routes the token and stages x; then one unit = (slot j, output column n):
// lanes 0-31 the gate row n, lanes 32-63 the up row I + n, lane l % 32 the groups l % 32 + 32 i,
// i < GPL.  A wavefront runs upw consecutive units in steps of one group per lane (GPL steps per
// unit, few registers per step so that more wavefronts are resident), the weights of the next step
// in flight while it computes one.
// ------------------------------------------------------------------------------------------------
template <int DT, int GPL>
__global__ void __launch_bounds__(kSThreads) single_up_kernel(SingleParams p) {
  extern __shared__ uint32_t s_dyn[];
  __shared__ RouteLds s_route;
  const int K = p.H, I = p.I;
  const int G = K / 128;
  uint32_t* sx = s_dyn;
  float* ssum = (float*)(s_dyn + K / 2);

  constexpr int P = GPL;                  // steps per unit (one group per lane and step)
  constexpr int QN = P == 1 ? 2 : P;      // steps per loop iteration (two slots alternate)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int U = p.topk * I;
  const int N = 2 * I;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const uint32_t srow = (uint32_t)G * 2;
  const uint32_t zrow = (uint32_t)(K / 256);
  constexpr uint32_t mask = DT == 0 ? 0x03C003C0u : 0x00780078u;
  constexpr uint32_t magic = DT == 0 ? 0x64006400u : 0x43004300u;
  const int u0 = (blockIdx.x * kSWaves + wave) * p.upw;

  // every workgroup routes the token; the first one publishes the result
  const float logit = (int)threadIdx.x < p.E ? p.logits[threadIdx.x] : 0.0f;
  const float wgt = route_single(logit, p.E, p.topk, p.rp, s_route);
  const int* s_ids = s_route.wid;
  if (blockIdx.x == 0 && (int)threadIdx.x < p.topk) {
    p.topk_ids[threadIdx.x] = s_ids[threadIdx.x];
    p.topk_w[threadIdx.x] = wgt;
  }

  u32x4_t wq[2][4];
  uint32_t sq[2], zq[2];
  auto load_step = [&](int slot, int k, int part) {
    const int u = min(u0 + k, U - 1);  // units past the end reload the last one (not stored)
    const int j = u / I;
    const int n = u - j * I;
    int e = s_ids[j];
    e = (unsigned)e < (unsigned)p.E ? e : 0;  // no id (NaN logits): rows of expert 0, unused
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.s13 + (size_t)e * N * srow), (short)0, (int)(N * srow), kRsrcS);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.z13 + (size_t)e * N * zrow), (short)0, (int)(N * zrow), kRsrcS);
    const uint32_t row = (uint32_t)(h ? I + n : n);
    // the weights through plain global loads: for this pattern (32 lanes x 64 bytes per row, two
    // rows per instruction) they stream faster than buffer loads (Mixtral shape 32.2 -> 29.4 us);
    // every address is inside expert e's rows
    const uint8_t* wrow = p.w13 + (size_t)e * N * row_bytes + (size_t)row * row_bytes;
    const int g = min(l32 + 32 * part, G - 1);  // past the row's groups: its last one
#pragma unroll
    for (int q = 0; q < 4; ++q) wq[slot][q] = *(const u32x4_t*)(wrow + g * 64 + q * 16);
    sq[slot] = __builtin_amdgcn_raw_buffer_load_b16(rs, row * srow + g * 2, 0, 0);
    zq[slot] = __builtin_amdgcn_raw_buffer_load_b8(rz, row * zrow + (g >> 1), 0, 0);
  };
  float acc = 0.f;
  auto compute_step = [&](int slot, int k, int part) {
    const int g = l32 + 32 * part;
    if (g < G) {
      float sc, off;
      group_terms<DT>(sq[slot], zq[slot], g, sc, off);
      const float d = group_dot<DT>(wq[slot], sx, g, mask, magic);
      acc += sc * (d - off * ssum[g]);
    }
    if (part != P - 1) return;
    // sum over the 32 lanes of each half, then gate (lane 0) and up (lane 32)
    acc = lane_group_sum(acc, 32);
    const float gate = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 0));
    const float up = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 32));
    const int u = u0 + k;
    if (lane == 0 && u < U) {
      const float v = gate / (1.0f + __expf(-gate)) * up;
      ((uint16_t*)p.inter)[u] = float_to_bits<DT>(v);  // u = j * I + n
    }
    acc = 0.f;
  };

  load_step(0, 0, 0);  // in flight while x is staged
  stage_vectors<DT>((const uint16_t*)p.x, 1, K, sx, ssum);
  __syncthreads();

  // step t = k * P + part uses slot t % 2
  for (int k = 0; k < p.upw; k += QN / P) {
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int kn = k + (q + 1) / P;
      if (kn < p.upw) load_step((q + 1) & 1, kn, (q + 1) % P);
      if (k + q / P < p.upw) compute_step(q & 1, k + q / P, q % P);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// down: a workgroup covers RW consecutive output rows; wavefront w takes slot j = w % topk and the
// rows of part w / topk (nrp = 8 / topk parts, RPW rows each; topk > 8: slots w, w + 8, ...).  A
// row's G groups spread over L lanes (the smallest power of two >= G, at most 64; TPL groups per
// lane, one per step: fewer registers, so more wavefronts in flight), 64 / L rows per pass.  Each
// wavefront leaves w_j * (row . inter[j]) per row in LDS; the workgroup then adds the slots in
// ascending j and writes the rows.  The first step's weights are requested before the
// intermediate rows are staged.
// ------------------------------------------------------------------------------------------------
template <int DT, int TPL>
__global__ void __launch_bounds__(kSThreads) single_down_kernel(SingleParams p) {
  extern __shared__ uint32_t s_dyn[];
  const int K = p.I, H = p.H, topk = p.topk;
  const int G = K / 128;
  uint32_t* sx = s_dyn;                                   // topk vectors of K
  float* ssum = (float*)(s_dyn + (size_t)topk * K / 2);  // topk x G
  float* spart = ssum + topk * G;                         // topk x RW row results

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int L = p.lanes_per_row;       // power of two, >= G / TPL
  const int RPP = kWave / L;           // rows per pass
  const int sub = lane & (L - 1);
  const int rsub = lane / L;
  const int RW = p.rows_per_wg;
  const int n0 = blockIdx.x * RW;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const uint32_t srow = (uint32_t)G * 2;
  const uint32_t zrow = (uint32_t)(K / 256);
  constexpr uint32_t mask = DT == 0 ? 0x03C003C0u : 0x00780078u;
  constexpr uint32_t magic = DT == 0 ? 0x64006400u : 0x43004300u;
  const int nrp = topk >= kSWaves ? 1 : kSWaves / topk;
  const int RPW = RW / nrp;            // rows of one wavefront's part (a multiple of RPP)
  const int passes = RPW / RPP;
  constexpr int P = TPL;               // steps per pass of rows (one group per lane and step)
  constexpr int QN = P == 1 ? 2 : P;   // steps per loop iteration (two slots alternate)

  // the (slot, part) a wavefront works on, set by select()
  int j = 0, part = 0;
  bool valid = false;
  float wj = 0.f;
  __amdgpu_buffer_rsrc_t rw, rs, rz;
  auto select = [&](int jw) {
    j = jw % topk;
    part = jw / topk;
    int e = p.topk_ids[j];
    valid = (unsigned)e < (unsigned)p.E;  // routing gives [0, E); anything else adds nothing
    wj = valid ? p.topk_w[j] : 0.0f;
    e = valid ? e : 0;
    rw = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w2 + (size_t)e * H * row_bytes), (short)0,
                                           (int)(H * row_bytes), kRsrcS);
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)p.s2 + (size_t)e * H * srow),
                                           (short)0, (int)(H * srow), kRsrcS);
    rz = __builtin_amdgcn_make_buffer_rsrc((void*)(p.z2 + (size_t)e * H * zrow), (short)0,
                                           (int)(H * zrow), kRsrcS);
  };

  u32x4_t wq[2][4];
  uint32_t sq[2], zq[2];
  auto load_step = [&](int slot, int ps, int gp) {
    const uint32_t row = (uint32_t)min(n0 + part * RPW + ps * RPP + rsub, H - 1);
    const int g = min(sub + L * gp, G - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wq[slot][q] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, row * row_bytes + g * 64 + q * 16, 0, 0));
    sq[slot] = __builtin_amdgcn_raw_buffer_load_b16(rs, row * srow + g * 2, 0, 0);
    zq[slot] = __builtin_amdgcn_raw_buffer_load_b8(rz, row * zrow + (g >> 1), 0, 0);
  };
  float acc = 0.f;
  auto compute_step = [&](int slot, int ps, int gp) {
    const uint32_t* sv = sx + (size_t)j * K / 2;
    const float* sj = ssum + j * G;
    const int g = sub + L * gp;
    if (g < G) {
      float sc, off;
      group_terms<DT>(sq[slot], zq[slot], g, sc, off);
      const float d = group_dot<DT>(wq[slot], sv, g, mask, magic);
      acc += sc * (d - off * sj[g]);
    }
    if (gp != P - 1) return;
    acc = lane_group_sum(acc, L);
    const int r = part * RPW + ps * RPP + rsub;  // row within the workgroup
    if (sub == 0) spart[j * RW + r] = valid ? wj * acc : 0.0f;
    acc = 0.f;
  };

  const int njw = topk * nrp;
  if (wave < njw) {  // in flight while the intermediate rows are staged
    select(wave);
    load_step(0, 0, 0);
  }
  stage_vectors<DT>((const uint16_t*)p.inter, topk, K, sx, ssum);
  __syncthreads();

  for (int jw = wave; jw < njw; jw += kSWaves) {
    if (jw != wave) {
      select(jw);
      load_step(0, 0, 0);
    }
    // step t = ps * P + gp uses slot t % 2
    for (int ps = 0; ps < passes; ps += QN / P) {
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const int pn = ps + (q + 1) / P;
        if (pn < passes) load_step((q + 1) & 1, pn, (q + 1) % P);
        if (ps + q / P < passes) compute_step(q & 1, ps + q / P, q % P);
      }
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < RW; r += kSThreads) {
    const int n = n0 + r;
    if (n >= H) continue;
    float v = 0.f;
    for (int jj = 0; jj < topk; ++jj) v += spart[jj * RW + r];
    ((uint16_t*)p.out)[n] = float_to_bits<DT>(v);
  }
}

// ------------------------------------------------------------------------------------------------
// A few tokens (2 <= M, at most kFewSlots slots): every workgroup sorts the slots by (expert, slot)
// itself; each distinct expert's weight rows are then read once and dotted with the rows of all
// the slots routed to it.  Launches: routing, few_up, few_down.
// ------------------------------------------------------------------------------------------------
constexpr int kFewSlots = 256;
constexpr int kFewUsers = 8;   // tokens at most

struct __attribute__((aligned(16))) GroupLds {
  int id[kFewSlots];            // expert of slot s (E for an id outside [0, E)); past S: INT_MAX
  int order[kFewSlots];         // the slots sorted by (expert, slot)
  int first[kFewSlots + 1];     // distinct expert d owns order[first[d] .. first[d + 1])
  int exp[kFewSlots];           // distinct expert d's id (E: ids outside [0, E), sorted last)
  float tw[kFewSlots];          // routing weight of slot s
  int wsum[kSWaves];
  int nd;                       // distinct experts
};

// Sort the S slots of ids by (expert, slot) and list the distinct experts; w (nullable): the slots'
// routing weights, copied to LDS.  Ends with a barrier.
__device__ void group_slots(const int32_t* __restrict__ ids, const float* __restrict__ w, int S,
                            int E, GroupLds& g) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  if (t < kFewSlots) {
    int e = t < S ? ids[t] : 0x7fffffff;
    if (t < S && (unsigned)e >= (unsigned)E) e = E;
    g.id[t] = e;
    if (w) g.tw[t] = t < S ? w[t] : 0.0f;
  }
  __syncthreads();
  if (t < S) {
    // place = slots before this one in (expert, slot) order; four ids per LDS read
    const int mine = g.id[t];
    int before = 0;
    for (int s4 = 0; s4 < S; s4 += 4) {
      const int4 o = *(const int4*)(g.id + s4);
      before += (o.x < mine || (o.x == mine && s4 + 0 < t)) ? 1 : 0;
      before += (o.y < mine || (o.y == mine && s4 + 1 < t)) ? 1 : 0;
      before += (o.z < mine || (o.z == mine && s4 + 2 < t)) ? 1 : 0;
      before += (o.w < mine || (o.w == mine && s4 + 3 < t)) ? 1 : 0;
    }
    g.order[before] = t;
  }
  __syncthreads();
  // runs of equal experts in sorted order: their starts, numbered by a ballot prefix count
  bool start = false;
  int eid = 0;
  if (t < S) {
    eid = g.id[g.order[t]];
    start = t == 0 || g.id[g.order[t - 1]] != eid;
  }
  const uint64_t m = __ballot(start);
  if (lane == 0) g.wsum[wave] = __popcll(m);
  __syncthreads();
  int d = __popcll(m & lanemask_lt(lane));
  for (int w = 0; w < wave; ++w) d += g.wsum[w];
  if (start) {
    g.first[d] = t;
    g.exp[d] = eid;
  }
  if (t == 0) {
    int nd = 0;
    for (int w = 0; w < kSWaves; ++w) nd += g.wsum[w];
    g.nd = nd;
    g.first[nd] = S;
  }
  __syncthreads();
}

// few_up: workgroup (d, chunk) takes distinct expert d's columns chunk * 8 upw ...; wavefront w its
// upw consecutive columns n.  Up to 32 groups per row (GPL 1): gate row n on lanes 0-31 and up row
// I + n on lanes 32-63, one group per lane, as single_up.  33 to 64 groups (GPL 2): the whole
// wavefront on one row at a time, gate row n, then up row I + n, one group per lane (each slot's
// gate value waits in LDS for its up value).  The x rows of the expert's slots (at most M, since a
// token's slots go to distinct experts) are staged in LDS; every row's weights, in registers,
// meet all of them.
template <int DT, int GPL>
__global__ void __launch_bounds__(kSThreads) few_up_kernel(SingleParams p) {
  static_assert(GPL == 1 || GPL == 2, "few_up: at most 64 groups per row");
  constexpr bool ROWS = GPL == 2;
  extern __shared__ uint32_t s_dyn[];
  __shared__ GroupLds sg;
  __shared__ float s_gate[kSWaves][kFewUsers];  // ROWS: each slot's gate value
  const int K = p.H, I = p.I;
  const int G = K / 128;
  const int S = p.M * p.topk;
  group_slots(p.topk_ids, nullptr, S, p.E, sg);
  const int cpw = kSWaves * p.upw;
  const int chunks = (I + cpw - 1) / cpw;
  const int d = blockIdx.x / chunks;
  const int ch = blockIdx.x - d * chunks;
  if (d >= sg.nd) return;  // uniform: the whole workgroup leaves
  const int e = sg.exp[d];
  if (e >= p.E) return;
  const int f0 = sg.first[d];
  const int nu = sg.first[d + 1] - f0;
  uint32_t* sx = s_dyn;                                    // M vectors of K
  float* ssum = (float*)(s_dyn + (size_t)p.M * K / 2);  // M x G

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int h = lane >> 5;
  const int gl = ROWS ? lane : (lane & 31);  // this lane's group
  const int N = 2 * I;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const uint32_t srow = (uint32_t)G * 2;
  const uint32_t zrow = (uint32_t)(K / 256);
  constexpr uint32_t mask = DT == 0 ? 0x03C003C0u : 0x00780078u;
  constexpr uint32_t magic = DT == 0 ? 0x64006400u : 0x43004300u;
  const int n_first = ch * cpw + wave * p.upw;
  const int nw = max(0, min(p.upw, I - n_first));  // this wavefront's columns
  const int nsteps = ROWS ? 2 * nw : nw;          // ROWS: step 2k gate row, 2k + 1 up row
  const uint8_t* wexp = p.w13 + (size_t)e * N * row_bytes;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)p.s13 + (size_t)e * N * srow), (short)0, (int)(N * srow), kRsrcS);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.z13 + (size_t)e * N * zrow), (short)0, (int)(N * zrow), kRsrcS);

  u32x4_t wq[2][1][4];
  uint16_t sq[2];
  uint8_t zq[2];
  auto load_step = [&](int slot, int st) {
    st = min(st, nsteps - 1);
    const int k = ROWS ? st >> 1 : st;
    const int n = n_first + k;
    const bool upper = ROWS ? (st & 1) : h;
    const uint32_t row = (uint32_t)(upper ? I + n : n);
    const uint8_t* wrow = wexp + (size_t)row * row_bytes;
    const int g = min(gl, G - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) wq[slot][0][q] = *(const u32x4_t*)(wrow + g * 64 + q * 16);
    sq[slot] = __builtin_amdgcn_raw_buffer_load_b16(rs, row * srow + g * 2, 0, 0);
    zq[slot] = __builtin_amdgcn_raw_buffer_load_b8(rz, row * zrow + (g >> 1), 0, 0);
  };

  {
    const int nb = nu;  // <= M (a token's slots go to distinct experts)
    if (nsteps > 0) load_step(0, 0);  // in flight while the rows are staged
    const int tk = p.topk;
    const int* ord = sg.order + f0;
    stage_vectors<DT>((const uint16_t*)p.x, nb, K, sx, ssum,
                      [ord, tk](int v) { return ord[v] / tk; });
    __syncthreads();
    if (nsteps == 0) return;
    // each slot's dot product is finished, reduced and written (or kept) in turn
    auto compute_step = [&](int slot, int st) {
      const int k = ROWS ? st >> 1 : st;
      const int n = n_first + k;
      float sc = 0.f, off = 0.f;
      if (gl < G) group_terms<DT>(sq[slot], zq[slot], gl, sc, off);
#pragma unroll 1
      for (int u = 0; u < nb; ++u) {
        float acc = 0.f;
        if (gl < G) {
          const float dd = group_dot_lean<DT>(wq[slot][0], sx + (size_t)u * K / 2, gl, mask, magic);
          acc = sc * (dd - off * ssum[u * G + gl]);
        }
        float gate, up;
        if constexpr (ROWS) {
          acc = lane_group_sum(acc, 64);
          if ((st & 1) == 0) {
            if (lane == 0) s_gate[wave][u] = acc;
            continue;
          }
          gate = s_gate[wave][u];
          up = acc;
        } else {
          acc = lane_group_sum(acc, 32);
          gate = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 0));
          up = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 32));
        }
        if (lane == 0) {
          const float v = gate / (1.0f + __expf(-gate)) * up;
          ((uint16_t*)p.inter)[(size_t)ord[u] * I + n] = float_to_bits<DT>(v);
        }
      }
    };
    // the next step's weights in flight while one is computed
    for (int st = 0; st < nsteps; st += 2) {
      load_step(1, st + 1);
      compute_step(0, st);
      load_step(0, st + 2);
      if (st + 1 < nsteps) compute_step(1, st + 1);
    }
  }
}

// few_down: a workgroup covers RW consecutive output rows for every slot; wavefront w takes the
// distinct experts d = w, w + 8, ... and, for each, the row sets of the block (64 / L rows per
// set, as single_down), dotting every row with the intermediate rows of all of d's slots.  The
// results w_s * (row . inter[s]) wait in LDS per slot; each token's output row is the sum over its
// slots j = 0 .. topk - 1 in ascending order.
template <int DT, int TPL>
__global__ void __launch_bounds__(kSThreads) few_down_kernel(SingleParams p) {
  static_assert(TPL == 1, "few_down: one group per lane");
  extern __shared__ uint32_t s_dyn[];
  __shared__ GroupLds sg;
  const int K = p.I, H = p.H, topk = p.topk;
  const int G = K / 128;
  const int S = p.M * topk;
  const int RW = p.rows_per_wg;
  uint32_t* sx = s_dyn;                                // S vectors of K
  float* ssum = (float*)(s_dyn + (size_t)S * K / 2);  // S x G
  float* spart = ssum + S * G;                        // S x RW
  group_slots(p.topk_ids, p.topk_w, S, p.E, sg);
  stage_vectors<DT>((const uint16_t*)p.inter, S, K, sx, ssum);
  for (int i = threadIdx.x; i < S * RW; i += kSThreads) spart[i] = 0.0f;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int L = p.lanes_per_row;
  const int RPP = kWave / L;
  const int sub = lane & (L - 1);
  const int rsub = lane / L;
  const int n0 = blockIdx.x * RW;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const uint32_t srow = (uint32_t)G * 2;
  const uint32_t zrow = (uint32_t)(K / 256);
  constexpr uint32_t mask = DT == 0 ? 0x03C003C0u : 0x00780078u;
  constexpr uint32_t magic = DT == 0 ? 0x64006400u : 0x43004300u;
  constexpr int CH = 1;  // one group per lane
  const int passes = RW / RPP;
  const int nd = sg.nd;
  const int nmine = wave < nd ? (nd - wave + kSWaves - 1) / kSWaves : 0;  // experts of this wave
  const int n_items = nmine * passes;  // item it = (expert wave + 8 (it / passes), pass it % passes)

  u32x4_t wq[2][CH][4];
  uint16_t sq[2][CH];
  uint8_t zq[2][CH];
  auto load_step = [&](int slot, int it, int gp) {
    it = min(it, n_items - 1);
    const int kd = it / passes;
    const int ps = it - kd * passes;
    int e = sg.exp[wave + kSWaves * kd];
    e = e < p.E ? e : 0;  // ids outside [0, E): loaded from expert 0, not used
    const uint32_t row = (uint32_t)min(n0 + ps * RPP + rsub, H - 1);
    const uint8_t* wrow = p.w2 + ((size_t)e * H + row) * row_bytes;
    const uint8_t* srw = (const uint8_t*)p.s2 + ((size_t)e * H + row) * srow;
    const uint8_t* zrw = p.z2 + ((size_t)e * H + row) * zrow;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int g = min(sub + L * (gp * CH + i), G - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) wq[slot][i][q] = *(const u32x4_t*)(wrow + g * 64 + q * 16);
      sq[slot][i] = *(const uint16_t*)(srw + g * 2);
      zq[slot][i] = zrw[g >> 1];
    }
  };
  auto compute_step = [&](int slot, int it, int gp) {
    const int kd = it / passes;
    const int ps = it - kd * passes;
    const int dd = wave + kSWaves * kd;
    if (sg.exp[dd] >= p.E) return;  // slots without an expert keep their zero results
    const int f0 = sg.first[dd];
    const int nu = sg.first[dd + 1] - f0;
    const int r = ps * RPP + rsub;
#pragma unroll 1
    for (int u = 0; u < nu; ++u) {
      const int s = sg.order[f0 + u];
      const uint32_t* su = sx + (size_t)s * K / 2;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int g = sub + L * i;
        if (g < G) {
          float sc, off;
          group_terms<DT>(sq[slot][i], zq[slot][i], g, sc, off);
          const float d = group_dot_lean<DT>(wq[slot][i], su, g, mask, magic);
          acc += sc * (d - off * ssum[s * G + g]);
        }
      }
      acc = lane_group_sum(acc, L);
      if (sub == 0) spart[s * RW + r] = sg.tw[s] * acc;
    }
  };
  if (n_items > 0) {
    // the next item's weights in flight while one is computed
    load_step(0, 0, 0);
    for (int it = 0; it < n_items; it += 2) {
      if (it + 1 < n_items) load_step(1, it + 1, 0);
      compute_step(0, it, 0);
      if (it + 2 < n_items) load_step(0, it + 2, 0);
      if (it + 1 < n_items) compute_step(1, it + 1, 0);
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < p.M * RW; idx += kSThreads) {
    const int m = idx / RW;
    const int r = idx - m * RW;
    const int n = n0 + r;
    if (n >= H) continue;
    float v = 0.f;
    for (int j = 0; j < topk; ++j) v += spart[(m * topk + j) * RW + r];
    ((uint16_t*)p.out)[(size_t)m * H + n] = float_to_bits<DT>(v);
  }
}

constexpr int kCUs = 256;              // MI355X compute units
constexpr size_t kLdsPerCU = 160 * 1024;

// Workgroups of a kernel that one compute unit holds at once by its registers.
template <typename F>
int occupancy_of(F kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kSThreads, 0) != hipSuccess || n < 1)
    n = 1;
  return n;
}
// ... and by its LDS as well (`lds` dynamic bytes plus the static arrays)
constexpr size_t kStaticLds = sizeof(RouteLds);
int resident_per_cu(int by_regs, size_t lds) {
  return std::max(1, std::min(by_regs, (int)(kLdsPerCU / (lds + kStaticLds))));
}

// Launch shape of the down kernel: L lanes per row (a power of two covering the row's groups in at
// most 4 per lane), rows per workgroup a multiple of nrp * (64 / L).
struct DownPlan {
  int lanes, tpl, unit;
  size_t lds_fixed;  // staged rows and group sums (the row results add topk * 4 bytes per row)
};

DownPlan down_plan(int H, int I, int topk) {
  DownPlan d{};
  const int G = I / 128;
  d.lanes = 1;
  while (d.lanes < G && d.lanes < kWave) d.lanes <<= 1;
  d.tpl = (G + d.lanes - 1) / d.lanes;
  const int nrp = topk >= kSWaves ? 1 : kSWaves / topk;
  d.unit = nrp * (kWave / d.lanes);
  d.lds_fixed = (size_t)topk * I * 2 + (size_t)topk * G * 4;
  return d;
}

size_t up_lds(int H) { return (size_t)H * 2 + (size_t)(H / 128) * 4; }

template <int DT, int GPL>
hipError_t launch_up(SingleParams& p, hipStream_t stream) {
  static const int occ = occupancy_of(single_up_kernel<DT, GPL>);
  const size_t lds = up_lds(p.H);
  const int U = p.topk * p.I;
  // one round of resident workgroups, each wavefront a run of consecutive units
  const int slots = kCUs * resident_per_cu(occ, lds);
  int grid = std::min((U + kSWaves - 1) / kSWaves, slots);
  p.upw = (U + grid * kSWaves - 1) / (grid * kSWaves);
  grid = (U + kSWaves * p.upw - 1) / (kSWaves * p.upw);
  hipLaunchKernelGGL((single_up_kernel<DT, GPL>), dim3(grid), dim3(kSThreads), lds, stream, p);
  return hipGetLastError();
}

template <int DT, int TPL>
hipError_t launch_down(SingleParams& p, const DownPlan& d, hipStream_t stream) {
  static const int occ = occupancy_of(single_down_kernel<DT, TPL>);
  // one round of resident workgroups (rows per workgroup a multiple of the plan's unit)
  const int units = (p.H + d.unit - 1) / d.unit;
  size_t lds = d.lds_fixed + (size_t)p.topk * d.unit * 4;
  const int slots = kCUs * resident_per_cu(occ, lds);
  p.rows_per_wg = d.unit * ((units + slots - 1) / slots);
  p.lanes_per_row = d.lanes;
  const int grid = (p.H + p.rows_per_wg - 1) / p.rows_per_wg;
  lds = d.lds_fixed + (size_t)p.topk * p.rows_per_wg * 4;
  hipLaunchKernelGGL((single_down_kernel<DT, TPL>), dim3(grid), dim3(kSThreads), lds, stream, p);
  return hipGetLastError();
}

// ---- a few tokens
size_t few_up_lds(int H, int M) { return (size_t)M * ((size_t)H * 2 + (size_t)(H / 128) * 4); }
size_t few_down_lds(int I, int S, int rows) {
  return (size_t)S * I * 2 + (size_t)S * (I / 128) * 4 + (size_t)S * rows * 4;
}

template <int DT, int GPL>
hipError_t launch_few_up(SingleParams& p, hipStream_t stream) {
  const int S = p.M * p.topk;
  const int dmax = std::min(p.E + 1, S);
  // about 512 workgroups when dmax experts are active, each a run of columns of one expert
  const int chunks = std::max(1, std::min(p.I / kSWaves, 512 / dmax));
  const int cpw = ((p.I + chunks - 1) / chunks + kSWaves - 1) / kSWaves * kSWaves;
  p.upw = cpw / kSWaves;
  const int grid = dmax * ((p.I + cpw - 1) / cpw);
  hipLaunchKernelGGL((few_up_kernel<DT, GPL>), dim3(grid), dim3(kSThreads),
                     few_up_lds(p.H, p.M), stream, p);
  return hipGetLastError();
}

template <int DT, int TPL>
hipError_t launch_few_down(SingleParams& p, int lanes, hipStream_t stream) {
  const int S = p.M * p.topk;
  const int rpp = kWave / lanes;
  const int sets = (p.H + rpp - 1) / rpp;
  int rows = rpp * ((sets + kCUs - 1) / kCUs);
  while (rows > rpp && few_down_lds(p.I, S, rows) + sizeof(GroupLds) > kLdsPerCU) rows -= rpp;
  p.rows_per_wg = rows;
  p.lanes_per_row = lanes;
  const int grid = (p.H + rows - 1) / rows;
  hipLaunchKernelGGL((few_down_kernel<DT, TPL>), dim3(grid), dim3(kSThreads),
                     few_down_lds(p.I, S, rows), stream, p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_few_dt(const SingleParams& p_in, hipStream_t stream) {
  SingleParams p = p_in;
  const int Gu = p.H / 128;
  hipError_t e = Gu <= 32 ? launch_few_up<DT, 1>(p, stream) : launch_few_up<DT, 2>(p, stream);
  if (e != hipSuccess) return e;
  const int Gd = p.I / 128;
  int L = 1;
  while (L < Gd && L < kWave) L <<= 1;
  const int tpl = (Gd + L - 1) / L;
  (void)tpl;  // I <= 8192: at most 64 groups, one per lane
  return launch_few_down<DT, 1>(p, L, stream);
}

template <int DT>
hipError_t launch_single_dt(const SingleParams& p_in, hipStream_t stream) {
  SingleParams p = p_in;
  const int Gu = p.H / 128;
  hipError_t e = Gu <= 32   ? launch_up<DT, 1>(p, stream)
                 : Gu <= 64  ? launch_up<DT, 2>(p, stream)
                 : Gu <= 128 ? launch_up<DT, 4>(p, stream)
                             : launch_up<DT, 8>(p, stream);
  if (e != hipSuccess) return e;
  const DownPlan d = down_plan(p.H, p.I, p.topk);
  return d.tpl <= 1   ? launch_down<DT, 1>(p, d, stream)
         : d.tpl <= 2 ? launch_down<DT, 2>(p, d, stream)
                      : launch_down<DT, 4>(p, d, stream);  // I <= 32768: at most 4 per lane
}

}  // namespace

bool single_fits(int H, int I, int E, int topk) {
  if (H % 256 || I % 256 || E < 1 || E > 256 || topk < 1 || topk > E || topk > kWave) return false;
  if (H > 32768 || I > 32768) return false;  // at most 8 (up) and 4 (down) groups per lane
  const DownPlan d = down_plan(H, I, topk);
  // the most rows a down workgroup takes: one round over at least kCUs workgroups
  const size_t units = (size_t)((H + d.unit - 1) / d.unit);
  const size_t rows = (size_t)d.unit * ((units + kCUs - 1) / kCUs);
  return up_lds(H) + kStaticLds <= kLdsPerCU && d.lds_fixed + (size_t)topk * rows * 4 <= kLdsPerCU;
}

hipError_t launch_single(const SingleParams& p, int dtype, hipStream_t stream) {
  if (!single_fits(p.H, p.I, p.E, p.topk)) return hipErrorInvalidValue;
  return dtype == 0 ? launch_single_dt<0>(p, stream) : launch_single_dt<1>(p, stream);
}

bool few_fits(int M, int H, int I, int E, int topk) {
  const int S = M * topk;
  if (M < 2 || M > kFewUsers || S > kFewSlots || H % 256 || I % 256 || E < 1 || topk < 1)
    return false;
  if (H > 8192 || I > 8192) return false;  // at most 64 groups per row: one per lane
  int L = 1;
  while (L < I / 128 && L < kWave) L <<= 1;
  return few_down_lds(I, S, kWave / L) + sizeof(GroupLds) <= kLdsPerCU &&
         few_up_lds(H, M) + sizeof(GroupLds) <= kLdsPerCU;
}

hipError_t launch_few(const SingleParams& p, int dtype, hipStream_t stream) {
  if (!few_fits(p.M, p.H, p.I, p.E, p.topk)) return hipErrorInvalidValue;
  return dtype == 0 ? launch_few_dt<0>(p, stream) : launch_few_dt<1>(p, stream);
}

}  // namespace moe
