// Device-side helpers shared by the gfx950 kernels of the moe_wna16 library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// (value, index) order used by every top-k: larger value first, equal values -> lower index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// DPP lane movements inside a 16-lane row (no LDS round trip): partner = lane ^ 1, lane ^ 2, the
// mirror lane in the 8-lane half row, the mirror lane in the row.  After the four steps of a
// butterfly every lane of a row holds the row's result.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ void argbest_step(float& v, int& i) {
  const float ov = dpp_f<CTRL>(v);
  const int oi = dpp_i<CTRL>(i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Exchange between 16-lane rows (r0<->r1, r2<->r3) and between the 32-lane halves, gfx950
// v_permlane16_swap / v_permlane32_swap: with both operands = x, the two results hold x of both
// rows (halves) of the lane's pair, in every lane.
template <bool HALVES>
__device__ __forceinline__ void swap_pair(uint32_t x, uint32_t& a, uint32_t& b) {
  if constexpr (HALVES) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  }
}

template <bool HALVES>
__device__ __forceinline__ void argbest_swap(float& v, int& i) {
  uint32_t va, vb, ia, ib;
  swap_pair<HALVES>(__float_as_uint(v), va, vb);
  swap_pair<HALVES>((uint32_t)i, ia, ib);
  const float fa = __uint_as_float(va), fb = __uint_as_float(vb);
  const bool a_wins = better(fa, (int)ia, fb, (int)ib);
  v = a_wins ? fa : fb;
  i = a_wins ? (int)ia : (int)ib;
}

// Wave-wide arg-best over (value, index) pairs; every lane returns the winner.  Rows of 16 lanes
// reduce with DPP, then rows pair up and halves pair up through lane swaps, all in vector
// registers (the order is total, so the result does not depend on the reduction order).
__device__ __forceinline__ void wave_argbest(float& v, int& i) {
  argbest_step<kDppXor1>(v, i);
  argbest_step<kDppXor2>(v, i);
  argbest_step<kDppHalfMirror>(v, i);
  argbest_step<kDppMirror>(v, i);
  argbest_swap<false>(v, i);
  argbest_swap<true>(v, i);
}

// Wave-wide sum in a fixed order (rows by DPP, then (row0 + row1) + (row2 + row3)); every lane
// returns the same value.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  uint32_t a, b;
  swap_pair<false>(__float_as_uint(v), a, b);
  v = __uint_as_float(a) + __uint_as_float(b);
  swap_pair<true>(__float_as_uint(v), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  // round to nearest even (gfx950 v_cvt_pk_bf16_f32)
  typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
  bf162_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi) {
  half2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

template <int DT>
__device__ __forceinline__ uint16_t float_to_bits(float f) {
  if constexpr (DT == 0) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  } else {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  }
}

template <int DT>
__device__ __forceinline__ float bits_to_float(uint16_t b) {
  if constexpr (DT == 0) {
    return (float)__builtin_bit_cast(_Float16, b);
  } else {
    return __uint_as_float((uint32_t)b << 16);
  }
}

// four float32 values rounded to dtype (0 fp16, 1 bf16) and stored as 8 bytes
template <int DT>
__device__ __forceinline__ void store4(uint16_t* dst, floatx4_t v) {
  const uint32_t lo = DT == 0 ? f32x2_to_f16x2(v[0], v[1]) : f32x2_to_bf16x2(v[0], v[1]);
  const uint32_t hi = DT == 0 ? f32x2_to_f16x2(v[2], v[3]) : f32x2_to_bf16x2(v[2], v[3]);
  *(uint2*)dst = make_uint2(lo, hi);
}

}  // namespace moe
