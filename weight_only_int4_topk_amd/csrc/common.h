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

// Wave-wide arg-best over (value, index) pairs; every lane returns the winner.
__device__ __forceinline__ void wave_argbest(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off, kWave);
    int oi = __shfl_xor(i, off, kWave);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
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

}  // namespace moe
