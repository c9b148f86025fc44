// Small device helpers shared by the kernels of libmla.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32 (round to nearest even on the way down; NaN kept quiet)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// round-to-nearest-even fp32 -> bf16 (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// load element i of a tensor stored as f32 / bf16 (dtype code 0 / 1)
__device__ __forceinline__ float load_elem(const void* p, long long i, int dtype) {
  if (dtype == 0) return ((const float*)p)[i];
  return bf16_bits_to_f32(((const uint16_t*)p)[i]);
}
__device__ __forceinline__ void store_elem(void* p, long long i, float v, int dtype) {
  if (dtype == 0)
    ((float*)p)[i] = v;
  else
    ((uint16_t*)p)[i] = f32_to_bf16_bits(v);
}

// OCP e4m3fn byte -> fp32 (exact), written from the format definition
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag;
  if (e == 0)
    mag = (float)m * 0.001953125f;  // m/8 * 2^-6
  else if (e == 15 && m == 7)
    mag = __builtin_nanf("");
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace mla
