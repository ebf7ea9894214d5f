// Device helpers shared by the libcsa2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// 16 bytes holding 8 bf16 -> 8 floats
__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ----------------------------------------------------------------- 4-bit formats
// E2M1 magnitude of a 3-bit field (exponent bias 1, one mantissa bit, subnormal at e=0):
// 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Built from the field, not from a table.
__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
  uint32_t e = (nib >> 1) & 3u, mb = nib & 1u;
  float mag = (e == 0) ? 0.5f * (float)mb : __uint_as_float((e - 1u + 127u) << 23) * (1.0f + 0.5f * (float)mb);
  return (nib & 8u) ? -mag : mag;
}
// OCP E4M3 ("FN"): bias 7, 3 mantissa bits, subnormal at e=0, S.1111.111 is NaN
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, mt = b & 7u;
  float mag;
  if (e == 0) mag = (float)mt * 0.001953125f;  // mt * 2^-9
  else if (e == 15u && mt == 7u) mag = __uint_as_float(0x7fc00000u);
  else mag = __uint_as_float((e - 7u + 127u) << 23) * (1.0f + 0.125f * (float)mt);
  return (b & 0x80u) ? -mag : mag;
}
// E8M0: 2^(b-127); b == 255 is NaN; b == 0 is 2^-127 (a float subnormal)
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  if (b == 255u) return __uint_as_float(0x7fc00000u);
  if (b == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(b << 23);
}

// ----------------------------------------------------------------- order-preserving keys
// Larger float -> larger key; -0 maps to +0's key so the two tie.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ----------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// sum over aligned groups of G lanes (G a power of two <= 64)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ----------------------------------------------------------------- RoPE angle
// cos/sin of pos * theta^(-2u/r): the angle is formed and reduced modulo 2*pi in fp64
// (positions reach 2^20, where an fp32 product loses ~0.06 rad), then evaluated in fp32.
__device__ __forceinline__ void rope_cos_sin(double pos, int u, int r, float theta, float* c, float* s) {
  double freq = exp2(-2.0 * (double)u / (double)r * log2((double)theta));
  double a = pos * freq;
  const double two_pi = 6.283185307179586476925286766559;
  a = a - two_pi * floor(a / two_pi);
  float af = (float)a;
  sincosf(af, s, c);
}

}  // namespace csa2
