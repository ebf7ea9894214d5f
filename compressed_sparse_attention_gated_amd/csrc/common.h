// Device helpers shared by the libcsa2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
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
// round to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
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
// Lane exchanges without address arithmetic: DPP within 16-lane rows, ds_swizzle across
// the two 16-lane rows of a 32-lane half, ds_bpermute (precomputed address) across halves.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16 lanes

// Index of the calling wave in its workgroup as a scalar: the compiler cannot prove that
// threadIdx.x / 64 is the same across a wave, so loops bounded by it would otherwise
// compile to exec-masked (divergent) control flow.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x / 64); }
// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load of the wave (vmcnt 0), which would drain register prefetches
// issued before it; this one waits for the wave's LDS operations alone, so prefetched
// tiles stay in flight across it.  Use it where the barrier orders LDS accesses only.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ float swz_xor16(float v) {  // lane l <- lane l^16 (within 32)
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (0x10 << 10) | 0x1F));
}
__device__ __forceinline__ float xor32(float v) {  // lane l <- lane l^32
  const int addr = ((__lane_id() ^ 32) << 2);
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}
// sum over all 64 lanes, returned in every lane
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  v += swz_xor16(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  v = fmaxf(v, swz_xor16(v));
  return fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
               __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)));
}
// gfx950 VALU lane swaps, no LDS round trip.  v_permlane16_swap exchanges the odd 16-lane
// rows of one register with the even rows of another, v_permlane32_swap the upper half of
// one with the lower half of the other.  Given two copies of v, each lane gets back its own
// value and that of lane l ^ 16 (or l ^ 32), in an order that depends on the lane, so they
// serve symmetric reductions only (a + b == b + a exactly, likewise max).
__device__ __forceinline__ void pair_xor16(float v, float* a, float* b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  *a = __uint_as_float(r[0]);
  *b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair_xor32(float v, float* a, float* b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  *a = __uint_as_float(r[0]);
  *b = __uint_as_float(r[1]);
}
// v of lane l plus v of lane l ^ 32 (the same sum, bit for bit, as an exchange through LDS)
__device__ __forceinline__ float sum_xor32(float v) {
  float a, b;
  pair_xor32(v, &a, &b);
  return a + b;
}
// sum / max over the 4 lanes l, l^16, l^32, l^48 (the four 16-lane rows); every lane active
__device__ __forceinline__ float rows_sum(float v) {
  float a, b;
  pair_xor16(v, &a, &b);
  pair_xor32(a + b, &a, &b);
  return a + b;
}
__device__ __forceinline__ float rows_max(float v) {
  float a, b;
  pair_xor16(v, &a, &b);
  pair_xor32(fmaxf(a, b), &a, &b);
  return fmaxf(a, b);
}
// sum over aligned groups of G lanes (G a power of two <= 64)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<kDppXor1>(v);
  if constexpr (G >= 4) v += dpp<kDppXor2>(v);
  if constexpr (G >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp<kDppMirror>(v);
  if constexpr (G >= 32) v += swz_xor16(v);
  if constexpr (G >= 64) v += xor32(v);
  return v;
}
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ----------------------------------------------------------------- RoPE angle
// Frequencies theta^(-2u/r), u < r/2, computed on the host in double precision and passed
// by value with the kernel arguments.
constexpr int kMaxRopePairs = 64;
struct RopeFreq {
  double f[kMaxRopePairs];
};
inline void rope_freq_host(RopeFreq* rf, int r, float theta) {
  for (int u = 0; u < kMaxRopePairs; ++u)
    rf->f[u] = (r > 0 && u < r / 2) ? pow((double)theta, -2.0 * (double)u / (double)r) : 0.0;
}

// cos/sin of pos * freq.  The angle (|pos| <= 2^31, freq <= 1) is formed and reduced by
// pi/2 in fp64 - a single fp32 product would lose ~0.06 rad at positions near 2^20 - and
// the reduced argument |x| <= pi/4 goes through the Taylor series of sin and cos in fp32
// (truncation below 2e-9), with the quadrant applied afterwards.
__device__ __forceinline__ void rope_cs(double pos, double freq, float* c, float* s) {
  const double a = pos * freq;
  const double q = rint(a * 0.63661977236758134308);          // 2/pi
  const double r = fma(-q, 1.5707963267948966192, a);         // pi/2
  const float x = (float)r, x2 = x * x;
  // sin x = x - x^3/3! + x^5/5! - x^7/7! + x^9/9!
  float sn = fmaf(x2, 1.0f / 362880.0f, -1.0f / 5040.0f);
  sn = fmaf(x2, sn, 1.0f / 120.0f);
  sn = fmaf(x2, sn, -1.0f / 6.0f);
  sn = fmaf(x2 * x, sn, x);
  // cos x = 1 - x^2/2! + x^4/4! - x^6/6! + x^8/8! - x^10/10!
  float cs = fmaf(x2, -1.0f / 3628800.0f, 1.0f / 40320.0f);
  cs = fmaf(x2, cs, -1.0f / 720.0f);
  cs = fmaf(x2, cs, 1.0f / 24.0f);
  cs = fmaf(x2, cs, -0.5f);
  cs = fmaf(x2, cs, 1.0f);
  const long long qi = (long long)q;
  switch (qi & 3) {
    case 0: *c = cs; *s = sn; break;
    case 1: *c = -sn; *s = cs; break;
    case 2: *c = -cs; *s = -sn; break;
    default: *c = sn; *s = -cs; break;
  }
}

}  // namespace csa2
