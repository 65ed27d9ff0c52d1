// Shared device helpers of the CSA / HCA HIP library (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ----------------------------------------------------------------------------
// bf16 <-> fp32.  Writes round to nearest, ties to even (NaN stays NaN).
// ----------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ----------------------------------------------------------------------------
// OCP fp8 e4m3 ("fn"): decode and RNE-saturating encode of an fp32 value.
// ----------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t mt = c & 0x7u;
  float v;
  if (e == 0) v = (float)mt * 0.001953125f;                    // mt * 2^-9
  else v = __uint_as_float(((e + 120u) << 23) | (mt << 20));  // (8+mt) * 2^(e-10)
  return __uint_as_float(__float_as_uint(v) | s);
}

__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t s = (u >> 24) & 0x80u;
  float a = fabsf(y);
  if (!(a < 448.0f)) return s | 0x7eu;  // saturate (and NaN -> max, unspecified input)
  if (a < 0.015625f) {                   // below 2^-6: subnormal grid, step 2^-9
    float q = rintf(a * 512.0f);         // exact scaling, RNE
    return s | (uint32_t)q;              // q == 8 encodes 2^-6 (exp 1, mant 0)
  }
  uint32_t ua = __float_as_uint(a);
  int e = (int)((ua >> 23) & 0xffu) - 127;
  uint32_t m23 = ua & 0x7fffffu;
  uint32_t m3 = m23 >> 20, rem = m23 & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  if (m3 == 8u) { m3 = 0; ++e; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | m3;
  if (code > 0x7eu) code = 0x7eu;
  return s | code;
}

// ----------------------------------------------------------------------------
// MXFP4 (e2m1 elements, e8m0 block scale over 32 elements)
// ----------------------------------------------------------------------------
// scale exponent e = floor(log2(amax)) - 2, clamped to [-127, 127]; amax = 0 -> -127
__device__ __forceinline__ int mx_scale_exp(float amax) {
  uint32_t E = (__float_as_uint(amax) >> 23) & 0xffu;
  if (amax == 0.0f || E == 0) return -127;  // zero or subnormal: floor(log2) <= -127
  int e = (int)E - 127 - 2;
  return e < -127 ? -127 : e;
}

// |v| already divided by 2^e -> magnitude code 0..7, nearest, ties to even code
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  return a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
       : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
}

__device__ __forceinline__ uint32_t f32_to_e2m1(float x, int e) {
  float a = ldexpf(fabsf(x), -e);
  return e2m1_mag_code(a) | ((__float_as_uint(x) >> 28) & 0x8u);
}

// ----------------------------------------------------------------------------
// order-preserving uint32 key of a float (descending float == descending key);
// -0.0 is mapped to +0.0 first so the two compare equal.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum over the wave: DPP within rows of 16 (quad_perm [1,0,3,2] and [2,3,0,1],
// row_half_mirror, row_mirror), then the four row results by readlane (no LDS permutes).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Element loaders used by the plain (VALU) kernels.
__device__ __forceinline__ float load_elem(const void* p, int dtype, int64_t i) {
  if (dtype == CSA_F32) return ((const float*)p)[i];
  if (dtype == CSA_BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  return e4m3_to_f32(((const uint8_t*)p)[i]);
}

// Wave-wide min / max of a uint32 with DPP row ops (VALU, no LDS round trip):
// reduce within each 16-lane row, then combine the four rows via readlane.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  // quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ int visible_blocks(int t, int m) { return t < 0 ? 0 : (t + 1) / m; }

}  // namespace csa
