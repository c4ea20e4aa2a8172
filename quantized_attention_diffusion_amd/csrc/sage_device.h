// Device helpers for the gfx950 kernels: bf16 and e4m3 conversions, reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Unpack 8 bf16 values held in a 128-bit word.
__device__ __forceinline__ void bf16x8_to_f32(const uint4& w, float (&x)[8]) {
  x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
  x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
  x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xffff0000u);
  x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xffff0000u);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values -> two e4m3 codes in the low 16 bits (first value in the low byte).
// v_cvt_pk_fp8_f32 rounds to nearest even and yields NaN codes for magnitudes of
// 464 and more, so the inputs are clamped to +-448 first (saturating conversion).
__device__ __forceinline__ uint32_t e4m3x2_sat(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Reductions over the 4 lanes l, l^16, l^32, l^48 (one query's 4 lane groups) with the
// gfx950 cross-lane swaps: with both operands equal, v_permlane32_swap returns the low
// and the high 32 lanes each broadcast to both halves (v_permlane16_swap likewise for
// rows of 16), so combining its two results combines lane l with lane l^32 (l^16).
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// The maxima of two values (one per query group) over the 4 lane groups, in 7
// instructions for both: swapping a's upper half against b's lower half leaves lanes
// 0-31 holding a's and lanes 32-63 holding b's lane pairs (l, l^32), so one reduction
// serves both; a final swap broadcasts each half.  (The attention kernel is compiled
// without NaN semantics, so these maxima are single v_max_f32.)
__device__ __forceinline__ float max2_nan_free(float x, float y) { return fmaxf(x, y); }
__device__ __forceinline__ void max_over_lane_groups_pair(float& a, float& b) {
  const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const float r1 = max2_nan_free(__uint_as_float(s1[0]), __uint_as_float(s1[1]));
  const auto s2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(r1), __float_as_uint(r1), false, false);
  const float r2 = max2_nan_free(__uint_as_float(s2[0]), __uint_as_float(s2[1]));
  const auto s3 = __builtin_amdgcn_permlane32_swap(__float_as_uint(r2), __float_as_uint(r2), false, false);
  a = __uint_as_float(s3[0]);
  b = __uint_as_float(s3[1]);
}

__device__ __forceinline__ float sum_over_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Maximum over a 256-thread workgroup; `red` is 4 floats of LDS.  Ends with a barrier
// so `red` can be reused.
__device__ __forceinline__ float block256_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

}  // namespace sage
