// Device-side helpers shared by the decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace dec {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

// bf16 bit patterns packed two per 32-bit word: element 0 in the low half.
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// float32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}

// DPP lane moves inside one 16-lane row. Controls: quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16, 32, 64); every lane of
// a group receives the same, bitwise identical, group sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
  v += dpp_mov<0xB1>(v);
  if constexpr (N >= 4) v += dpp_mov<0x4E>(v);
  if constexpr (N >= 8) v += dpp_mov<0x141>(v);
  if constexpr (N >= 16) v += dpp_mov<0x140>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_mov<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_mov<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_mov<0x140>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float swiglu(float g, float u) { return silu(g) * u; }

// RoPE rotation of the pair (a, b) = (h_i, h_{i+d/2}) by the angle whose
// cosine and sine are c and s: (a c - b s, a s + b c). Written with explicit
// fused multiply-adds so every kernel that rotates rounds identically.
__device__ __forceinline__ void rope_rotate(float& a, float& b, float c, float s) {
  const float p0 = fmaf(a, c, -(b * s));
  const float p1 = fmaf(a, s, b * c);
  a = p0;
  b = p1;
}

}  // namespace dec
