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
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140,
// row_ror:8 = 0x128.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Values of lanes l and l ^ 16 (k = 16) or l and l ^ 32 (k = 32), as a pair
// that every lane of the two receives in the same order (lower lane first):
// v_permlane16_swap exchanges the odd 16-lane rows of one operand with the
// even rows of the other, v_permlane32_swap the upper half of one with the
// lower half of the other; with both operands v, the two results are the
// pair. No LDS traffic, unlike a shuffle through ds_bpermute.
template <int K>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  static_assert(K == 16 || K == 32, "pair distance");
  const uint32_t b = __float_as_uint(v);
  if constexpr (K == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  }
}

template <int K>
__device__ __forceinline__ float pair_sum(float v) {
  float lo, hi;
  lane_pair<K>(v, lo, hi);
  return lo + hi;
}

template <int K>
__device__ __forceinline__ float pair_max(float v) {
  float lo, hi;
  lane_pair<K>(v, lo, hi);
  return fmaxf(lo, hi);
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
  if constexpr (N >= 32) v = pair_sum<16>(v);
  if constexpr (N >= 64) v = pair_sum<32>(v);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_mov<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_mov<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_mov<0x140>(v));
  if constexpr (N >= 32) v = pair_max<16>(v);
  if constexpr (N >= 64) v = pair_max<32>(v);
  return v;
}

// Sum of v over the lanes l, l ^ S, l ^ 2S, ... (S = 8, 16 or 32): folds the
// groups of S lanes of a wave onto each other lane by lane. row_ror:8
// (0x128) gives lane l ^ 8 inside a 16-lane row.
template <int S>
__device__ __forceinline__ float fold_groups(float v) {
  static_assert(S == 8 || S == 16 || S == 32, "group width");
  if constexpr (S <= 8) v += dpp_mov<0x128>(v);
  if constexpr (S <= 16) v = pair_sum<16>(v);
  return pair_sum<32>(v);
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// Data other workgroups of the same launch read or wrote (they may run on
// other XCDs, whose L2 caches are not coherent with this one): two floats
// as one agent-scope atomic store (8-byte aligned address).
__device__ __forceinline__ void store_pair_agent(float* p, float lo, float hi) {
  const uint64_t v = uint64_t(__float_as_uint(lo)) | (uint64_t(__float_as_uint(hi)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two floats with one agent-scope atomic load (8-byte aligned address).
__device__ __forceinline__ float2 load_pair_agent(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(uint32_t(v)), __uint_as_float(uint32_t(v >> 32)));
}

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
