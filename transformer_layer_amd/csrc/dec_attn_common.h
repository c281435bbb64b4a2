// Split-K decode attention: what every attention kernel shares. The split
// partials (o unnormalized, and (m, l) with m in log2 units) are stored with
// agent-scope atomic stores, which reach the device-coherent level by
// themselves; unless the output projection combines them, the last
// workgroups of a kv head to arrive (one per ~8 KB of partials, at most
// kCombiners) combine them with a log-sum-exp rescale, each a slice of the
// head group's outputs. Every lane waits until its partial stores have
// completed (vmcnt 0), the workgroup meets at a barrier, and one thread
// increments the head's arrival counter with an agent-scope atomic.
// Combiners that arrive before the last one poll that counter (bounded: on
// giving up they set DEC_ERR_SYNC and write nothing) and read the partials
// with agent-scope loads. Every counter line is 64 bytes, so the heads'
// arrivals do not queue on one line; the last combiner to finish resets the
// line, so a kernel replays unchanged inside a graph.
#pragma once

#include "dec_device.h"
#include "dec_internal.h"

namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Part p (0: hi, 1: mid, 2: lo) of x as bf16 bits, for query operands of
// the matrix cores: hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi -
// mid), each difference exact in float32; hi + mid + lo holds x's 24-bit
// significand. Any other p gives lo as well.
__device__ __forceinline__ uint32_t q_part_bf16(float x, int p) {
  const uint16_t hi = f32_to_bf16(x);
  if (p == 0) return hi;
  const float r = x - bf16_to_f32(hi);
  const uint16_t mid = f32_to_bf16(r);
  if (p == 1) return mid;
  return f32_to_bf16(r - bf16_to_f32(mid));
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// The int8 query operand of the matrix cores: a head's scaled query x is
// taken as the integers X = rint(x 2^E), E chosen per head so that
// max |x| 2^E lies in [2^21, 2^22) (query_exp_i8), and each X splits
// exactly into three int8 digits, X = d0 + 2^8 d1 + 2^16 d2 with d0 and d1
// in [-128, 127] and |d2| <= 65. Returns the digits as the low bytes of
// an int each.
__device__ __forceinline__ int query_exp_i8(float m) {   // m = max |x| over the head
  return m > 0.0f ? 22 - __builtin_amdgcn_frexp_expf(m) : 0;
}
__device__ __forceinline__ void query_digits_i8(float x, int e, int& d0, int& d1, int& d2) {
  const float y = rintf(ldexpf(x, e));
  const int X = fabsf(y) <= 4194304.0f ? int(y) : 0;   // 2^22; a non-finite x (poisoned head) gives 0
  d0 = ((X + 128) & 255) - 128;
  const int X1 = (X - d0) >> 8;   // X - d0 is a multiple of 256
  d1 = ((X1 + 128) & 255) - 128;
  d2 = (X1 - d1) >> 8;
}
// A head whose query holds a NaN or an infinity gets exponent
// kQueryPoison instead: its scores are NaN, as the float arithmetic would
// make them, rather than whatever the digits of a non-finite value give.
constexpr int kQueryPoison = -1000000;
__device__ __forceinline__ int query_exp_i8_checked(float m, bool finite) {
  return finite ? query_exp_i8(m) : kQueryPoison;
}
// S0 + 2^8 S1 + 2^16 S2 of a row's three digit sums, times 2^-e
__device__ __forceinline__ float digit_score(int s0, int s1, int s2, int e) {
  const float v = ldexpf(fmaf(float(s2), 65536.0f, fmaf(float(s1), 256.0f, float(s0))), -e);
  return e == kQueryPoison ? __builtin_nanf("") : v;
}
template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

constexpr int kChunkMax = 256;  // cache positions per split
constexpr int kSplitMax = 256;  // splits per kv head
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCombiners = 8;          // workgroups that combine one kv head's splits
constexpr unsigned kSpinMax = 1u << 14;  // polls of a waiting combiner before it gives up
constexpr int kNotCombiner = -1, kGaveUp = -2;   // workgroup roles after arrival (else the combiner slot)

// 16 bytes of a cache row as floats: 4 f32 (KVT 0), 8 bf16 (KVT 1) or 16
// int8 codes (KVT 2, still to be multiplied by the row's scale)
template <int KVT>
__device__ __forceinline__ void unpack_row(u32x4 v, float* f) {
  if constexpr (KVT == 1) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
  } else if constexpr (KVT == 2) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * k + b] = float(int8_t(uint8_t(w[k] >> (8 * b))));
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

// One int8 cache row held two elements a lane across a wave (a row of 128):
// scale = max |x| / 127 and inv = 127 / max |x| (float32 divisions, rounded
// to nearest: the compiler's default for HIP), codes x * inv rounded half to
// even and clamped to [-127, 127]; a zero row gives scale 0, codes 0.
__device__ __forceinline__ void quantize_pair_i8(float2 x, float& c0, float& c1, float& scale) {
  const float m = wave_max(fmaxf(fabsf(x.x), fabsf(x.y)));
  const float inv = m > 0.0f ? 127.0f / m : 0.0f;
  scale = m > 0.0f ? m / 127.0f : 0.0f;
  c0 = fminf(fmaxf(rintf(x.x * inv), -127.0f), 127.0f);
  c1 = fminf(fmaxf(rintf(x.y * inv), -127.0f), 127.0f);
}

// two codes (integral floats in [-127, 127]) as the bytes of one 16-bit store
__device__ __forceinline__ uint16_t pack_i8_pair(float c0, float c1) {
  return uint16_t(uint8_t(int8_t(int(c0)))) | uint16_t(uint16_t(uint8_t(int8_t(int(c1)))) << 8);
}

// LDS the finish step reads or uses: the per-wave output sums
// ored [NW][G][D], the split's (m, l) stat [G][2], and the combine's
// scratch: wts [kSplitMax][G], den [G], accs [NW * 64], role.
struct AttnShared {
  float* ored;
  float* stat;
  float* wts;
  float* den;
  float4* accs;
  int* role;
};

// Split s of kv head j (of ns live splits): store its partials from LDS,
// then (unless the output projection combines) arrive and, for the last
// arrivals, combine. Every thread of the workgroup calls it.
// OW: how many per-wave copies of the output sums ored holds (their sum is
// the split's o); NW unless the waves wrote disjoint dims into copy 0.
template <int D, int G, int NW, int OW = NW>
__device__ __forceinline__ void attn_finish(const AttnArgs& a, int j, int s, int ns, AttnShared sh) {
  // ---- this split's partials: o [j][s][G][D] and (m, l) [j][s][G][2], as
  // agent-scope 64-bit atomic stores (pairs of floats)
  constexpr int kWaves = NW;
  constexpr int kBlock = NW * 64;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  float* po = a.part + (size_t(j) * a.nsplit + s) * G * D;
  float* pml = a.part + size_t(a.nkv) * a.nsplit * G * D + (size_t(j) * a.nsplit + s) * G * 2;
  auto osum = [&](int idx) {
    const int hh = idx / D, dd = idx % D;
    float r = sh.ored[hh * D + dd];
#pragma unroll
    for (int w = 1; w < OW; ++w) r += sh.ored[(w * G + hh) * D + dd];
    return r;
  };
  for (int i2 = threadIdx.x; i2 < G * D / 2; i2 += kBlock) store_pair_agent(po + 2 * i2, osum(2 * i2), osum(2 * i2 + 1));
  if (threadIdx.x < G) store_pair_agent(pml + threadIdx.x * 2, sh.stat[threadIdx.x * 2], sh.stat[threadIdx.x * 2 + 1]);

  if (a.partials_only) return;   // the output projection combines them

  // ---- arrival. The last ncomb splits of this kv head to arrive each
  // combine a slice of its outputs: the earlier ones wait (bounded) until
  // every split has arrived. Word 0 of the head's counter line counts
  // arrivals, word 1 finished combiners; the last combiner to finish resets
  // both for the next launch.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this lane's partial stores have completed
  __syncthreads();
  uint32_t* cnt = a.counters + size_t(j) * kCounterStride;
  // one combiner per ~8 KB of partials (o of every split), at most kCombiners
  int ncomb = ns * G * D / 2048;
  ncomb = ncomb < 1 ? 1 : ncomb > kCombiners ? kCombiners : ncomb;
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int slot = int(prev) - (ns - ncomb);   // combiner slot; negative: not a combiner
    bool gave_up = false;
    if (slot >= 0 && prev != unsigned(ns - 1)) {
      unsigned n = 0;
      // (no_wait, tests of this path: give up without polling)
      const unsigned spin_max = a.no_wait ? 0u : kSpinMax;
      while (a.no_wait || __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < unsigned(ns)) {
        if (++n > spin_max) {   // give up: flag it, write nothing, still count as finished
          atomicOr(a.err, kErrSync);
          gave_up = true;
          break;
        }
      }
    }
    *sh.role = slot < 0 ? kNotCombiner : gave_up ? kGaveUp : slot;
  }
  __syncthreads();
  const int w = *sh.role;
  if (w == kNotCombiner) return;

  if (w >= 0) {
    // (drop_last, tests of the parity gates: the last split is left out)
    const int nsum = a.drop_last && ns > 1 ? ns - 1 : ns;
    const float* pj = a.part + size_t(j) * a.nsplit * G * D;
    const float* mlj = a.part + size_t(a.nkv) * a.nsplit * G * D + size_t(j) * a.nsplit * G * 2;
    // this combiner's slice of the float4 outputs; `parts` threads share an
    // output, each summing every parts-th split, then meet in LDS. The first
    // kPre splits of each thread are requested before the (m, l) pass, so
    // both round trips overlap.
    constexpr int NV = G * D / 4;
    constexpr int kPre = 8;
    const int f0 = w * NV / ncomb, f1 = (w + 1) * NV / ncomb;
    const int len = f1 - f0;
    const int parts = kBlock / len;
    const int fi = threadIdx.x % len, part = threadIdx.x / len;
    const bool active = part < parts;
    const int f = f0 + fi;
    float4 pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int t = part + k * parts;
      pre[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (active && t < nsum) {
        const float* pv = pj + size_t(t) * G * D + f * 4;
        const float2 lo = load_pair_agent(pv), hi = load_pair_agent(pv + 2);
        pre[k] = make_float4(lo.x, lo.y, hi.x, hi.y);
      }
    }
    // per (split, head): weight exp2(m - M) and the denominator sum of weight * l,
    // read with agent-scope loads (the partials of other workgroups)
    float* wts = sh.wts;   // [kSplitMax][G]
    float* den = sh.den;   // [G]
    for (int hh = wv; hh < G; hh += kWaves) {
      float2 ml[kSplitMax / kWave];
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < kSplitMax / kWave; ++k) {
        const int t = lane + k * kWave;
        ml[k] = t < nsum ? load_pair_agent(mlj + (t * G + hh) * 2) : make_float2(-INFINITY, 0.0f);
        M = fmaxf(M, ml[k].x);
      }
      M = wave_max(M);
      float dsum = 0.0f;
#pragma unroll
      for (int k = 0; k < kSplitMax / kWave; ++k) {
        const int t = lane + k * kWave;
        if (t < nsum) {
          const float wt = exp2f(ml[k].x - M);
          wts[t * G + hh] = wt;
          dsum = fmaf(wt, ml[k].y, dsum);
        }
      }
      dsum = wave_sum(dsum);
      if (lane == 0) den[hh] = dsum;
    }
    __syncthreads();
    float4* accs = sh.accs;   // [kBlock]
    if (active) {
      const int hh = (f * 4) / D;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < kPre; ++k) {
        const int t = part + k * parts;
        const float wt = t < nsum ? wts[t * G + hh] : 0.0f;
        acc.x = fmaf(pre[k].x, wt, acc.x); acc.y = fmaf(pre[k].y, wt, acc.y);
        acc.z = fmaf(pre[k].z, wt, acc.z); acc.w = fmaf(pre[k].w, wt, acc.w);
      }
      for (int t = part + kPre * parts; t < nsum; t += parts) {
        const float* pv = pj + size_t(t) * G * D + f * 4;
        const float2 lo = load_pair_agent(pv), hi = load_pair_agent(pv + 2);
        const float wt = wts[t * G + hh];
        acc.x = fmaf(lo.x, wt, acc.x); acc.y = fmaf(lo.y, wt, acc.y);
        acc.z = fmaf(hi.x, wt, acc.z); acc.w = fmaf(hi.y, wt, acc.w);
      }
      accs[part * len + fi] = acc;
    }
    __syncthreads();
    if (threadIdx.x < len) {
      const int f = f0 + threadIdx.x;
      const int hh = (f * 4) / D;
      float4 acc = accs[threadIdx.x];
      for (int p = 1; p < parts; ++p) {
        const float4 v = accs[p * len + threadIdx.x];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      const float r = 1.0f / den[hh];
      reinterpret_cast<float4*>(a.out + j * G * D)[f] = make_float4(acc.x * r, acc.y * r, acc.z * r, acc.w * r);
    }
  }
  if (threadIdx.x == 0) {
    if (__hip_atomic_fetch_add(cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == unsigned(ncomb - 1)) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}


}  // namespace dec
