// Split-K decode attention over the KV cache (one token, batch 1).
//
// Grid: n_kv * nsplit workgroups, split-major (block b serves kv head
// b % n_kv and split b / n_kv), so the splits that hold cache positions come
// first and the ones past the current position exit at once. A workgroup
// streams its chunk of K once to score all query heads of its kv head, turns
// the scores into exp(s - m) in LDS, streams the same chunk of V once, and
// writes (m, l, o) partials. The last workgroup of a kv head to arrive
// (device-scope counter) combines the partials with a log-sum-exp rescale and
// resets the counter, so the kernel replays unchanged inside a graph.
#include "dec_device.h"
#include "dec_internal.h"

namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkMax = 256;  // cache positions per split
constexpr int kSplitMax = 256;  // splits per kv head

template <int KVT>
__device__ __forceinline__ void unpack_row(u32x4 v, float* f) {
  if constexpr (KVT == 1) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

template <int D, int KVT, int G>
__global__ __launch_bounds__(kBlock) void attn_kernel(AttnArgs a) {
  constexpr int EB = KVT == 1 ? 2 : 4;  // bytes per cache element
  constexpr int DPL = 16 / EB;          // dims per lane
  constexpr int LPR = D / DPL;          // lanes per cache row
  constexpr int RPW = kWave / LPR;      // rows per wave load
  constexpr int RPS = RPW * kWaves;     // rows per workgroup step
  constexpr int U = 4;                  // row steps in flight
  static_assert(LPR >= 2 && LPR <= 32, "row layout");

  if (a.null_kernel) return;
  const int j = blockIdx.x % a.nkv;
  const int s = blockIdx.x / a.nkv;
  const int pos = *a.pos;
  if (pos < 0 || pos >= a.max_ctx) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.err, kErrPos);
    return;
  }
  const int L = pos + 1;
  const int ns = (L + a.chunk - 1) / a.chunk;
  if (s >= ns) return;
  const int t0 = s * a.chunk;
  const int t1 = min(t0 + a.chunk, L);
  const int n = t1 - t0;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane / LPR;
  const int li = lane % LPR;
  const int d0 = li * DPL;
  const float scale = 1.0f / sqrtf(float(D));

  __shared__ float sc[G][kChunkMax];
  __shared__ float stat[G][2];
  __shared__ float ored[kWaves][G][D];
  __shared__ int last;

  float qv[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[hh][e] = a.q[(j * G + hh) * D + d0 + e] * scale;

  const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.kc) + size_t(j) * a.max_ctx * D * EB;
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.vc) + size_t(j) * a.max_ctx * D * EB;
  const int nsteps = (n + RPS - 1) / RPS;

  // ---- scores: s_t = (q . k_t) / sqrt(d) for every query head of the group
  for (int it = 0; it < nsteps; it += U) {
    u32x4 kv[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int t = t0 + (it + uu) * RPS + wv * RPW + sub;
      const bool ok = (it + uu < nsteps) && t < t1;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kv[uu] = ok ? *reinterpret_cast<const u32x4*>(kb + (size_t(t) * D + d0) * EB) : z;
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int t = t0 + (it + uu) * RPS + wv * RPW + sub;
      const bool ok = (it + uu < nsteps) && t < t1;
      float kf[DPL];
      unpack_row<KVT>(kv[uu], kf);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float p = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) p = fmaf(qv[hh][e], kf[e], p);
        p = group_sum<LPR>(p);
        if (ok && li == 0) sc[hh][t - t0] = p;
      }
    }
  }
  __syncthreads();

  // ---- per-head max and sum of exp over the chunk
  for (int hh = wv; hh < G; hh += kWaves) {
    float m = -INFINITY;
    for (int i = lane; i < n; i += kWave) m = fmaxf(m, sc[hh][i]);
    m = wave_max(m);
    float l = 0.0f;
    for (int i = lane; i < n; i += kWave) {
      const float p = expf(sc[hh][i] - m);
      sc[hh][i] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) { stat[hh][0] = m; stat[hh][1] = l; }
  }
  __syncthreads();

  // ---- o = sum_t p_t v_t
  float o[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[hh][e] = 0.0f;
  for (int it = 0; it < nsteps; it += U) {
    u32x4 vv[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int t = t0 + (it + uu) * RPS + wv * RPW + sub;
      const bool ok = (it + uu < nsteps) && t < t1;
      const u32x4 z = {0u, 0u, 0u, 0u};
      vv[uu] = ok ? *reinterpret_cast<const u32x4*>(vb + (size_t(t) * D + d0) * EB) : z;
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int t = t0 + (it + uu) * RPS + wv * RPW + sub;
      const bool ok = (it + uu < nsteps) && t < t1;
      if (ok) {
        float vf[DPL];
        unpack_row<KVT>(vv[uu], vf);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = sc[hh][t - t0];
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[hh][e] = fmaf(p, vf[e], o[hh][e]);
        }
      }
    }
  }
  // rows of one wave load sit LPR lanes apart: fold them
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[hh][e] += __shfl_xor(o[hh][e], off);
  if (sub == 0)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; ++e) ored[wv][hh][d0 + e] = o[hh][e];
  __syncthreads();

  // ---- partials (m, l, o) of this split
  constexpr int PS = D + 2;
  float* pp = a.part + (size_t(j) * a.nsplit + s) * G * PS;
  for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
    const int hh = idx / D, dd = idx % D;
    pp[hh * PS + dd] = ((ored[0][hh][dd] + ored[1][hh][dd]) + ored[2][hh][dd]) + ored[3][hh][dd];
  }
  if (threadIdx.x < G) {
    pp[threadIdx.x * PS + D] = stat[threadIdx.x][0];
    pp[threadIdx.x * PS + D + 1] = stat[threadIdx.x][1];
  }

  // ---- arrival: the last split of this kv head combines
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&a.counters[j], 1u);
    last = (prev == unsigned(ns - 1));
  }
  __syncthreads();
  if (!last) return;
  __threadfence();

  __shared__ float wts[kSplitMax][G];
  __shared__ float den[G];
  const float* pj = a.part + size_t(j) * a.nsplit * G * PS;
  for (int hh = wv; hh < G; hh += kWaves) {
    float M = -INFINITY;
    for (int t = lane; t < ns; t += kWave) M = fmaxf(M, pj[(size_t(t) * G + hh) * PS + D]);
    M = wave_max(M);
    float dsum = 0.0f;
    for (int t = lane; t < ns; t += kWave) {
      const float* e = pj + (size_t(t) * G + hh) * PS;
      const float w = expf(e[D] - M);
      wts[t][hh] = w;
      dsum = fmaf(w, e[D + 1], dsum);
    }
    dsum = wave_sum(dsum);
    if (lane == 0) den[hh] = dsum;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
    const int hh = idx / D, dd = idx % D;
    const float* e = pj + hh * PS + dd;
    float acc = 0.0f;
    int t = 0;
    for (; t + 8 <= ns; t += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = e[size_t(t + k) * G * PS];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc = fmaf(v[k], wts[t + k][hh], acc);
    }
    for (; t < ns; ++t) acc = fmaf(e[size_t(t) * G * PS], wts[t][hh], acc);
    a.out[(j * G + hh) * D + dd] = acc / den[hh];
  }
  if (threadIdx.x == 0) atomicExch(&a.counters[j], 0u);
}

void attn_plan(int n_kv, int max_ctx, int chunk_req, int* chunk, int* nsplit) {
  int c = chunk_req;
  if (c <= 0) {
    // aim at about 768 workgroups over the whole cache
    const long target = 768;
    c = int((long(max_ctx) * n_kv + target - 1) / target);
    c = ((c + 15) / 16) * 16;
  }
  const int cmin = (max_ctx + kSplitMax - 1) / kSplitMax;
  if (c < cmin) c = cmin;
  if (c < 16) c = 16;
  if (c > kChunkMax) c = kChunkMax;
  *chunk = c;
  *nsplit = (max_ctx + c - 1) / c;
}

template <int D, int KVT>
static hipError_t go_attn(const AttnArgs& a, hipStream_t s) {
  const int g = a.nq / a.nkv;
  const dim3 grid(a.nkv * a.nsplit), block(kBlock);
  switch (g) {
    case 1: hipLaunchKernelGGL((attn_kernel<D, KVT, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<D, KVT, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_kernel<D, KVT, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_kernel<D, KVT, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  if (a.nsplit > kSplitMax || a.chunk > kChunkMax) return hipErrorInvalidValue;
  if (a.d == 64) return a.kvtype == 1 ? go_attn<64, 1>(a, s) : go_attn<64, 0>(a, s);
  if (a.d == 128) return a.kvtype == 1 ? go_attn<128, 1>(a, s) : go_attn<128, 0>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dec
