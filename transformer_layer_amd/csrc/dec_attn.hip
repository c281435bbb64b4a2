// Split-K decode attention over the KV cache (one token, batch 1).
//
// Grid: n_kv * nsplit workgroups, split-major (block b serves kv head
// b % n_kv and split b / n_kv), so the splits that hold cache positions come
// first and the ones past the current position exit at once. A workgroup
// reads its chunk of K once to score every query head of its kv head (scores
// kept in LDS, in log2 units), turns them into exp2(s - m) with one
// exponential per (head, position), reads the same chunk of V once, and
// writes the split's partials: o (unnormalized) and (m, l). When a
// workgroup has several row steps, its first batch of V rows is requested
// once the scores are done (VLATE): with every workgroup's K and V requests
// in the memory queues together, K arrived later (measured: 0.9 µs on the
// 9B-shaped bf16 layer, 2.6 µs at 8192 positions), while V now streams
// during the softmax. With a single row step the scores are too short to
// cover V's latency, and V is requested right after K.
//
// The last workgroups of a kv head to arrive (one per ~8 KB of partials, at
// most kCombiners) combine its partials with a log-sum-exp rescale, each a
// slice of the head group's outputs (one workgroup alone fetches the partials
// too slowly). Ordering without an L2
// write-back: the partials are written with agent-scope atomic stores, which
// reach the device-coherent level by themselves; every lane waits until its
// stores have completed (vmcnt 0), the workgroup meets at a barrier, and one
// thread increments the head's arrival counter with an agent-scope atomic.
// Combiners that arrive before the last one poll that counter (bounded: on
// giving up they set DEC_ERR_SYNC and write nothing) and read the partials
// with agent-scope loads. Every counter line is 64 bytes, so the heads'
// arrivals do not queue on one line; the last combiner to finish resets the
// line, so the kernel replays unchanged inside a graph.
#include "dec_device.h"
#include "dec_internal.h"

namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkMax = 256;  // cache positions per split
constexpr int kSplitMax = 256;  // splits per kv head
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCombiners = 8;          // workgroups that combine one kv head's splits
constexpr unsigned kSpinMax = 1u << 14;  // polls of a waiting combiner before it gives up
constexpr int kNotCombiner = -1, kGaveUp = -2;   // workgroup roles after arrival (else the combiner slot)

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

// Two floats as one agent-scope atomic store (8-byte aligned address).
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

template <int D, int KVT, int G, int NW, bool VLATE>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  constexpr int kWaves = NW;        // waves per workgroup (4 or 8)
  constexpr int kBlock = NW * 64;
  constexpr int EB = KVT == 1 ? 2 : 4;  // bytes per cache element
  constexpr int DPL = 16 / EB;          // dims per lane
  constexpr int LPR = D / DPL;          // lanes per cache row
  constexpr int RPW = kWave / LPR;      // rows per wave load
  constexpr int RPS = RPW * kWaves;     // rows per workgroup step
  constexpr int U = 8;                  // row steps in flight per batch
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
  const int nsteps = (n + RPS - 1) / RPS;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane / LPR;
  const int li = lane % LPR;
  const int d0 = li * DPL;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.kc) + size_t(j) * a.max_ctx * D * EB;
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.vc) + size_t(j) * a.max_ctx * D * EB;
  const u32x4 z = {0u, 0u, 0u, 0u};
  auto row = [&](int step) { return t0 + step * RPS + wv * RPW + sub; };

  // first batch of K rows, of V rows (VLATE: once the scores are done),
  // then the queries
  u32x4 kv[U], vv[U];
  auto first_v = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = row(u);
      const bool ok = u < nsteps && t < t1;
      vv[u] = ok ? *reinterpret_cast<const u32x4*>(vb + (size_t(t) * D + d0) * EB) : z;
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = row(u);
    const bool ok = u < nsteps && t < t1;
    kv[u] = ok ? *reinterpret_cast<const u32x4*>(kb + (size_t(t) * D + d0) * EB) : z;
  }
  if constexpr (!VLATE) first_v();
  const float qscale = kLog2e / sqrtf(float(D));
  float qv[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(a.q + (j * G + hh) * D + d0 + e);
      qv[hh][e] = x.x * qscale; qv[hh][e + 1] = x.y * qscale;
      qv[hh][e + 2] = x.z * qscale; qv[hh][e + 3] = x.w * qscale;
    }

  __shared__ float sc[G][kChunkMax];
  __shared__ float stat[G][2];
  __shared__ float ored[kWaves][G][D];
  __shared__ int role;

  // ---- scores (log2 units): s_t = (q . k_t) log2(e) / sqrt(d)
  for (int b = 0; b < nsteps; b += U) {
    if (b > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = row(b + u);
        const bool ok = b + u < nsteps && t < t1;
        kv[u] = ok ? *reinterpret_cast<const u32x4*>(kb + (size_t(t) * D + d0) * EB) : z;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = row(b + u);
      const bool ok = b + u < nsteps && t < t1;
      float kf[DPL];
      unpack_row<KVT>(kv[u], kf);
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
  if constexpr (VLATE) first_v();
  __syncthreads();

  // ---- per head: m = max s, p = exp2(s - m), l = sum p (one exponential per entry)
  for (int hh = wv; hh < G; hh += kWaves) {
    float m = -INFINITY;
    for (int i = lane; i < n; i += kWave) m = fmaxf(m, sc[hh][i]);
    m = wave_max(m);
    float l = 0.0f;
    for (int i = lane; i < n; i += kWave) {
      const float p = exp2f(sc[hh][i] - m);
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
  for (int b = 0; b < nsteps; b += U) {
    if (b > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = row(b + u);
        const bool ok = b + u < nsteps && t < t1;
        vv[u] = ok ? *reinterpret_cast<const u32x4*>(vb + (size_t(t) * D + d0) * EB) : z;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = row(b + u);
      if (b + u < nsteps && t < t1) {
        float vf[DPL];
        unpack_row<KVT>(vv[u], vf);
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
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[hh][e] = fold_groups<LPR>(o[hh][e]);
  if (sub == 0)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; ++e) ored[wv][hh][d0 + e] = o[hh][e];
  __syncthreads();

  // ---- this split's partials: o [j][s][G][D] and (m, l) [j][s][G][2], as
  // agent-scope 64-bit atomic stores (pairs of floats)
  float* po = a.part + (size_t(j) * a.nsplit + s) * G * D;
  float* pml = a.part + size_t(a.nkv) * a.nsplit * G * D + (size_t(j) * a.nsplit + s) * G * 2;
  auto osum = [&](int idx) {
    const int hh = idx / D, dd = idx % D;
    float r = ored[0][hh][dd];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r += ored[w][hh][dd];
    return r;
  };
  for (int i2 = threadIdx.x; i2 < G * D / 2; i2 += kBlock) store_pair_agent(po + 2 * i2, osum(2 * i2), osum(2 * i2 + 1));
  if (threadIdx.x < G) store_pair_agent(pml + threadIdx.x * 2, stat[threadIdx.x][0], stat[threadIdx.x][1]);

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
    role = slot < 0 ? kNotCombiner : gave_up ? kGaveUp : slot;
  }
  __syncthreads();
  const int w = role;
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
    __shared__ float wts[kSplitMax][G];
    __shared__ float den[G];
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
          wts[t][hh] = wt;
          dsum = fmaf(wt, ml[k].y, dsum);
        }
      }
      dsum = wave_sum(dsum);
      if (lane == 0) den[hh] = dsum;
    }
    __syncthreads();
    __shared__ float4 accs[kBlock];
    if (active) {
      const int hh = (f * 4) / D;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < kPre; ++k) {
        const int t = part + k * parts;
        const float wt = t < nsum ? wts[t][hh] : 0.0f;
        acc.x = fmaf(pre[k].x, wt, acc.x); acc.y = fmaf(pre[k].y, wt, acc.y);
        acc.z = fmaf(pre[k].z, wt, acc.z); acc.w = fmaf(pre[k].w, wt, acc.w);
      }
      for (int t = part + kPre * parts; t < nsum; t += parts) {
        const float* pv = pj + size_t(t) * G * D + f * 4;
        const float2 lo = load_pair_agent(pv), hi = load_pair_agent(pv + 2);
        const float wt = wts[t][hh];
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

void attn_plan(int n_q, int n_kv, int head_dim, int kvtype, int max_ctx, int chunk_req, int* chunk, int* nsplit,
               int* waves) {
  int c = chunk_req;
  int nw = 4;
  if (c <= 0) {
    // about one workgroup per compute unit over the whole cache (at most
    // 64 splits per kv head), chunks a multiple of 16 rows and no longer
    // than one batch of rows in flight
    const int lanes_per_row = head_dim * (kvtype == 1 ? 2 : 4) / 16;
    const int one_batch = (kWave / lanes_per_row) * 4 * 8;
    int splits = 256 / n_kv;
    if (splits > 64) splits = 64;
    if (splits < 1) splits = 1;
    c = (max_ctx + splits - 1) / splits;
    c = ((c + 15) / 16) * 16;
    if (c > one_batch) c = one_batch;
    // bf16 head_dim 128: at most 96 rows, three quarters of a batch (more
    // splits, shorter chains per workgroup; measured against 128: 9B-shaped
    // layer at 8320 positions 16.6 -> 16.0 us, 7B-shaped at 2112 positions
    // 12.3 -> 11.95 us)
    if (head_dim == 128 && kvtype == 1 && c > 96) c = 96;
    // bf16 head_dim 128 with four or more query heads per kv head and up to
    // 4608 positions (measured on the 9B-shaped layer): 192-row chunks over
    // 8 waves, one batch per wave and fewer splits to combine
    if (head_dim == 128 && kvtype == 1 && n_q >= 4 * n_kv && max_ctx <= 4608) {
      nw = 8;
      c = 192;
    }
  }
  const int cmin = (max_ctx + kSplitMax - 1) / kSplitMax;
  if (c < cmin) c = cmin;
  if (c < 16) c = 16;
  if (c > kChunkMax) c = kChunkMax;
  *chunk = c;
  *nsplit = (max_ctx + c - 1) / c;
  *waves = nw;
}

template <int D, int KVT, int NW, bool VL>
static hipError_t go_attn(const AttnArgs& a, hipStream_t s) {
  const int g = a.nq / a.nkv;
  const dim3 grid(a.nkv * a.nsplit), block(NW * 64);
  switch (g) {
    case 1: hipLaunchKernelGGL((attn_kernel<D, KVT, 1, NW, VL>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<D, KVT, 2, NW, VL>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_kernel<D, KVT, 4, NW, VL>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_kernel<D, KVT, 8, NW, VL>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// V requested after the scores when a workgroup has more than one row step
// (rows per step: 64 / lanes-per-row rows per wave, times the waves)
template <int D, int KVT, int NW>
static hipError_t go_attn_vl(const AttnArgs& a, hipStream_t s) {
  constexpr int rows_per_step = (kWave / (D * (KVT == 1 ? 2 : 4) / 16)) * NW;
  return a.chunk > rows_per_step ? go_attn<D, KVT, NW, true>(a, s) : go_attn<D, KVT, NW, false>(a, s);
}

template <int D, int KVT>
static hipError_t go_attn_waves(const AttnArgs& a, hipStream_t s) {
  if (a.waves == 8) return go_attn_vl<D, KVT, 8>(a, s);
  if (a.waves == 4) return go_attn_vl<D, KVT, 4>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  if (a.nsplit > kSplitMax || a.chunk > kChunkMax) return hipErrorInvalidValue;
  if (a.d == 64) return a.kvtype == 1 ? go_attn_waves<64, 1>(a, s) : go_attn_waves<64, 0>(a, s);
  if (a.d == 128) return a.kvtype == 1 ? go_attn_waves<128, 1>(a, s) : go_attn_waves<128, 0>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dec
