// Split-K decode attention with a softmax per wave.
//
// Grid: n_kv * nsplit workgroups of NW waves, split-major, about one per
// compute unit. Row r of a split's chunk belongs to wave (r / RPW) % NW at
// step r / (RPW NW); a wave requests the queries, every key row of its
// steps, then every value row, all at launch, so the whole chunk is in
// flight at once and nothing waits for anything but its own rows. Each wave
// then works alone on its rows: scores (log2 units), its own maximum m_w,
// p = exp2(s - m_w), l_w = sum p and o_w = sum p v, all in registers (no
// scores or values in LDS, no barrier between the keys and the values).
// The waves meet once: with M = max_w m_w, wave w's output and sum are
// scaled by exp2(m_w - M), the same log-sum-exp rescale the splits get in
// the combine, and the split's (M, l, o) go to attn_finish.
//
// "RDNA4 Decode Kernel Fusion...", section "Where fusion stops": attention
// is the step that reads the cache and stays a kernel of its own; the split
// along positions and the rescale of partial softmaxes are the standard
// flash-decoding reduction (the combine in dec_attn_common.h).
#include "dec_attn_common.h"

namespace dec {

template <int D, int KVT>
struct LocalShape {
  static constexpr int EB = KVT == 1 ? 2 : 4;   // bytes per cache element
  static constexpr int RB = D * EB;             // bytes per cache row
  static constexpr int DPL = 16 / EB;           // dims per lane (16 bytes)
  static constexpr int LPR = D / DPL;           // lanes per row
  static constexpr int RPW = kWave / LPR;       // rows per wave load
};

// max over the lanes l, l ^ S, l ^ 2S, ... (S = 8, 16 or 32): every lane
// receives the same value
template <int S>
__device__ __forceinline__ float fold_max(float v) {
  static_assert(S == 8 || S == 16 || S == 32, "group width");
  if constexpr (S <= 8) v = fmaxf(v, dpp_mov<0x128>(v));
  if constexpr (S <= 16) v = pair_max<16>(v);
  return pair_max<32>(v);
}

template <int D, int KVT, int G, int NW, int S>
__global__ __launch_bounds__(NW * 64) void attn_local_kernel(AttnArgs a) {
  using Sh = LocalShape<D, KVT>;
  constexpr int RB = Sh::RB, DPL = Sh::DPL, LPR = Sh::LPR, RPW = Sh::RPW;
  constexpr int RPS = RPW * NW;   // rows per step of the workgroup
  static_assert(LPR >= 8 && LPR <= 32, "row layout");

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
  const int n = min(t0 + a.chunk, L) - t0;   // 1 <= n <= chunk <= S * RPS

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int sub = lane / LPR;
  const int li = lane % LPR;
  const int d0 = li * DPL;
  const size_t base = (size_t(j) * a.max_ctx + t0) * RB + li * 16;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.kc) + base;
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.vc) + base;
  auto row = [&](int u) { return u * RPS + wv * RPW + sub; };

  // ---- the kv head's queries (a few 16-byte loads per lane), every key
  // row of this wave, then every value row. Loads complete in order, so
  // the queries arrive first, each key row can be scored as it arrives and
  // each value row summed as it arrives. The queries go through this
  // wave's slice of LDS (the slice its output takes later): with every lane
  // requesting its own slice of every head's query, a workgroup asked for
  // the kv head's queries 32 times over (four heads of 128, eight waves).
  constexpr int NQ4 = G * D / 4;                  // float4s of the kv head's queries
  constexpr int QPL = (NQ4 + kWave - 1) / kWave;  // per lane
  float4 qraw[QPL];
#pragma unroll
  for (int i = 0; i < QPL; ++i) {
    const int idx = lane + i * kWave < NQ4 ? lane + i * kWave : NQ4 - 1;
    qraw[i] = *reinterpret_cast<const float4*>(a.q + size_t(j) * G * D + idx * 4);
  }
  // Every load is issued (a row past the chunk reads the chunk's last row
  // again, and its score is -inf): predicated loads became branches, and
  // the compiler then waited for all loads in flight at each one.
  auto rclamp = [&](int u) { const int r = row(u); return size_t(r < n ? r : n - 1) * RB; };
  u32x4 kv[S], vv[S];
#pragma unroll
  for (int u = 0; u < S; ++u) kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + rclamp(u)));
#pragma unroll
  for (int u = 0; u < S; ++u) vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + rclamp(u)));
  // keep every request here, at launch (the scheduler otherwise moved the
  // value loads after the scores, so the values were requested only once
  // all keys had arrived)
  __builtin_amdgcn_sched_barrier(0);

  __shared__ float ored[NW][G][D];   // this wave's queries, later its output
  const float qscale = kLog2e / sqrtf(float(D));
  float* qs = &ored[wv][0][0];
#pragma unroll
  for (int i = 0; i < QPL; ++i) {
    const int idx = lane + i * kWave;
    if (idx < NQ4) {
      const float4 x = qraw[i];
      *reinterpret_cast<float4*>(qs + idx * 4) = make_float4(x.x * qscale, x.y * qscale, x.z * qscale, x.w * qscale);
    }
  }
  float qv[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(qs + hh * D + d0 + e);
      qv[hh][e] = x.x; qv[hh][e + 1] = x.y; qv[hh][e + 2] = x.z; qv[hh][e + 3] = x.w;
    }

  // ---- scores s = (q . k) log2(e) / sqrt(d); rows past the chunk score -inf
  float p[G][S];
#pragma unroll
  for (int u = 0; u < S; ++u) {
    float kf[DPL];
    unpack_row<KVT>(kv[u], kf);
    const bool ok = row(u) < n;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) d = fmaf(qv[hh][e], kf[e], d);
      d = group_sum<LPR>(d);
      p[hh][u] = ok ? d : -INFINITY;
    }
  }
  // ---- this wave's softmax: m_w, p = exp2(s - m_w), l_w (a wave with no
  // rows has m_w = -inf and contributes nothing)
  float mw[G], lw[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float m = p[hh][0];
#pragma unroll
    for (int u = 1; u < S; ++u) m = fmaxf(m, p[hh][u]);
    m = fold_max<LPR>(m);
    const float ms = m == -INFINITY ? 0.0f : m;
    float l = 0.0f;
#pragma unroll
    for (int u = 0; u < S; ++u) {
      p[hh][u] = exp2f(p[hh][u] - ms);
      l += p[hh][u];
    }
    mw[hh] = m;
    lw[hh] = fold_groups<LPR>(l);
  }
  // ---- o_w = sum p v over this wave's rows
  float o[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[hh][e] = 0.0f;
#pragma unroll
  for (int u = 0; u < S; ++u) {
    float vf[DPL];
    unpack_row<KVT>(vv[u], vf);
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[hh][e] = fmaf(p[hh][u], vf[e], o[hh][e]);
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[hh][e] = fold_groups<LPR>(o[hh][e]);

  // ---- the waves meet: M = max_w m_w, wave w scaled by exp2(m_w - M)
  __shared__ float wml[NW][G][2];
  __shared__ float stat[G][2];
  __shared__ int role;
  __shared__ float cwts[kSplitMax][G];
  __shared__ float cden[G];
  __shared__ float4 caccs[NW * 64];
  if (lane == 0)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) { wml[wv][hh][0] = mw[hh]; wml[wv][hh][1] = lw[hh]; }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float M = wml[0][hh][0];   // wave 0 holds row 0: finite
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, wml[w][hh][0]);
    const float c = mw[hh] == -INFINITY ? 0.0f : exp2f(mw[hh] - M);
    if (sub == 0)
#pragma unroll
      for (int e = 0; e < DPL; ++e) ored[wv][hh][d0 + e] = o[hh][e] * c;
    if (tid == hh) {
      float l = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float m = wml[w][hh][0];
        if (m != -INFINITY) l = fmaf(exp2f(m - M), wml[w][hh][1], l);
      }
      stat[hh][0] = M;
      stat[hh][1] = l;
    }
  }
  __syncthreads();

  attn_finish<D, G, NW>(a, j, s, ns, AttnShared{&ored[0][0][0], &stat[0][0], &cwts[0][0], cden, caccs, &role});
}

template <int D, int KVT, int NW, int S>
static hipError_t go_local_g(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.nkv * a.nsplit), block(NW * 64);
  switch (a.nq / a.nkv) {
    case 1: hipLaunchKernelGGL((attn_local_kernel<D, KVT, 1, NW, S>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_local_kernel<D, KVT, 2, NW, S>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_local_kernel<D, KVT, 4, NW, S>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_local_kernel<D, KVT, 8, NW, S>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// rows per workgroup step for a shape
static int local_rps(int head_dim, int kvtype) {
  const int lpr = head_dim * (kvtype == 1 ? 2 : 4) / 16;
  return (kWave / lpr) * kLocalWaves;
}

int attn_local_max_chunk(int head_dim, int kvtype) {
  return kLocalMaxSteps * local_rps(head_dim, kvtype);
}

template <int D>
static hipError_t go_local(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = kLocalWaves;
  const int steps = (a.chunk + local_rps(D, 1) - 1) / local_rps(D, 1);
  if (steps <= 1) return go_local_g<D, 1, NW, 1>(a, s);
  if (steps <= 2) return go_local_g<D, 1, NW, 2>(a, s);
  if (steps <= 3) return go_local_g<D, 1, NW, 3>(a, s);
  if (steps <= 5) return go_local_g<D, 1, NW, 5>(a, s);
  if (steps <= 9) return go_local_g<D, 1, NW, 9>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_local(const AttnArgs& a, hipStream_t s) {
  static_assert(kLocalMaxSteps == 9, "instantiated step counts");
  if (a.nsplit > kSplitMax || a.kvtype != 1 || a.chunk < 1 || a.chunk > attn_local_max_chunk(a.d, a.kvtype))
    return hipErrorInvalidValue;
  if (a.d == 64) return go_local<64>(a, s);
  if (a.d == 128) return go_local<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dec
