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
// An int8 cache (KVT 2) keeps one float scale per row: the score of a row is
// its code dot product times the key row's scale, and its weight in p.v is
// p times the value row's scale. Each lane loads the scales of its rows of
// the softmax pass (t0 + lane + 64 k) once at launch, and the softmax pass
// applies them: the row loops read codes only. The token's own row is not
// read from the cache: the split that holds position p stops its loops one
// row short, and its wave 0 (which requests the staged float k and v rows at
// launch) quantizes them (one scale per row: max |x| / 127; codes
// x * (127 / max |x|) rounded half to even, all in float32), stores codes and
// scales into slot p, and scores and sums the token from those codes.
//
// A bf16 cache with at most four query heads per kv head scores on the
// matrix cores (v_mfma_f32_16x16x32_bf16): a 16-row tile of K is the A
// operand as stored (lane l: row l % 16, dims 32 ks + 8 (l / 16) .. + 7 for
// step ks), and the B operand's columns hold each query head three times, as
// three bf16 parts hi + mid + lo of q scaled (column p G + h: part p of head
// h; the other columns zero). A bf16 x bf16 product is exact in float32 and
// the three parts keep every bit of q's float32 significand, so a row's
// score is the float32 dot product up to the order of its additions; two DPP
// adds sum the three columns of a head. On the vector ALUs each 16 rows cost
// about 250 instructions a wave (unpacking, products, lane folds), here 4
// matrix operations and about 10 instructions. An int8 cache does the same
// with v_mfma_i32_16x16x64_i8: the codes as stored, and each query head as
// 22-bit integers in three int8 digits (query_digits_i8), whose exact
// integer sums combine in float32 and scale by 2^-E; its tile stores leave
// out the token's own row, which wave 0 scores.
//
// Partials, arrival and combine: attn_finish (dec_attn_common.h).
#include "dec_attn_common.h"

namespace dec {

template <int D, int KVT, int G, int NW, bool VLATE>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  constexpr int kWaves = NW;        // waves per workgroup (4 or 8)
  constexpr int kBlock = NW * 64;
  constexpr int EB = KVT == 1 ? 2 : KVT == 2 ? 1 : 4;  // bytes per cache element
  constexpr bool I8 = KVT == 2;
  constexpr int DPL = 16 / EB;          // dims per lane
  constexpr int LPR = D / DPL;          // lanes per cache row
  constexpr int RPW = kWave / LPR;      // rows per wave load
  constexpr int RPS = RPW * kWaves;     // rows per workgroup step
  constexpr int U = 8;                  // row steps in flight per batch
  static_assert(LPR >= 2 && LPR <= 32, "row layout");
  // scores on the matrix cores: bf16 caches (three bf16 parts of q) and
  // int8 caches (three int8 digits of q)
  constexpr bool MSB = KVT == 1 && 3 * G <= 16 && D % 32 == 0;
  constexpr bool MSI = KVT == 2 && 3 * G <= 16 && D == 128;
  constexpr bool MS = MSB || MSI;
  constexpr int KPS = MSI ? 64 : 32;     // dims per matrix step
  constexpr int KSTEPS = D / KPS;        // matrix steps per 16-row tile
  constexpr int UT = KSTEPS >= 4 ? 2 : 4;   // tiles in flight per wave
  constexpr int QPAIRS = 16 * D / 2;     // B operand: 16 columns of D bf16, two a word
  constexpr int QPT = (QPAIRS + kBlock - 1) / kBlock;
  // value loads in flight per lane: with matrix-core scores the wait for
  // a second batch of values is no longer hidden, so 128-wide rows keep a
  // whole default chunk (96 rows) in flight (9B-shaped 4-bit stack 500.2 ->
  // 509.7 tok/s; 64-wide rows lost 0.6% and keep 8)
  constexpr int UV = MSB && D == 128 ? 12 : U;

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
  // int8 cache: the split holding the token's position leaves that row to
  // wave 0 (below); the loops read rows t0 .. tl-1 from the cache
  const bool newrow = I8 && s == ns - 1;
  const int tl = newrow ? t1 - 1 : t1;
  const int nsteps = (tl - t0 + RPS - 1) / RPS;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane / LPR;
  const int li = lane % LPR;
  const int d0 = li * DPL;
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.kc) + size_t(j) * a.max_ctx * D * EB;
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.vc) + size_t(j) * a.max_ctx * D * EB;
  const u32x4 z = {0u, 0u, 0u, 0u};
  auto row = [&](int step) { return t0 + step * RPS + wv * RPW + sub; };
  // int8 cache: the scales of this lane's softmax rows (t0 + lane + 64 k;
  // the index is clamped into the cache rows read, the values past them are
  // never used), and wave 0 of the token's split requests the staged rows
  constexpr int KS = I8 ? kChunkMax / kWave : 1;
  const size_t scale_off = I8 ? kv_i8_scale_off(a.nkv, a.max_ctx, D) : 0;
  float rks[KS], rvs[KS];
  float2 kx = {0.0f, 0.0f}, vx = {0.0f, 0.0f};
  if constexpr (I8) {
    const float* ksc = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.kc) + scale_off) +
                       size_t(j) * a.max_ctx;
    const float* vsc = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.vc) + scale_off) +
                       size_t(j) * a.max_ctx;
    const int tmax = tl > t0 ? tl - 1 : t0;   // t0 <= pos < max_ctx
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int t = min(t0 + lane + k * kWave, tmax);
      rks[k] = ksc[t];
      rvs[k] = vsc[t];
    }
    if (newrow && wv == 0) {
      const size_t so = kv_i8_stage_off(a.nkv, a.max_ctx, D);
      kx = *reinterpret_cast<const float2*>(
          reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.kc) + so) + size_t(j) * D + 2 * lane);
      vx = *reinterpret_cast<const float2*>(
          reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.vc) + so) + size_t(j) * D + 2 * lane);
    }
  }

  // int8 and bf16 value rows are read eight bytes a lane (8 codes or 4
  // bf16 dims), so the rows of a wave load sit more lanes apart and the fold
  // of the p.v sums below takes fewer steps over fewer accumulators (int8:
  // 16 codes a lane took three steps over 64; bf16: two over 32 became one
  // over 16; 9B-shaped 4-bit stack 486.6 -> 489.8, 1B-shaped 1685 -> 1694.5
  // tok/s, same box)
  constexpr bool V8 = I8 || KVT == 1;        // value rows in 8-byte lane loads
  constexpr int VDPL8 = I8 ? 8 : 4;           // dims per 8-byte load
  constexpr int VLPR = V8 ? D / VDPL8 : LPR;  // lanes per value row
  constexpr int VRPS = (kWave / VLPR) * kWaves;  // value rows per workgroup step
  const int vsub = lane / VLPR;
  const int vd0 = (lane % VLPR) * VDPL8;      // first dim of the lane (8-byte loads)
  const int nvsteps = V8 ? (tl - t0 + VRPS - 1) / VRPS : nsteps;
  auto vrow8 = [&](int step) { return t0 + step * VRPS + wv * (kWave / VLPR) + vsub; };
  uint2 v8[V8 ? UV : 1];
  auto load_v8 = [&](int step, int u) {
    const int t = vrow8(step);
    const bool ok = step < nvsteps && t < tl;
    v8[u] = ok ? *reinterpret_cast<const uint2*>(vb + (size_t(t) * D + vd0) * EB) : make_uint2(0u, 0u);
  };

  // matrix-core scores: this thread's words of the B operand (q read
  // first, so that waiting for it does not wait for K), then the wave's
  // first tiles of K (tiles wv, wv + NW, ...; lane l reads row l % 16)
  const int nrow = tl - t0;
  const int ntile = (nrow + 15) / 16;
  const int kr = lane & 15, kg = lane >> 4;
  float2 qx[MSB ? QPT : 1];
  float2 qi = {0.0f, 0.0f};   // int8: wave wv < G holds dims 2 lane, 2 lane + 1 of head wv
  u32x4 kt[MS ? UT : 1][MS ? KSTEPS : 1];
  auto load_tiles = [&](int b) {
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      const int tile = wv + kWaves * (b + u);
      const int t = t0 + 16 * tile + kr;
      const bool ok = tile < ntile && t < tl;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        kt[u][ks] = ok ? *reinterpret_cast<const u32x4*>(kb + (size_t(t) * D + KPS * ks + KPS / 4 * kg) * EB) : z;
    }
  };
  if constexpr (MSB) {
#pragma unroll
    for (int r = 0; r < QPT; ++r) {
      const int e = threadIdx.x + r * kBlock;   // word e: column e / (D / 2), dims 2 (e % (D / 2)) + 0, 1
      const int c = e / (D / 2), dd = 2 * (e % (D / 2));
      qx[r] = e < QPAIRS && c < 3 * G ? *reinterpret_cast<const float2*>(a.q + (j * G + c % G) * D + dd)
                                      : make_float2(0.0f, 0.0f);
    }
  }
  if constexpr (MSI) {
    if (wv < G) qi = *reinterpret_cast<const float2*>(a.q + (j * G + wv) * D + 2 * lane);
  }
  if constexpr (MS) load_tiles(0);

  // first batch of K rows, of V rows (VLATE: once the scores are done),
  // then the queries
  u32x4 kv[MS ? 1 : U], vv[V8 ? 1 : U];
  auto first_v = [&]() {
    if constexpr (V8) {
#pragma unroll
      for (int u = 0; u < UV; ++u) load_v8(u, u);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = row(u);
        const bool ok = u < nsteps && t < tl;
        vv[u] = ok ? *reinterpret_cast<const u32x4*>(vb + (size_t(t) * D + d0) * EB) : z;
      }
    }
  };
  if constexpr (!MS) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = row(u);
      const bool ok = u < nsteps && t < tl;
      kv[u] = ok ? *reinterpret_cast<const u32x4*>(kb + (size_t(t) * D + d0) * EB) : z;
    }
  }
  if constexpr (!VLATE) first_v();
  const float qscale = kLog2e / sqrtf(float(D));
  float qv[MS ? 1 : G][MS ? 1 : DPL];
  if constexpr (!MS) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(a.q + (j * G + hh) * D + d0 + e);
        qv[hh][e] = x.x * qscale; qv[hh][e + 1] = x.y * qscale;
        qv[hh][e + 2] = x.z * qscale; qv[hh][e + 3] = x.w * qscale;
      }
  }

  __shared__ __align__(16) float sc[G][kChunkMax];
  __shared__ __align__(16) uint32_t qp[MS ? 16 : 1][MS ? D / 2 : 1];   // B operand, column-major words
  __shared__ int qe[MSI ? G : 1];   // int8: each head's exponent E
  __shared__ float stat[G][2];
  __shared__ float ored[kWaves][G][D];
  __shared__ int role;
  __shared__ float cwts[kSplitMax][G];
  __shared__ float cden[G];
  __shared__ float4 caccs[kBlock];

  // ---- scores (log2 units): s_t = (q . k_t) log2(e) / sqrt(d)
  if constexpr (MS) {
    if constexpr (MSB) {
#pragma unroll
      for (int r = 0; r < QPT; ++r) {
        const int e = threadIdx.x + r * kBlock;
        if (e < QPAIRS) {
          const int p = (e / (D / 2)) / G;   // 3 and above: a zero column (its q words are zero)
          qp[e / (D / 2)][e % (D / 2)] =
              q_part_bf16(qx[r].x * qscale, p) | (q_part_bf16(qx[r].y * qscale, p) << 16);
        }
      }
    } else {
      // int8: wave h < G builds head h's digit columns h, G + h, 2G + h
      // (column c holds D bytes; columns 3G and up are never read)
      if (wv < G) {
        const float x0 = qi.x * qscale, x1 = qi.y * qscale;
        const bool finite = __all(fabsf(x0) <= 3.4028235e38f && fabsf(x1) <= 3.4028235e38f);
        const int e = query_exp_i8_checked(wave_max(fmaxf(fabsf(x0), fabsf(x1))), finite);
        int a0, a1, a2, b0, b1, b2;
        query_digits_i8(x0, e, a0, a1, a2);
        query_digits_i8(x1, e, b0, b1, b2);
        uint16_t* qd = reinterpret_cast<uint16_t*>(&qp[0][0]);   // [16][D / 2] pairs of int8
        qd[(0 * G + wv) * (D / 2) + lane] = uint16_t((a0 & 255) | ((b0 & 255) << 8));
        qd[(1 * G + wv) * (D / 2) + lane] = uint16_t((a1 & 255) | ((b1 & 255) << 8));
        qd[(2 * G + wv) * (D / 2) + lane] = uint16_t((a2 & 255) | ((b2 & 255) << 8));
        if (lane == 0) qe[wv] = e;
      }
    }
    __syncthreads();
    u32x4 qb[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qb[ks] = MSB ? *reinterpret_cast<const u32x4*>(&qp[kr][16 * ks + 4 * kg])
                   : *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(&qp[0][0]) + kr * D +
                                                     64 * ks + 16 * kg);
    const int ekr = MSI ? qe[kr < G ? kr : 0] : 0;
    for (int b = 0; wv + kWaves * b < ntile; b += UT) {
      if (b > 0) load_tiles(b);
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        const int tile = wv + kWaves * (b + u);   // wave-uniform
        if (tile < ntile) {
          // lane kr < G: column kr (rows 4 kg .. 4 kg + 3 of the tile) with
          // columns kr + G and kr + 2G (DPP row shifts left by G and 2G)
          float sv[4];
          if constexpr (MSB) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kt[u][ks]),
                                                            __builtin_bit_cast(bf16x8, qb[ks]), acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sv[i] = acc[i] + dpp_mov<0x100 + G>(acc[i]) + dpp_mov<0x100 + 2 * G>(acc[i]);
          } else {
            i32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
              acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, kt[u][ks]),
                                                          __builtin_bit_cast(i32x4, qb[ks]), acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sv[i] = digit_score(acc[i], dpp_mov_i<0x100 + G>(acc[i]), dpp_mov_i<0x100 + 2 * G>(acc[i]), ekr);
          }
          if (kr < G) {
            float* dst = &sc[kr][16 * tile + 4 * kg];
            if constexpr (MSB) {
              // rows past the chunk score 0 and are never read; the index
              // stays below kChunkMax (16 ceil(n / 16) <= kChunkMax)
              *reinterpret_cast<float4*>(dst) = make_float4(sv[0], sv[1], sv[2], sv[3]);
            } else {
              // int8: only the cache rows (row nrow may be the token's, scored by wave 0)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (16 * tile + 4 * kg + i < nrow) dst[i] = sv[i];
            }
          }
        }
      }
    }
  } else
  for (int b = 0; b < nsteps; b += U) {
    if (b > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = row(b + u);
        const bool ok = b + u < nsteps && t < tl;
        kv[u] = ok ? *reinterpret_cast<const u32x4*>(kb + (size_t(t) * D + d0) * EB) : z;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = row(b + u);
      const bool ok = b + u < nsteps && t < tl;
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
  // int8 cache, the split holding the token: wave 0 quantizes the staged k
  // and v rows (two dims a lane), appends them at slot pos and scores the
  // token's row; its value codes wait in registers for the sum below
  float nv0 = 0.0f, nv1 = 0.0f, nvs = 0.0f;
  if constexpr (I8) {
    static_assert(!I8 || D == 2 * kWave, "int8 cache rows: two dims a lane");
    if (newrow && wv == 0) {
      float kc0, kc1, kscale, vc0, vc1, vscale;
      quantize_pair_i8(kx, kc0, kc1, kscale);
      quantize_pair_i8(vx, vc0, vc1, vscale);
      const size_t slot = size_t(j) * a.max_ctx + pos;
      uint8_t* kcw = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.kc));
      uint8_t* vcw = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.vc));
      *reinterpret_cast<uint16_t*>(kcw + slot * D + 2 * lane) = pack_i8_pair(kc0, kc1);
      *reinterpret_cast<uint16_t*>(vcw + slot * D + 2 * lane) = pack_i8_pair(vc0, vc1);
      if (lane == 0) {
        *reinterpret_cast<float*>(kcw + scale_off + slot * 4) = kscale;
        *reinterpret_cast<float*>(vcw + scale_off + slot * 4) = vscale;
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float2 qx = *reinterpret_cast<const float2*>(a.q + (j * G + hh) * D + 2 * lane);
        float d = wave_sum(fmaf(qx.x, kc0, qx.y * kc1));
        if (lane == 0) sc[hh][n - 1] = d * kscale * qscale;
      }
      nv0 = vc0;
      nv1 = vc1;
      nvs = vscale;
    }
  }
  if constexpr (VLATE) first_v();
  __syncthreads();

  // ---- per head: m = max s, p = exp2(s - m), l = sum p (one exponential per
  // entry); an int8 cache's row scales enter here: s = the code score times
  // the key scale, and the PV loop reads p times the value scale (the
  // token's row, already scaled, keeps factor 1)
  for (int hh = wv; hh < G; hh += kWaves) {
    float m = -INFINITY;
    if constexpr (I8) {
      const int nc = tl - t0;   // rows read from the cache
      float sv[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int i = lane + k * kWave;
        sv[k] = i < n ? sc[hh][i] * (i < nc ? rks[k] : 1.0f) : -INFINITY;
        m = fmaxf(m, sv[k]);
      }
      m = wave_max(m);
      float l = 0.0f;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int i = lane + k * kWave;
        if (i < n) {
          const float p = exp2f(sv[k] - m);
          sc[hh][i] = i < nc ? p * rvs[k] : p;
          l += p;
        }
      }
      l = wave_sum(l);
      if (lane == 0) { stat[hh][0] = m; stat[hh][1] = l; }
    } else {
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
  }
  __syncthreads();

  // ---- o = sum_t p_t v_t
  if constexpr (V8) {
    float o8[G][VDPL8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < VDPL8; ++e) o8[hh][e] = 0.0f;
    for (int b = 0; b < nvsteps; b += UV) {
      if (b > 0) {
#pragma unroll
        for (int u = 0; u < UV; ++u) load_v8(b + u, u);
      }
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        const int t = vrow8(b + u);
        if (b + u < nvsteps && t < tl) {
          float vf[VDPL8];
          if constexpr (I8) {
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) {
              vf[bi] = float(int8_t(uint8_t(v8[u].x >> (8 * bi))));
              vf[4 + bi] = float(int8_t(uint8_t(v8[u].y >> (8 * bi))));
            }
          } else {
            vf[0] = bf_lo(v8[u].x); vf[1] = bf_hi(v8[u].x); vf[2] = bf_lo(v8[u].y); vf[3] = bf_hi(v8[u].y);
          }
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            const float p = sc[hh][t - t0];
#pragma unroll
            for (int e = 0; e < VDPL8; ++e) o8[hh][e] = fmaf(p, vf[e], o8[hh][e]);
          }
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < VDPL8; ++e) o8[hh][e] = fold_groups<VLPR>(o8[hh][e]);
    if (vsub == 0)
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < VDPL8; ++e) ored[wv][hh][vd0 + e] = o8[hh][e];
  } else {
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
        const bool ok = b + u < nsteps && t < tl;
        vv[u] = ok ? *reinterpret_cast<const u32x4*>(vb + (size_t(t) * D + d0) * EB) : z;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = row(b + u);
      if (b + u < nsteps && t < tl) {
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
  }
  if constexpr (I8) {
    // the token's own value row (its score is now its weight in sc)
    if (newrow && wv == 0)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = sc[hh][n - 1] * nvs;
        ored[0][hh][2 * lane] += p * nv0;
        ored[0][hh][2 * lane + 1] += p * nv1;
      }
  }
  __syncthreads();

  attn_finish<D, G, NW>(a, j, s, ns, AttnShared{&ored[0][0][0], &stat[0][0], &cwts[0][0], cden, caccs, &role});
}

// splits per kv head for about one workgroup per compute unit (at most 64)
constexpr int kLongChunkGroups = 512;   // two workgroups per compute unit of the 256

static int target_splits(int n_kv) {
  int splits = kLdsTargetGroups / n_kv;
  return splits < 1 ? 1 : splits > 64 ? 64 : splits;
}

// default chunk of the batched kernel: about one workgroup per compute unit
// over the whole cache, a multiple of 16 rows and no longer than one batch
// of rows in flight
static int batched_default_chunk(int n_kv, int head_dim, int kvtype, int max_ctx) {
  const int lanes_per_row = head_dim * (kvtype == 1 ? 2 : kvtype == 2 ? 1 : 4) / 16;
  const int one_batch = (kWave / lanes_per_row) * 4 * 8;
  const int splits = target_splits(n_kv);
  int c = (max_ctx + splits - 1) / splits;
  c = ((c + 15) / 16) * 16;
  if (c > one_batch) c = one_batch;
  // bf16 and int8 heads of 128 (scores on the matrix cores): 256-row chunks
  // once they still give two workgroups per compute unit, else at most 96
  // rows (more splits, shorter chains per workgroup). Measured, 9B-shaped
  // stacks: 4-bit at 16640 positions 437.8 -> 448.5 tok/s with 256 rows
  // (520 workgroups), at 33024 332.1 -> 360.4 (1032), bf16 at 16640 274.6 ->
  // 279.4 and at 33024 229.4 -> 241.8; at 12544 positions (392 workgroups)
  // 256 rows lost (469.9 -> 464.2, 287.2 -> 285.2), and 96 rows beat 256 on
  // the int8 cache at 8448 (496.1 -> 499.1)
  if (head_dim == 128 && (kvtype == 1 || kvtype == 2)) {
    if (n_kv * ((max_ctx + kChunkMax - 1) / kChunkMax) >= kLongChunkGroups) return kChunkMax;
    if (c > 96) c = 96;
  }
  return c;
}

// default chunk of the streaming and wave-local kernels: about one
// workgroup per compute unit over the whole cache, a multiple of 8 rows, at
// most cmax
static int wide_default_chunk(int n_kv, int max_ctx, int cmax) {
  const int splits = target_splits(n_kv);
  int c = (max_ctx + splits - 1) / splits;
  c = (c + 7) / 8 * 8;
  return c > cmax ? cmax / 8 * 8 : c;
}

bool attn_plan(int n_q, int n_kv, int head_dim, int kvtype, int max_ctx, int chunk_req, int kind_req, int* chunk,
               int* nsplit, int* waves, int* kind) {
  // an int8 cache runs on the batched and streaming kernels (128-wide heads;
  // streamed chunks of at most kChunkMax rows)
  const bool i8 = kvtype == 2;
  int smax = attn_lds_max_chunk(n_q, n_kv, head_dim, kvtype);   // streaming kernel: 0 if none fits
  if (i8 && smax > kChunkMax) smax = kChunkMax;
  const int lmax = kvtype == 1 ? attn_local_max_chunk(head_dim, kvtype) : 0;
  int k = kind_req;
  if (k == kAttnDefault) {
    if (chunk_req > 0) {
      // a requested chunk: the streaming kernel when its values fit in LDS
      k = chunk_req <= smax ? kAttnStream : kAttnBatched;
    } else if (lmax > 0 && n_q == n_kv) {
      // one query head per kv head: the wave-local kernel (its scores and
      // sums are a quarter of a four-head group's; measured on the 7B-shaped
      // bf16 layer: 385.4 -> 397.0 tok/s against the batched kernel). With
      // four heads per kv head it lost (9B-shaped bf16 layer 327.8 -> 323.0,
      // 4-bit 490.8 -> 478.9, 1B-shaped 1686.8 -> 1667.8): their arithmetic
      // waits for the rows, where the streaming kernel scores as they arrive
      // and the batched kernel's smaller workgroups overlap it.
      k = kAttnLocal;
    } else {
      // only mid-length chunks stream: a stream of a few rows never fills
      // (the batched kernel's single pass has fewer barriers), and with
      // 260+ rows per workgroup the batched kernel's three times as many
      // shorter workgroups balance the compute units better (measured:
      // 7B- and 9B-shaped 4-bit caches, 34 MB per layer, 8.6 -> 10.2 us
      // and 15.8 -> 17.4 us streamed)
      const int c = smax > 0 ? wide_default_chunk(n_kv, max_ctx, smax) : 0;
      k = (c >= kStreamMinRows && c <= kStreamMaxRows) ? kAttnStream : kAttnBatched;
    }
  }
  int c = 0, w = 4;
  bool ok = true;
  if (k == kAttnLocal) {
    c = chunk_req > 0 ? chunk_req : wide_default_chunk(n_kv, max_ctx, lmax);
    ok = lmax > 0 && c <= lmax;
    w = kLocalWaves;
  } else if (k == kAttnStream) {
    c = chunk_req > 0 ? chunk_req : wide_default_chunk(n_kv, max_ctx, smax);
    ok = smax > 0 && c <= smax;
    w = kLdsWaves;
  } else {
    ok = k == kAttnBatched && (!i8 || head_dim == 128);
    k = kAttnBatched;
    c = chunk_req > 0 ? chunk_req : batched_default_chunk(n_kv, head_dim, kvtype, max_ctx);
    const int cmin = (max_ctx + kSplitMax - 1) / kSplitMax;
    if (c < cmin) c = cmin;
    if (c < 16) c = 16;
    if (c > kChunkMax) c = kChunkMax;
  }
  if (c < 1) c = 1;
  *chunk = c;
  *nsplit = (max_ctx + c - 1) / c;
  *waves = w;
  *kind = k;
  return ok && *nsplit <= kSplitMax;
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
  constexpr int rows_per_step = (kWave / (D * (KVT == 1 ? 2 : KVT == 2 ? 1 : 4) / 16)) * NW;
  return a.chunk > rows_per_step ? go_attn<D, KVT, NW, true>(a, s) : go_attn<D, KVT, NW, false>(a, s);
}

template <int D, int KVT>
static hipError_t go_attn_waves(const AttnArgs& a, hipStream_t s) {
  if (a.waves == 8) return go_attn_vl<D, KVT, 8>(a, s);
  if (a.waves == 4) return go_attn_vl<D, KVT, 4>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  if (a.kind == kAttnStream) return launch_attn_lds(a, s);
  if (a.kind == kAttnLocal) return launch_attn_local(a, s);
  if (a.nsplit > kSplitMax || a.chunk > kChunkMax) return hipErrorInvalidValue;
  if (a.kvtype == 2) return a.d == 128 && a.waves == 4 ? go_attn_vl<128, 2, 4>(a, s) : hipErrorInvalidValue;
  if (a.d == 64) return a.kvtype == 1 ? go_attn_waves<64, 1>(a, s) : go_attn_waves<64, 0>(a, s);
  if (a.d == 128) return a.kvtype == 1 ? go_attn_waves<128, 1>(a, s) : go_attn_waves<128, 0>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dec
