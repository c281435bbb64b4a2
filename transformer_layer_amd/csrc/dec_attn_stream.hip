// Split-K decode attention with the keys and the values streaming at once.
//
// Grid: n_kv * nsplit workgroups of eight waves, split-major, about one per
// compute unit. From launch, waves 0-3 stream the chunk's key rows and waves
// 4-7 its value rows, each lane keeping U 16-byte loads in flight (a ring:
// each load consumed is replaced at once by the load U rows ahead), so a
// workgroup has 64 KB in flight for its whole life and the cache streams at
// the rate a plain streaming kernel reaches. The key waves score each row
// for every query head of the kv head as it arrives (log2 units, into LDS);
// the value waves write their rows into LDS. Then one exponential per
// (head, position) with the chunk's max, the sum of p * v from the LDS
// values by all eight waves, and the split's partials go to attn_finish
// (stored, then combined by the last arrivals unless the output projection
// combines them).
//
// The keys are never stored: each is used once, as it arrives. The values
// wait in LDS for the softmax; only the chunk's values, its scores and the
// reduction scratch live there.
//
// An int8 cache (KVT 2): the rows hold codes, and the key waves also load
// the chunk's row scales into LDS; the softmax pass applies them (score =
// code dot product times the key scale; the sum of p * v reads p times the
// value scale). The token's own row is not read from the cache: the split
// holding position p streams one row fewer, and wave 0 quantizes the staged
// float k and v rows (the batched kernel's rule), stores codes and scales
// into slot p of the cache, and puts the token's code score, its scales and
// its value codes into the LDS row the cache would have filled, so the
// softmax and the sum treat it like any other row.
//
// A bf16 cache with at most four query heads per kv head scores on the
// matrix cores, as the batched kernel does (its header gives the operand
// layout): each key wave takes 16-row tiles (wave hw: tiles hw, hw + 4, ...;
// lane l reads row l % 16), its ring slots holding the tiles' 16-byte steps.
// The B operand (three bf16 parts of each scaled query head) is built by all
// eight waves, before any row arrives, in the per-wave output sums' LDS,
// which stays unused until the sum of p * v. The sum of p * v runs on the
// matrix cores as well: the value waves store their rows transposed in
// blocks of eight (the A operand layout, dims as its rows), the softmax
// pass stores p as three bf16 parts (the B operand), and wave w sums dims
// 16 w .. 16 w + 15 over every row, so no fold across waves is needed.
//
// LDS layout (bytes), rows padded to cpad (a whole number of eight-wave
// row steps): [values cpad x row][scores G x cpad f32][per-wave output sums
// NW x G x D f32][combine scratch][(m, l) G x 2 f32][role][int8: key and
// value scales 2 x cpad f32][bf16 on the matrix cores: p parts 16 x cpad
// bf16, 16-byte aligned].
#include "dec_attn_common.h"

namespace dec {

template <int D, int KVT>
struct StreamShape {
  static constexpr int EB = KVT == 1 ? 2 : KVT == 2 ? 1 : 4;   // bytes per cache element
  static constexpr int RB = D * EB;             // bytes per cache row
  static constexpr int DPL = 16 / EB;           // dims per lane (16 bytes)
  static constexpr int LPR = D / DPL;           // lanes per row
  static constexpr int RPW = kWave / LPR;       // rows per wave read
  static constexpr int RPH = RPW * 4;           // rows per step of four waves (keys or values)
  static constexpr int RPS = RPW * kLdsWaves;   // rows per step of all eight waves
};

constexpr int kRing = 8;   // loads in flight per lane

__host__ __device__ constexpr int stream_comb_bytes(int G) {
  return ((kSplitMax * G + G) * 4 + 15) / 16 * 16 + kLdsWaves * 64 * 16;
}
// bf16 caches with at most four query heads per kv head: scores and the sum
// of p v on the matrix cores (the latter reads p as three bf16 parts)
__host__ __device__ constexpr bool stream_matrix_cores(int kvtype, int G, int D) {
  return kvtype == 1 && 3 * G <= 16 && D % 32 == 0;
}
__host__ __device__ constexpr int stream_lds_bytes(int cpad, int rb, int G, int D, bool i8, bool pvm) {
  return cpad * rb + G * cpad * 4 + kLdsWaves * G * D * 4 + stream_comb_bytes(G) + G * 2 * 4 + 16 +
         (i8 ? 2 * cpad * 4 : 0) + (pvm ? 16 * cpad * 2 + 16 : 0);
}

template <int D, int KVT, int G>
__global__ __launch_bounds__(kLdsWaves * 64) void attn_stream_kernel(AttnArgs a) {
  using S = StreamShape<D, KVT>;
  constexpr int NW = kLdsWaves;
  constexpr int RB = S::RB, DPL = S::DPL, LPR = S::LPR, RPW = S::RPW, RPH = S::RPH, RPS = S::RPS;
  constexpr int U = kRing;
  static_assert(LPR >= 2 && LPR <= 32, "row layout");
  extern __shared__ __align__(16) uint8_t smem[];

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
  const int n = min(t0 + a.chunk, L) - t0;
  const int cpad = (a.chunk + RPS - 1) / RPS * RPS;
  // int8 cache: the split holding the token streams its rows 0 .. n - 2 and
  // makes row n - 1 from the staged rows
  constexpr bool I8 = KVT == 2;
  const bool newrow = I8 && s == ns - 1;
  const int nc = newrow ? n - 1 : n;   // rows streamed from the cache

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int sub = lane / LPR;
  const int li = lane % LPR;
  const int d0 = li * DPL;
  // scores on the matrix cores: bf16 caches (three bf16 parts of q) and
  // int8 caches (three int8 digits of q, the batched kernel's scheme)
  constexpr bool MSB = stream_matrix_cores(KVT, G, D);
  constexpr bool MSI = KVT == 2 && 3 * G <= 16 && D == 128;
  constexpr bool MS = MSB || MSI;
  constexpr int KPS = MSI ? 64 : 32;    // dims per matrix step
  constexpr int KSTEPS = D / KPS;       // matrix steps (ring slots) per 16-row tile
  static_assert(!MS || U % KSTEPS == 0, "whole tiles per ring");
  constexpr int QPAIRS = 16 * D / 2;    // B operand words
  constexpr int QPT = (QPAIRS + NW * 64 - 1) / (NW * 64);
  const int kr = lane & 15, kg = lane >> 4;

  uint8_t* vbuf = smem;                                                   // [cpad][RB]
  float* sc = reinterpret_cast<float*>(smem + cpad * RB);                 // [G][cpad]
  float* ored = sc + G * cpad;                                            // [NW][G][D]
  float* wts = ored + NW * G * D;                                         // [kSplitMax][G]
  float* den = wts + kSplitMax * G;                                       // [G]
  uint8_t* after = reinterpret_cast<uint8_t*>(ored + NW * G * D) + stream_comb_bytes(G) - NW * 64 * 16;
  float4* accs = reinterpret_cast<float4*>(after);                        // [NW * 64]
  float* stat = reinterpret_cast<float*>(after + NW * 64 * 16);           // [G][2]
  int* role = reinterpret_cast<int*>(stat + G * 2);
  float* ksl = reinterpret_cast<float*>(role + 4);                        // int8: [cpad] key scales
  float* vsl = ksl + cpad;                                                // int8: [cpad] value scales
  // bf16, matrix cores: p as three bf16 parts, [16][cpad] (column part G + head)
  uint16_t* pp = reinterpret_cast<uint16_t*>(
      smem + (int(reinterpret_cast<uint8_t*>(I8 ? vsl + cpad : ksl) - smem) + 15) / 16 * 16);

  // waves 0-3 stream keys, waves 4-7 values: row r of the chunk is read by
  // wave (r / RPW) % 4 of its half at step r / RPH
  const bool keys = wv < 4;
  const int hw = keys ? wv : wv - 4;
  const int nsteps = (nc + RPH - 1) / RPH;
  const int rlast = nc > 0 ? nc - 1 : 0;   // a valid row (slot t0 <= pos) even when none is streamed
  const uint8_t* src = reinterpret_cast<const uint8_t*>(keys ? a.kc : a.vc) +
                       (size_t(j) * a.max_ctx + t0) * RB + li * 16;
  auto row_of = [&](int step) { return step * RPH + hw * RPW + sub; };
  auto load = [&](int step) {
    int r = row_of(step);
    r = r < nc ? r : rlast;   // every load is issued: past the chunk, its last row again
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + size_t(r) * RB));
  };
  // matrix-core key waves: slot k holds step k % KSTEPS of the wave's tile
  // k / KSTEPS (chunk tile hw + 4 (k / KSTEPS)), row kr, dims KPS step + KPS / 4 kg
  const uint8_t* ksrc = reinterpret_cast<const uint8_t*>(a.kc) + (size_t(j) * a.max_ctx + t0) * RB;
  auto kload = [&](int k) {
    int r = 16 * (hw + 4 * (k / KSTEPS)) + kr;
    r = r < nc ? r : rlast;
    return __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(ksrc + size_t(r) * RB + (KPS * (k % KSTEPS) + KPS / 4 * kg) * S::EB));
  };
  // the B operand's words of this thread: q first, so waiting for it does
  // not wait for the ring
  float2 qx[MSB ? QPT : 1];
  float2 qi = {0.0f, 0.0f};   // int8: wave wv < G holds dims 2 lane, 2 lane + 1 of head wv
  if constexpr (MSI) {
    if (wv < G) qi = *reinterpret_cast<const float2*>(a.q + (j * G + wv) * D + 2 * lane);
  }
  if constexpr (MSB) {
#pragma unroll
    for (int r = 0; r < QPT; ++r) {
      const int e = tid + r * NW * 64;   // word e: column e / (D / 2), dims 2 (e % (D / 2)) + 0, 1
      const int c = e / (D / 2), dd = 2 * (e % (D / 2));
      qx[r] = e < QPAIRS && c < 3 * G ? *reinterpret_cast<const float2*>(a.q + (j * G + c % G) * D + dd)
                                      : make_float2(0.0f, 0.0f);
    }
  }
  // the ring: slot u holds step k0 + u; a consumed slot is refilled at once
  // with the step U ahead. Every load is issued (a step past the chunk
  // re-reads its last row, a cache hit): refilled conditionally, the
  // compiler waited for the whole ring before each use.
  u32x4 ring[U];
#pragma unroll
  for (int u = 0; u < U; ++u) ring[u] = MS && keys ? kload(u) : load(u);

  // int8: the key waves request the chunk's row scales (rows hw * 64 + lane
  // + 256 k, clamped to the streamed rows; written to LDS once the scores
  // are done), wave 0 of the token's split the staged k and v rows
  constexpr int NSC = I8 ? (kChunkMax + 255) / 256 : 1;
  float rks[NSC], rvs[NSC];
  float2 kx = {0.0f, 0.0f}, vx = {0.0f, 0.0f};
  const size_t scale_off = I8 ? kv_i8_scale_off(a.nkv, a.max_ctx, D) : 0;
  if constexpr (I8) {
    if (keys) {
      const float* ksc = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.kc) + scale_off) +
                         size_t(j) * a.max_ctx + t0;
      const float* vsc = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.vc) + scale_off) +
                         size_t(j) * a.max_ctx + t0;
#pragma unroll
      for (int k = 0; k < NSC; ++k) {
        const int i = min(hw * kWave + lane + 256 * k, rlast);
        rks[k] = ksc[i];
        rvs[k] = vsc[i];
      }
      if (newrow && wv == 0) {
        const size_t so = kv_i8_stage_off(a.nkv, a.max_ctx, D);
        kx = *reinterpret_cast<const float2*>(
            reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.kc) + so) + size_t(j) * D + 2 * lane);
        vx = *reinterpret_cast<const float2*>(
            reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.vc) + so) + size_t(j) * D + 2 * lane);
      }
    }
  }

  uint32_t* qp = reinterpret_cast<uint32_t*>(ored);   // [16][D / 2] words; 16 D 2 <= NW G D 4 bytes
  int* qe = role;   // int8: each head's exponent (G <= 4 words; the role word is set only at the combine)
  if constexpr (MS) {
    const float qscale = kLog2e / sqrtf(float(D));
    if constexpr (MSB) {
#pragma unroll
      for (int r = 0; r < QPT; ++r) {
        const int e = tid + r * NW * 64;
        if (e < QPAIRS) {
          const int p = (e / (D / 2)) / G;   // 3 and above: a zero column (its q words are zero)
          qp[e] = q_part_bf16(qx[r].x * qscale, p) | (q_part_bf16(qx[r].y * qscale, p) << 16);
        }
      }
    } else if (wv < G) {
      // int8: wave h < G builds head h's digit columns h, G + h, 2G + h
      // (D bytes each; columns 3G and up are never read)
      const float x0 = qi.x * qscale, x1 = qi.y * qscale;
      const bool finite = __all(fabsf(x0) <= 3.4028235e38f && fabsf(x1) <= 3.4028235e38f);
      const int e = query_exp_i8_checked(wave_max(fmaxf(fabsf(x0), fabsf(x1))), finite);
      int a0, a1, a2, b0, b1, b2;
      query_digits_i8(x0, e, a0, a1, a2);
      query_digits_i8(x1, e, b0, b1, b2);
      uint16_t* qd = reinterpret_cast<uint16_t*>(qp);   // [16][D / 2] pairs of int8
      qd[(0 * G + wv) * (D / 2) + lane] = uint16_t((a0 & 255) | ((b0 & 255) << 8));
      qd[(1 * G + wv) * (D / 2) + lane] = uint16_t((a1 & 255) | ((b1 & 255) << 8));
      qd[(2 * G + wv) * (D / 2) + lane] = uint16_t((a2 & 255) | ((b2 & 255) << 8));
      if (lane == 0) qe[wv] = e;
    }
    __syncthreads();
  }

  if (keys) {
    if constexpr (MS) {
      // ---- scores (log2 units) on the matrix cores, 16-row tiles
      u32x4 qb[KSTEPS];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        qb[ks] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(qp) + kr * D * S::EB +
                                                 (KPS * ks + KPS / 4 * kg) * S::EB);
      const int ekr = MSI ? qe[kr < G ? kr : 0] : 0;
      const int ntile = (nc + 15) / 16;
      const int nk = hw < ntile ? (ntile - hw + 3) / 4 * KSTEPS : 0;   // slots this wave consumes
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      i32x4 iacc = {0, 0, 0, 0};
      for (int k0 = 0; k0 < nk; k0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const u32x4 w = ring[u];
          ring[u] = kload(k0 + U + u);
          if (k0 + u < nk) {   // wave-uniform
            const int ks = u % KSTEPS;   // a constant once unrolled
            if constexpr (MSB) {
              if (ks == 0) acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                            __builtin_bit_cast(bf16x8, qb[ks]), acc, 0, 0, 0);
            } else {
              if (ks == 0) iacc = i32x4{0, 0, 0, 0};
              iacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, w),
                                                           __builtin_bit_cast(i32x4, qb[ks]), iacc, 0, 0, 0);
            }
            if (ks == KSTEPS - 1) {
              // lane kr < G: head kr's three columns (DPP row shifts left by G, 2G)
              float sv[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if constexpr (MSB)
                  sv[i] = acc[i] + dpp_mov<0x100 + G>(acc[i]) + dpp_mov<0x100 + 2 * G>(acc[i]);
                else
                  sv[i] = digit_score(iacc[i], dpp_mov_i<0x100 + G>(iacc[i]), dpp_mov_i<0x100 + 2 * G>(iacc[i]), ekr);
              }
              const int tile = hw + 4 * ((k0 + u) / KSTEPS);
              float* dst = sc + kr * cpad + 16 * tile + 4 * kg;
              if (kr < G) {
                if constexpr (MSB) {
                  // rows 16 tile + 4 kg .. + 3 (past nc: never read); 16 ceil(nc / 16) <= cpad
                  *reinterpret_cast<float4*>(dst) = make_float4(sv[0], sv[1], sv[2], sv[3]);
                } else {
                  // int8: only the streamed rows (row nc may be the token's, scored by wave 0)
#pragma unroll
                  for (int i = 0; i < 4; ++i)
                    if (16 * tile + 4 * kg + i < nc) dst[i] = sv[i];
                }
              }
            }
          }
        }
      }
    } else {
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
      // ---- scores (log2 units): s_t = (q . k_t) log2(e) / sqrt(d)
      for (int k0 = 0; k0 < nsteps; k0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const u32x4 w = ring[u];
          ring[u] = load(k0 + U + u);
          if (k0 + u < nsteps) {
            const int t = row_of(k0 + u);
            float kf[DPL];
            unpack_row<KVT>(w, kf);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
              float p = 0.0f;
#pragma unroll
              for (int e = 0; e < DPL; ++e) p = fmaf(qv[hh][e], kf[e], p);
              p = group_sum<LPR>(p);
              if (t < nc && li == 0) sc[hh * cpad + t] = p;
            }
          }
        }
      }
    }
    if constexpr (I8) {
#pragma unroll
      for (int k = 0; k < NSC; ++k) {
        const int i = hw * kWave + lane + 256 * k;
        if (i < nc) {
          ksl[i] = rks[k];
          vsl[i] = rvs[k];
        }
      }
      // the token's row: quantized in float32, stored into slot pos, and
      // entered as LDS row n - 1 (code score, scales, value codes)
      static_assert(!I8 || D == 2 * kWave, "int8 cache rows: two dims a lane");
      if (newrow && wv == 0) {
        float kc0, kc1, kscale, vc0, vc1, vscale;
        quantize_pair_i8(kx, kc0, kc1, kscale);
        quantize_pair_i8(vx, vc0, vc1, vscale);
        const size_t slot = size_t(j) * a.max_ctx + pos;
        uint8_t* kcw = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.kc));
        uint8_t* vcw = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(a.vc));
        const uint16_t vpair = pack_i8_pair(vc0, vc1);
        *reinterpret_cast<uint16_t*>(kcw + slot * D + 2 * lane) = pack_i8_pair(kc0, kc1);
        *reinterpret_cast<uint16_t*>(vcw + slot * D + 2 * lane) = vpair;
        *reinterpret_cast<uint16_t*>(vbuf + (n - 1) * RB + 2 * lane) = vpair;
        if (lane == 0) {
          *reinterpret_cast<float*>(kcw + scale_off + slot * 4) = kscale;
          *reinterpret_cast<float*>(vcw + scale_off + slot * 4) = vscale;
          ksl[n - 1] = kscale;
          vsl[n - 1] = vscale;
        }
        const float qscale = kLog2e / sqrtf(float(D));
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float2 qx = *reinterpret_cast<const float2*>(a.q + (j * G + hh) * D + 2 * lane);
          const float d = wave_sum(fmaf(qx.x * qscale, kc0, (qx.y * qscale) * kc1));
          if (lane == 0) sc[hh * cpad + n - 1] = d;
        }
      }
    }
  } else {
    // ---- values into LDS as they arrive. For the matrix cores the rows go
    // in blocks of eight, transposed: dim d of rows 8 b .. 8 b + 7 is the 16
    // bytes at block b, position pi(d) = (d % 8) (D / 8) + d / 8 (so the 16
    // lanes of a row write 16 consecutive positions of a block)
    for (int k0 = 0; k0 < nsteps; k0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4 w = ring[u];
        ring[u] = load(k0 + U + u);
        if (k0 + u < nsteps) {
          const int t = row_of(k0 + u);   // < cpad: the steps cover at most cpad rows
          if constexpr (MSB) {
            uint16_t* vt = reinterpret_cast<uint16_t*>(vbuf) + ((t / 8) * D + li) * 8 + t % 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) vt[e * (D / 8) * 8] = uint16_t(w[e / 2] >> (16 * (e % 2)));
          } else if (!I8 || t < nc) {
            *reinterpret_cast<u32x4*>(vbuf + t * RB + li * 16) = w;   // int8: row nc is the token's
          }
        }
      }
    }
    if constexpr (MSB) {
      // rows past the streamed steps up to a whole 32-row matrix step: zero
      // (their p is zero too; uninitialized LDS could hold NaN bits)
      const int z0 = nsteps * RPH, z1 = (n + 31) / 32 * 32;
      for (int i = hw * kWave + lane; i < (z1 - z0) / 8 * D; i += 4 * kWave)
        *reinterpret_cast<u32x4*>(vbuf + ((z0 / 8) * D + i) * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();

  // ---- per head: m = max s, p = exp2(s - m), l = sum p (int8: s = code
  // score x key scale; the sum of p v below reads p x value scale)
  for (int hh = wv; hh < G; hh += NW) {
    float m = -INFINITY;
    for (int i = lane; i < n; i += kWave) m = fmaxf(m, I8 ? sc[hh * cpad + i] * ksl[i] : sc[hh * cpad + i]);
    m = wave_max(m);
    float l = 0.0f;
    for (int i = lane; i < n; i += kWave) {
      const float p = exp2f((I8 ? sc[hh * cpad + i] * ksl[i] : sc[hh * cpad + i]) - m);
      sc[hh * cpad + i] = I8 ? p * vsl[i] : p;
      if constexpr (MSB) {
#pragma unroll
        for (int pt = 0; pt < 3; ++pt) pp[(pt * G + hh) * cpad + i] = uint16_t(q_part_bf16(p, pt));
      }
      l += p;
    }
    if constexpr (MSB) {
      for (int i = n + lane; i < (n + 31) / 32 * 32; i += kWave)
#pragma unroll
        for (int pt = 0; pt < 3; ++pt) pp[(pt * G + hh) * cpad + i] = 0;
    }
    l = wave_sum(l);
    if (lane == 0) { stat[hh * 2] = m; stat[hh * 2 + 1] = l; }
  }
  __syncthreads();

  if constexpr (MSB) {
    // ---- o = sum_t p_t v_t on the matrix cores: wave w takes dims 16 w ..
    // 16 w + 15 (A operand: lane l holds dim 16 w + l % 16 of rows 32 ks +
    // 8 (l / 16) .. + 7, one block of the transposed values) over every row;
    // B holds p's three bf16 parts of each head (column part G + head), so
    // a head's three columns sum to the float32 p times exact bf16 values
    constexpr int NT = D / 16;
    if (wv < NT) {
      const int m = 16 * wv + kr;
      const int dp = (m % 8) * (D / 8) + m / 8;
      const int c = kr < 3 * G ? kr : 0;   // columns 3G and up repeat column 0 (never read)
      const int nks = (n + 31) / 32;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int ks = 0; ks < nks; ++ks) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(vbuf + ((4 * ks + kg) * D + dp) * 16);
        const u32x4 bv = *reinterpret_cast<const u32x4*>(pp + c * cpad + 32 * ks + 8 * kg);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
      }
      // lane kr < G: head kr, dims 16 w + 4 kg .. + 3 (every lane takes part in the shifts)
      float ov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = acc[i] + dpp_mov<0x100 + G>(acc[i]) + dpp_mov<0x100 + 2 * G>(acc[i]);
      if (kr < G)
        *reinterpret_cast<float4*>(ored + kr * D + 16 * wv + 4 * kg) = make_float4(ov[0], ov[1], ov[2], ov[3]);
    }
    __syncthreads();
    attn_finish<D, G, NW, 1>(a, j, s, ns, AttnShared{ored, stat, wts, den, accs, role});
    return;
  }

  // ---- o = sum_t p_t v_t, all eight waves over the LDS values. int8 and
  // bf16 rows are read eight bytes a lane (8 codes, 4 bf16 dims), so the rows
  // of a read sit more lanes apart and the fold below takes fewer steps over
  // fewer accumulators (int8: 16 codes a lane took three steps over 64; bf16:
  // two steps over 32 became one over 16, 9B-shaped layer 326.6 -> 329.3
  // tok/s on one box).
  constexpr bool PV8 = I8 || KVT == 1;   // 8-byte LDS reads of the value rows
  constexpr int PDPL = I8 ? 8 : PV8 ? 4 : DPL;    // dims per lane
  constexpr int PLPR = D / PDPL;        // lanes per row
  constexpr int PRPW = kWave / PLPR;    // rows per wave read
  constexpr int PRPS = PRPW * NW;       // rows per step of all eight waves
  static_assert(PLPR >= 2 && PLPR <= 32, "row layout");
  const int psub = lane / PLPR;
  const int pd0 = (lane % PLPR) * PDPL;
  float o[G][PDPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < PDPL; ++e) o[hh][e] = 0.0f;
  const int nsteps8 = (n + PRPS - 1) / PRPS;
  for (int b = 0; b < nsteps8; ++b) {
    const int t = b * PRPS + wv * PRPW + psub;
    if (t < n) {
      float vf[PDPL];
      if constexpr (I8) {
        const uint2 w = *reinterpret_cast<const uint2*>(vbuf + t * RB + pd0);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
          vf[bi] = float(int8_t(uint8_t(w.x >> (8 * bi))));
          vf[4 + bi] = float(int8_t(uint8_t(w.y >> (8 * bi))));
        }
      } else if constexpr (PV8) {
        const uint2 w = *reinterpret_cast<const uint2*>(vbuf + t * RB + pd0 * 2);
        vf[0] = bf_lo(w.x); vf[1] = bf_hi(w.x); vf[2] = bf_lo(w.y); vf[3] = bf_hi(w.y);
      } else {
        unpack_row<KVT>(*reinterpret_cast<const u32x4*>(vbuf + t * RB + pd0 * (RB / D)), vf);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = sc[hh * cpad + t];
#pragma unroll
        for (int e = 0; e < PDPL; ++e) o[hh][e] = fmaf(p, vf[e], o[hh][e]);
      }
    }
  }
  // rows of one wave read sit PLPR lanes apart: fold them
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < PDPL; ++e) o[hh][e] = fold_groups<PLPR>(o[hh][e]);
  if (psub == 0)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < PDPL; ++e) ored[(wv * G + hh) * D + pd0 + e] = o[hh][e];
  __syncthreads();

  attn_finish<D, G, NW>(a, j, s, ns, AttnShared{ored, stat, wts, den, accs, role});
}

// rows per eight-wave step and bytes per row of a shape
static void stream_row_shape(int head_dim, int kvtype, int* rps, int* rb) {
  const int eb = kvtype == 1 ? 2 : kvtype == 2 ? 1 : 4;
  *rb = head_dim * eb;
  const int lpr = head_dim * eb / 16;
  *rps = (kWave / lpr) * kLdsWaves;
}

static bool stream_fits(int n_q, int n_kv, int head_dim, int kvtype, int chunk) {
  int rps, rb;
  stream_row_shape(head_dim, kvtype, &rps, &rb);
  const int cpad = (chunk + rps - 1) / rps * rps;
  return stream_lds_bytes(cpad, rb, n_q / n_kv, head_dim, kvtype == 2,
                          stream_matrix_cores(kvtype, n_q / n_kv, head_dim)) <= kLdsBudget;
}

int attn_lds_max_chunk(int n_q, int n_kv, int head_dim, int kvtype) {
  // int8 rows: 128-wide heads (two dims a lane over a wave), groups of at most four heads
  if (kvtype == 2 && (head_dim != 128 || n_q / n_kv > 4)) return 0;
  int rps, rb;
  stream_row_shape(head_dim, kvtype, &rps, &rb);
  if (!stream_fits(n_q, n_kv, head_dim, kvtype, rps)) return 0;
  int c = rps;
  while (stream_fits(n_q, n_kv, head_dim, kvtype, c + rps)) c += rps;
  return c;
}

template <int D, int KVT>
static hipError_t go_attn_stream(const AttnArgs& a, hipStream_t s) {
  using S = StreamShape<D, KVT>;
  const int g = a.nq / a.nkv;
  const int cpad = (a.chunk + S::RPS - 1) / S::RPS * S::RPS;
  const int lds = stream_lds_bytes(cpad, S::RB, g, D, KVT == 2, stream_matrix_cores(KVT, g, D));
  if (lds > kLdsBudget) return hipErrorInvalidValue;
  const dim3 grid(a.nkv * a.nsplit), block(kLdsWaves * 64);
  switch (g) {
    case 1: hipLaunchKernelGGL((attn_stream_kernel<D, KVT, 1>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((attn_stream_kernel<D, KVT, 2>), grid, block, lds, s, a); break;
    case 4: hipLaunchKernelGGL((attn_stream_kernel<D, KVT, 4>), grid, block, lds, s, a); break;
    case 8:
      // int8 rows hold 16 dims a lane: eight heads' queries would not fit in registers
      if constexpr (KVT == 2) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((attn_stream_kernel<D, KVT, 8>), grid, block, lds, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_lds(const AttnArgs& a, hipStream_t s) {
  if (a.nsplit > kSplitMax) return hipErrorInvalidValue;
  // int8: 128-wide heads, at most kChunkMax rows (the key waves load the scales of 256 rows)
  if (a.kvtype == 2 && (a.d != 128 || a.chunk > kChunkMax)) return hipErrorInvalidValue;
  if (a.d == 64) return a.kvtype == 1 ? go_attn_stream<64, 1>(a, s) : go_attn_stream<64, 0>(a, s);
  if (a.d == 128) {
    if (a.kvtype == 2) return go_attn_stream<128, 2>(a, s);
    return a.kvtype == 1 ? go_attn_stream<128, 1>(a, s) : go_attn_stream<128, 0>(a, s);
  }
  if (a.kvtype == 2) return hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

}  // namespace dec
