// Four-bit GEMV on the int8 matrix cores.
//
// Streaming 4-bit weights at HBM speed through the vector ALUs costs about
// two VALU instructions per weight (a byte-to-float conversion and a
// multiply-add) and leaves the kernel ALU-bound. Here the products run on
// v_mfma_i32_16x16x64_i8 in exact integer arithmetic; the VALUs only unpack
// nibbles and apply the block scales.
//
// Input: per 32-element block b of the (normalized) input vector u, the
// workgroup picks the power of two 2^E_b that brings max|u| below 2^22 (and
// at least 2^21) and writes u_e 2^E_b = X_e as an integer (round to nearest
// even), split into three balanced base-256 digits X = d0 + 256 d1 + 65536 d2,
// each in [-128, 127], stored in LDS with E_b.
//
// Weights: a 16-byte load gives lane (n, g) (column n = lane % 16, k-group
// g = lane / 16) a whole block of one row: 32 nibbles. Masking with 0xf0
// (the high nibble of each byte in place, the low one shifted up by four)
// makes each byte the signed int8 16 * code. A step covers four consecutive
// blocks 4s + g of 16 rows: two MFMAs (elements 0..15 and 16..31 of each
// lane's block) with the digit operand
//   A[m][k] = digit p of block 4s + g at k,  m = 4 g + p  (p < 3), else 0
// give C[4 g + p][n] = 16 sum_e code_e d_p[e] exactly, in lane (n, g). The
// lane forms V = C0 + 256 C1 + 65536 C2 (= 16 sum_e code_e X_e, two float
// roundings) and adds scale_b 2^(-E_b - 4) V to its accumulator. Inside a
// lane the digits are ordered as the bytes unpack: low nibbles of a word
// first, then its high nibbles.
//
// A workgroup of NW waves loads the input, requests the weights of its
// first tile, and quantizes the input (its first four waves) while those
// stream in; a second tile's weights are requested once the input is
// quantized (measured: requested together with the first, they delayed it
// by about 0.9 µs on the 9B-shaped gated FFN). A tile is 8 row pairs (16
// rows, one per MFMA column); the waves split a tile's steps. A workgroup
// takes TT adjacent tiles (one, or two when one per workgroup would not fit
// on the chip at once, or three for large gated FFNs). Partial sums meet across the four k-groups with lane swaps
// and across waves in LDS, in a fixed order.
#pragma once

#include "dec_gemv.h"

namespace dec {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Block scales go through LDS for up to 12 steps per wave; for the longest
// rows (16 steps, up to 16384 columns) that would pass 64 KB, and each lane
// loads its own scales instead.
__host__ __device__ constexpr bool q4mfma_scales_in_lds(int spw) { return spw <= 12; }

// LDS bytes: the digits and exponents of `cols` elements (blocks padded to a
// whole step), the cross-wave sums (double-buffered), the sum-of-squares
// slots, 16 zero bytes, and (scales in LDS) every wave's block scales of its
// tiles ([nw][tt][16 rows][4 spw blocks] fp16). At most 64 KB for every
// shape the launcher accepts (64032 bytes at 12288 columns, two tiles).
__host__ __device__ constexpr int q4mfma_lds_bytes(int cols, int nw, int spw, int tt) {
  return ((cols / 32 + 3) / 4) * 4 * (96 + 4) + nw * 16 * 4 * 2 + 16 + 16 +
         (q4mfma_scales_in_lds(spw) ? nw * tt * 16 * 4 * spw * 2 : 0);
}

// Sum of squares of the input vector in the order the 4-bit kernels use
// (q4mfma_sumsq_regs): threads 0..255 each take float4 groups tid, tid + 256,
// ...; the caller adds the four wave sums in wave order. For the per-op
// RMSNorm.
__device__ __forceinline__ float q4mfma_sumsq_part(const float4* in4, int nf, int tid) {
  float ss = 0.0f;
  for (int f0 = 0; f0 < nf; f0 += 4 * 256) {   // four loads in flight, then their squares in order
    float4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int f = f0 + k * 256 + tid;
      if (f < nf) v[k] = in4[f];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (f0 + k * 256 + tid < nf) {
        ss = fmaf(v[k].x, v[k].x, ss);
        ss = fmaf(v[k].y, v[k].y, ss);
        ss = fmaf(v[k].z, v[k].z, ss);
        ss = fmaf(v[k].w, v[k].w, ss);
      }
    }
  }
  return wave_sum(ss);
}

// Float4 groups of the input vector held by each of the 256 quantizing
// threads: thread t holds groups t, t + 256, ... (group f: elements 4 (f % 8)
// .. of block f / 8). Enough for SPW steps on each of NW waves.
template <int NW, int SPW>
constexpr int q4mfma_groups() { return SPW * NW / 8; }

// Thread t's input groups (and, with NORM, the norm weights of the same
// elements, fp32 or bf16 pairs), requested before any weight so that they
// return first. Loads are clamped to the vector; padding groups are zeroed
// where they are used.
template <bool NORM, int NTYPE, int GQ>
__device__ __forceinline__ void q4mfma_load_input(const GemvArgs& a, int tid, float4 (&xv)[GQ], uint4 (&gv)[GQ]) {
  const int nf = a.cols / 4;
  const float4* in4 = reinterpret_cast<const float4*>(a.in);
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
    const int f = tid + 256 * i;
    const int fc = f < nf ? f : nf - 1;
    xv[i] = in4[fc];
    if constexpr (NORM) {
      if constexpr (NTYPE == 1) {
        const uint2 gb = reinterpret_cast<const uint2*>(a.norm)[fc];
        gv[i] = make_uint4(gb.x, gb.y, 0u, 0u);
      } else {
        gv[i] = reinterpret_cast<const uint4*>(a.norm)[fc];
      }
    }
  }
}

// Sum of squares over thread t's groups, in order (the per-op RMSNorm's
// q4mfma_sumsq_part adds the same values in the same order), then over the
// wave.
template <int GQ>
__device__ __forceinline__ float q4mfma_sumsq_regs(const float4 (&xv)[GQ], int nf, int tid) {
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
    if (tid + 256 * i < nf) {
      ss = fmaf(xv[i].x, xv[i].x, ss);
      ss = fmaf(xv[i].y, xv[i].y, ss);
      ss = fmaf(xv[i].z, xv[i].z, ss);
      ss = fmaf(xv[i].w, xv[i].w, ss);
    }
  }
  return wave_sum(ss);
}

// Thread t's groups as digits in LDS. The eight threads of a block share its
// maximum through lane moves. With NORM, u = (x r) g (the RMSNorm), with no
// contraction of these products into anything else.
template <bool NORM, int NTYPE, int GQ>
__device__ __forceinline__ void q4mfma_quantize(const GemvArgs& a, float r, const float4 (&xv)[GQ],
                                                const uint4 (&gv)[GQ], uint8_t* dig, int* ex, int GP, int tid) {
#pragma clang fp contract(off)
  const int nf = a.cols / 4;
#pragma unroll
  for (int i = 0; i < GQ; ++i) {   // uniform trip count: the block maxima use every lane
    const int f = tid + 256 * i;
    const bool in_vec = f < nf;
    float u[4] = {in_vec ? xv[i].x : 0.0f, in_vec ? xv[i].y : 0.0f, in_vec ? xv[i].z : 0.0f,
                  in_vec ? xv[i].w : 0.0f};
    if constexpr (NORM) {
      float gw[4];
      if constexpr (NTYPE == 1) {
        gw[0] = bf_lo(gv[i].x); gw[1] = bf_hi(gv[i].x); gw[2] = bf_lo(gv[i].y); gw[3] = bf_hi(gv[i].y);
      } else {
        gw[0] = __uint_as_float(gv[i].x); gw[1] = __uint_as_float(gv[i].y);
        gw[2] = __uint_as_float(gv[i].z); gw[3] = __uint_as_float(gv[i].w);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) u[t] = (u[t] * r) * gw[t];
    }
    float m = fmaxf(fmaxf(fabsf(u[0]), fabsf(u[1])), fmaxf(fabsf(u[2]), fabsf(u[3])));
    m = group_max<8>(m);
    int e = 0;
    (void)frexpf(m, &e);
    const int E = m > 0.0f ? 22 - e : 0;   // |u| 2^E < 2^22
    uint32_t ev[3], od[3];                 // digits of elements t = 0, 2 and of t = 1, 3 as byte pairs
#pragma unroll
    for (int p = 0; p < 3; ++p) ev[p] = od[p] = 0u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int X = int(rintf(ldexpf(u[t], E)));
      const int d0 = ((X + 128) & 255) - 128;
      const int X1 = (X - d0) >> 8;
      const int d1 = ((X1 + 128) & 255) - 128;
      const int d2 = (X1 - d1) >> 8;
      const int sh = 8 * (t >> 1);
      uint32_t* dst = (t & 1) ? od : ev;
      dst[0] |= (uint32_t(d0) & 255u) << sh;
      dst[1] |= (uint32_t(d1) & 255u) << sh;
      dst[2] |= (uint32_t(d2) & 255u) << sh;
    }
    if (f < GP * 8) {
      const int b = f >> 3, j = f & 7;
      const int h = j >> 2, jj = j & 3;
      // element 4 jj + t of half h: byte (4 jj + t) % 8 / 2 of word 2 (jj / 2) + (t & 1)
      const int off = 8 * (jj >> 1) + 2 * (jj & 1);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        uint8_t* base = dig + ((b * 3 + p) * 2 + h) * 16 + off;
        *reinterpret_cast<uint16_t*>(base) = uint16_t(ev[p]);
        *reinterpret_cast<uint16_t*>(base + 4) = uint16_t(od[p]);
      }
      if (j == 0) ex[b] = E;
    }
  }
}

// 16 * code of the high and of the low nibble of each byte, as int8 lanes
__device__ __forceinline__ int q4_hi16(uint32_t w) { return int(w & 0xf0f0f0f0u); }
__device__ __forceinline__ int q4_lo16(uint32_t w) { return int((w << 4) & 0xf0f0f0f0u); }

// One workgroup's share of a 4-bit GEMV: TT tiles of 16 rows, the input as
// digits in LDS, NW waves splitting each tile's steps. The kernels below
// compose its steps: request the input, the tiles' scales and weights; the
// prologue (RMSNorm for the fused epilogues, the digits, the staged scales);
// then each tile's products and epilogue.
template <int EPI, int NW, int SPW, int TT>
struct Q4Tiles {
  using PE = PairEpi<EPI>;
  static constexpr bool NORM = epi_has_norm(EPI);
  static_assert(NW >= 4, "the sum of squares uses the first four waves");
  // block scales of a wave's steps (4 SPW blocks from block 4 s0) for a
  // tile's 16 rows. In LDS mode: row-contiguous 2-byte loads (KL lanes per
  // row, so a load touches few cache lines) written to LDS, where each step
  // reads its lane's scale. Otherwise each lane loads the scale of each of
  // its steps (a 32-bit register per scale: two 16-bit values packed in one
  // register would make each load wait for the previous one).
  static constexpr bool SL = q4mfma_scales_in_lds(SPW);
  static constexpr int KB = 4 * SPW;                               // blocks per row of a wave's share
  static constexpr int KL = KB <= 16 ? 16 : KB <= 32 ? 32 : 64;    // lanes per row in a load
  static constexpr int NSL = SL ? 16 * KL / 64 : SPW;              // scale loads per tile
  static constexpr int GQ = q4mfma_groups<NW, SPW>();             // input groups per quantizing thread

  const GemvArgs& a;
  int tid, lane, wv, n, g;   // n: MFMA column (row n of the tile); g: k-group (block 4s + g of a step)
  int G, S, GP;              // blocks per row, steps of four blocks, blocks with padding
  uint8_t* dig;              // [GP][3][2][16] digits
  int* ex;                   // [GP] exponents E_b
  float* red;                // [2][NW][16] cross-wave sums
  float* ssq;                // [4] sums of squares
  uint8_t* zero16;           // 16 zero bytes
  uint16_t* scl;             // this wave's staged scales [TT][16][KB]
  size_t row_bytes;
  int npairs, s0, ns;        // row pairs; this wave's first step and step count (wave-uniform)

  __device__ __forceinline__ Q4Tiles(const GemvArgs& args, uint8_t* smem) : a(args) {
    tid = threadIdx.x;
    lane = tid & 63;
    wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    n = lane & 15;
    g = lane >> 4;
    G = a.cols / 32;
    S = (G + 3) / 4;
    GP = 4 * S;
    dig = smem;
    ex = reinterpret_cast<int*>(smem + size_t(GP) * 96);
    red = reinterpret_cast<float*>(ex + GP);
    ssq = red + 2 * NW * 16;
    zero16 = reinterpret_cast<uint8_t*>(ssq + 4);
    scl = reinterpret_cast<uint16_t*>(zero16 + 16) + wv * TT * 16 * KB;
    row_bytes = size_t(a.cols) / 2;
    npairs = PE::npairs(a);
    s0 = wv * SPW;
    ns = max(0, min(S - s0, SPW));
  }

  // the first four waves quantize the input
  __device__ __forceinline__ bool quant() const { return tid < 256; }

  // row c (0..15) of a tile: the first or second row of pair c % 8, in the
  // first matrix or (gate/up pairs, c >= 8) the second
  __device__ __forceinline__ int row_at(int tile, int c, bool& second) const {
    int p = tile * 8 + (c & 7);
    p = p < npairs ? p : npairs - 1;   // a tile past the last: valid rows, never stored
    int r0, r1;
    PE::rows(a, p, r0, r1);
    int r = c < 8 ? r0 : r1;
    second = PE::PAIRED && c >= 8;
    return r < a.rows ? r : a.rows - 1;
  }

  // weights of this lane's row of a tile, for this wave's steps. Every load
  // is issued (steps past this wave's share read a valid block and are not
  // used), so the compiler's count of loads in flight is exact and a wait
  // for one tile never waits for a later one.
  __device__ __forceinline__ void load_tile(int tile, u32x4 (&w)[SPW]) const {
    bool second;
    const int r = row_at(tile, n, second);
    const uint8_t* W = reinterpret_cast<const uint8_t*>(second ? a.W2 : a.W) + size_t(r) * row_bytes;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      int b = 4 * (s0 + i) + g;
      b = b < G ? b : G - 1;   // padding blocks: any row bytes (their digits are zero)
      w[i] = ldg16(W + size_t(b) * 16);
    }
  }

  __device__ __forceinline__ void load_scales(int tile, uint32_t (&v)[NSL]) const {
    if constexpr (SL) {
#pragma unroll
      for (int k = 0; k < NSL; ++k) {
        const int rr = k * (64 / KL) + lane / KL;   // row of the tile
        bool second;
        const int r = row_at(tile, rr, second);
        int b = 4 * s0 + lane % KL;
        b = b < G ? b : G - 1;
        v[k] = reinterpret_cast<const uint16_t*>(second ? a.S2 : a.S)[size_t(r) * G + b];
      }
    } else {
      bool second;
      const int r = row_at(tile, n, second);
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        int b = 4 * (s0 + i) + g;
        b = b < G ? b : G - 1;
        v[i] = reinterpret_cast<const uint16_t*>(second ? a.S2 : a.S)[size_t(r) * G + b];
      }
    }
  }

  // the input groups of a quantizing thread (and, with NORM, the norm
  // weights); AGENT: with agent-scope loads, for an input other workgroups
  // of the same launch wrote
  template <bool AGENT = false>
  __device__ __forceinline__ void load_input(float4 (&xv)[GQ], uint4 (&gv)[GQ]) const {
    if constexpr (AGENT) {
      static_assert(!NORM, "agent-scope input without a norm");
      const int nf = a.cols / 4;
#pragma unroll
      for (int i = 0; i < GQ; ++i) {
        const int f = tid + 256 * i;
        const int fc = f < nf ? f : nf - 1;
        const float2 lo = load_pair_agent(a.in + 4 * fc);
        const float2 hi = load_pair_agent(a.in + 4 * fc + 2);
        xv[i] = make_float4(lo.x, lo.y, hi.x, hi.y);
      }
    } else if constexpr (!NORM) {
      q4mfma_load_input<false, 0, GQ>(a, tid, xv, gv);
    } else if (a.ntype == 1) {
      q4mfma_load_input<true, 1, GQ>(a, tid, xv, gv);
    } else {
      q4mfma_load_input<true, 0, GQ>(a, tid, xv, gv);
    }
  }

  // RMSNorm (fused epilogues), then the input as digits in LDS and the
  // tiles' scales staged; ends with a workgroup barrier
  __device__ __forceinline__ void prologue(const float4 (&xv)[GQ], const uint4 (&gv)[GQ],
                                           const uint32_t (&sv)[TT][NSL]) const {
    if (tid == 0) *reinterpret_cast<i32x4*>(zero16) = i32x4{0, 0, 0, 0};
    float r = 1.0f;
    if constexpr (NORM) {
      if (quant()) {
        const float ss = q4mfma_sumsq_regs<GQ>(xv, a.cols / 4, tid);
        if (lane == 0) ssq[wv] = ss;
      }
      __syncthreads();
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) ss += ssq[k];
      r = 1.0f / sqrtf(ss / float(a.cols) + a.eps);
    }
    if (quant()) {
      if constexpr (!NORM)
        q4mfma_quantize<false, 0, GQ>(a, r, xv, gv, dig, ex, GP, tid);
      else if (a.ntype == 1)
        q4mfma_quantize<true, 1, GQ>(a, r, xv, gv, dig, ex, GP, tid);
      else
        q4mfma_quantize<true, 0, GQ>(a, r, xv, gv, dig, ex, GP, tid);
    }
    if constexpr (SL) {
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int k = 0; k < NSL; ++k) {
          const int rr = k * (64 / KL) + lane / KL;
          const int j = lane % KL;
          if (j < KB) scl[(t * 16 + rr) * KB + j] = uint16_t(sv[t][k]);
        }
    }
    __syncthreads();
  }

  // tile `tile` (the workgroup's iter-th): products, sums over k-groups and
  // waves, epilogue (ends with the workgroup barrier of the wave sums)
  __device__ __forceinline__ void run_tile(int tile, int iter, const u32x4 (&w)[SPW], const uint32_t (&sr)[NSL],
                                           int pos) const {
    // the digit operand of this lane: block 4 s + g, digit p = n % 4 when
    // n / 4 == g and p < 3 (step i at a stride of four blocks); 16 zero
    // bytes otherwise
    const bool has_a = (n >> 2) == g && (n & 3) < 3;
    const uint8_t* abase = has_a ? dig + ((4 * s0 + g) * 3 + (n & 3)) * 32 : zero16;
    const int astride = has_a ? 4 * 3 * 32 : 0;
    const int ahalf = has_a ? 16 : 0;
    const int* exl = ex + 4 * s0 + g;
    const uint16_t* sl = scl + (iter * 16 + n) * KB + g;   // LDS mode, step i: block 4 i + g of row n
    float e0 = 0.0f, e1 = 0.0f;
    if (wv == 0 && lane < 8) PE::inputs(a, pos, tile * 8 + lane, e0, e1);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      if (i < ns) {
        const uint8_t* ap = abase + i * astride;
        const i32x4 A0 = *reinterpret_cast<const i32x4*>(ap);
        const i32x4 A1 = *reinterpret_cast<const i32x4*>(ap + ahalf);
        const int E = exl[4 * i];
        const u32x4 wi = w[i];
        const i32x4 B0 = {q4_lo16(wi.x), q4_hi16(wi.x), q4_lo16(wi.y), q4_hi16(wi.y)};
        const i32x4 B1 = {q4_lo16(wi.z), q4_hi16(wi.z), q4_lo16(wi.w), q4_hi16(wi.w)};
        i32x4 C = {0, 0, 0, 0};
        C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, B0, C, 0, 0, 0);
        C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, B1, C, 0, 0, 0);
        const float V = fmaf(float(C.z), 65536.0f, fmaf(float(C.y), 256.0f, float(C.x)));
        const uint16_t sbits = SL ? sl[4 * i] : uint16_t(sr[SL ? 0 : i]);
        acc = fmaf(ldexpf(__half2float(__ushort_as_half(sbits)), -E - 4), V, acc);
      }
    }
    // the four k-groups of row n, then the waves
    acc = pair_sum<16>(acc);
    acc = pair_sum<32>(acc);
    float* rb = red + (iter & 1) * NW * 16;
    if (lane < 16) rb[wv * 16 + n] = acc;
    __syncthreads();
    if (wv == 0 && lane < 16) {
      float y = rb[n];
#pragma unroll
      for (int k = 1; k < NW; ++k) y += rb[k * 16 + n];
      const float y1 = dpp_mov<0x128>(y);   // row n + 8 of the tile: the pair's second row
      if (lane < 8) PE::finish(a, pos, tile * 8 + lane, y, y1, e0, e1);
    }
  }
};

template <int EPI, int NW, int SPW, int TT>
__global__ __launch_bounds__(NW * 64) void q4mfma_kernel(GemvArgs a) {
  using T = Q4Tiles<EPI, NW, SPW, TT>;
  extern __shared__ __align__(16) uint8_t smem[];

  if (a.null_kernel) return;
  const T q(a, smem);

  // the input first (it returns before the weights), then the scales of the
  // workgroup's tiles and the weights of its first tile
  float4 xv[T::GQ];
  uint4 gv[T::GQ];
  if (q.quant()) q.load_input(xv, gv);
  const int tile0 = blockIdx.x * TT;
  uint32_t sv[TT][T::NSL];
#pragma unroll
  for (int t = 0; t < TT; ++t) q.load_scales(tile0 + t, sv[t]);
  u32x4 wq[TT][SPW];
  q.load_tile(tile0, wq[0]);   // the second tile's weights: once the input is quantized

  // the position (QKV epilogue) is checked once the first tile's weights are
  // requested: read first, its round trip delayed every request of the
  // workgroup (9B-shaped 4-bit stack +0.9% tokens/s)
  int pos = 0;
  if constexpr (EPI == EPI_QKV) {
    if (!qkv_pos_ok(a, pos)) return;
  }

  q.prologue(xv, gv, sv);

  // several tiles per workgroup: two tiles' weights in flight; a buffer is
  // refilled with the tile after next as soon as its tile is done
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (t + 1 < TT) q.load_tile(tile0 + t + 1, wq[t + 1]);
    q.run_tile(tile0 + t, t, wq[t], sv[t], pos);
  }
}

}  // namespace dec
