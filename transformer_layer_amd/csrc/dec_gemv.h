// Weight-streaming GEMV core shared by the fused projection kernels.
//
// A wavefront owns a column slice of the input vector in registers and
// streams whole 16-byte "granules" of weight rows with coalesced loads: lane
// l of a wave reads granule (j*KS + ks)*64 + l of a row, so each load
// instruction of the wave covers 1 KiB of contiguous weight bytes. A granule
// is 4 fp32 or 8 bf16 weights (4-bit weights have their own kernel, on the
// matrix cores). KS waves (1 or 4) of a workgroup
// share one task's rows by splitting the columns; their partial dot products
// meet in LDS. Each lane's dot product is reduced across the wave with DPP
// row operations.
//
// The prologue (PRO_NORM) computes RMSNorm of the input vector and applies
// the norm weight while staging the slice in registers, so the normalized
// vector never leaves the chip. The epilogue is selected by EPI:
//   EPI_STORE     y[r] = W u                                   (per-op path)
//   EPI_RESIDUAL  x[r] += W u                                  (O / down projection)
//   EPI_QKV       RoPE on the pair (i, i+d/2) of a head, then q written or k/v
//                 appended to the cache at position *pos    (QKV projection)
//   EPI_SWIGLU    h[j] = silu(Wg[j] u) * (Wu[j] u)             (gated FFN)
//   EPI_STORE2    y[j] = Wg[j] u, y2[j] = Wu[j] u              (per-op gate/up)
//   EPI_NORM_STORE  y[r] = W norm(x) (final RMSNorm + LM head logits)
//   EPI_SWIGLU_PUB  as EPI_SWIGLU, h stored with agent-scope stores, so that
//                 workgroups on other XCDs can read it in the same launch
//                 (the gated FFN with the down projection folded in)
#pragma once

#include "dec_device.h"
#include "dec_internal.h"

namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct WF32 { static constexpr int GE = 4; static constexpr int ID = 0; };
struct WBF16 { static constexpr int GE = 8; static constexpr int ID = 1; };

enum { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_QKV = 2, EPI_SWIGLU = 3, EPI_STORE2 = 4, EPI_NORM_STORE = 5,
       EPI_SWIGLU_PUB = 6 };

// epilogues whose prologue is the RMSNorm of the input
__host__ __device__ constexpr bool epi_has_norm(int epi) {
  return epi == EPI_QKV || epi == EPI_SWIGLU || epi == EPI_SWIGLU_PUB || epi == EPI_NORM_STORE;
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// partial dot product of one granule with the lane's input values
template <class T>
__device__ __forceinline__ float granule_dot(u32x4 w, const float* u, float acc);

template <>
__device__ __forceinline__ float granule_dot<WF32>(u32x4 w, const float* u, float acc) {
  acc = fmaf(__uint_as_float(w.x), u[0], acc);
  acc = fmaf(__uint_as_float(w.y), u[1], acc);
  acc = fmaf(__uint_as_float(w.z), u[2], acc);
  acc = fmaf(__uint_as_float(w.w), u[3], acc);
  return acc;
}

template <>
__device__ __forceinline__ float granule_dot<WBF16>(u32x4 w, const float* u, float acc) {
  acc = fmaf(bf_lo(w.x), u[0], acc);
  acc = fmaf(bf_hi(w.x), u[1], acc);
  acc = fmaf(bf_lo(w.y), u[2], acc);
  acc = fmaf(bf_hi(w.y), u[3], acc);
  acc = fmaf(bf_lo(w.z), u[4], acc);
  acc = fmaf(bf_hi(w.z), u[5], acc);
  acc = fmaf(bf_lo(w.w), u[6], acc);
  acc = fmaf(bf_hi(w.w), u[7], acc);
  return acc;
}

// GE norm-weight values of granule gi (f32 or bf16), with 16-byte loads.
template <int GE>
__device__ __forceinline__ void load_norm_granule(const void* g, int ntype, int gi, float* out) {
  if (ntype == 1) {
    const uint8_t* b = reinterpret_cast<const uint8_t*>(g) + size_t(gi) * GE * 2;
    if constexpr (GE == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(b);
      out[0] = bf_lo(v.x); out[1] = bf_hi(v.x); out[2] = bf_lo(v.y); out[3] = bf_hi(v.y);
    } else {
#pragma unroll
      for (int e = 0; e < GE; e += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(b + e * 2);
        out[e + 0] = bf_lo(v.x); out[e + 1] = bf_hi(v.x); out[e + 2] = bf_lo(v.y); out[e + 3] = bf_hi(v.y);
        out[e + 4] = bf_lo(v.z); out[e + 5] = bf_hi(v.z); out[e + 6] = bf_lo(v.w); out[e + 7] = bf_hi(v.w);
      }
    }
  } else {
    const float* f = reinterpret_cast<const float*>(g) + size_t(gi) * GE;
#pragma unroll
    for (int e = 0; e < GE; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(f + e);
      out[e] = v.x; out[e + 1] = v.y; out[e + 2] = v.z; out[e + 3] = v.w;
    }
  }
}

// Row pairs of a projection and what is done with their two dot products.
// Pair p is (r0, r1): a RoPE pair (i, i + d/2) of a head (QKV), a gate row
// and an up row of the same index (gated FFN, per-op gate/up), or two
// consecutive rows (everything else). Shared by every GEMV kernel, so a row
// is stored the same way whichever kernel computed it.
template <int EPI>
struct PairEpi {
  static constexpr bool PAIRED = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_PUB || EPI == EPI_STORE2);  // rows from two matrices
  static constexpr bool CONSEC = (EPI == EPI_STORE || EPI == EPI_RESIDUAL || EPI == EPI_NORM_STORE);

  static __device__ __forceinline__ int npairs(const GemvArgs& a) {
    return CONSEC ? (a.rows + 1) / 2 : a.rows / (PAIRED ? 1 : 2);
  }

  static __device__ __forceinline__ void rows(const GemvArgs& a, int p, int& r0, int& r1) {
    if constexpr (EPI == EPI_QKV) {
      const int half = a.d / 2;
      r0 = (p / half) * a.d + (p % half);
      r1 = r0 + half;
    } else if constexpr (PAIRED) {
      r0 = p;
      r1 = p;
    } else {
      r0 = 2 * p;
      r1 = r0 + 1;
    }
  }

  // inputs of pair p's epilogue that do not depend on the dot products (the
  // residual's old x values; RoPE's cos and sin), so they can be requested
  // before the dot products are done
  static __device__ __forceinline__ void inputs(const GemvArgs& a, int pos, int p, float& e0, float& e1) {
    if (p >= npairs(a)) return;
    int r0, r1;
    rows(a, p, r0, r1);
    if constexpr (EPI == EPI_RESIDUAL) {
      e0 = r0 < a.rows ? a.x[r0] : 0.0f;
      e1 = r1 < a.rows ? a.x[r1] : 0.0f;
    } else if constexpr (EPI == EPI_QKV) {
      const int half = a.d / 2;
      const int i = p % half;
      e0 = a.rope[(size_t(pos) * half + i) * 2];
      e1 = a.rope[(size_t(pos) * half + i) * 2 + 1];
    }
  }

  // the epilogue of pair p (run by one lane)
  static __device__ __forceinline__ void finish(const GemvArgs& a, int pos, int p, float y0, float y1, float e0,
                                                float e1) {
    if (p >= npairs(a)) return;
    int r0, r1;
    rows(a, p, r0, r1);
    const bool v0 = r0 < a.rows;
    const bool v1 = r1 < a.rows;
    if constexpr (EPI == EPI_STORE || EPI == EPI_NORM_STORE) {
      if (v0) a.y[r0] = y0;
      if (v1) a.y[r1] = y1;
    } else if constexpr (EPI == EPI_RESIDUAL) {
      if (v0) a.x[r0] = e0 + y0;
      if (v1) a.x[r1] = e1 + y1;
    } else if constexpr (EPI == EPI_SWIGLU) {
      a.y[r0] = swiglu(y0, y1);
    } else if constexpr (EPI == EPI_SWIGLU_PUB) {
      __hip_atomic_store(a.y + r0, swiglu(y0, y1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (EPI == EPI_STORE2) {
      a.y[r0] = y0;
      a.y2[r0] = y1;
    } else {  // EPI_QKV
      const int half = a.d / 2;
      const int head = p / half;
      const int i = p % half;
      if (head < a.nq + a.nkv && !(a.fault & kFaultSkipRope)) rope_rotate(y0, y1, e0, e1);
      if (head < a.nq) {
        a.y[r0] = y0;
        a.y[r1] = y1;
      } else {
        const bool isk = head < a.nq + a.nkv;
        const int j = isk ? head - a.nq : head - a.nq - a.nkv;
        if (a.dbg_kv) {   // the rows before rounding (debug export)
          float* dk = a.dbg_kv + (isk ? 0 : a.nkv * a.d) + j * a.d + i;
          dk[0] = y0;
          dk[half] = y1;
        }
        const int slot = (a.fault & kFaultAppendNext) && pos + 1 < a.max_ctx ? pos + 1 : pos;
        const size_t off = (size_t(j) * a.max_ctx + slot) * a.d + i;
        void* cache = isk ? a.kc : a.vc;
        if (a.kvtype == 2) {   // int8 cache: the row is staged as float, the attention appends it
          float* st = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(cache) +
                                               kv_i8_stage_off(a.nkv, a.max_ctx, a.d)) + size_t(j) * a.d + i;
          st[0] = y0;
          st[half] = y1;
        } else if (a.kvtype == 1) {
          uint16_t* c16 = reinterpret_cast<uint16_t*>(cache);
          c16[off] = f32_to_bf16(y0);
          c16[off + half] = f32_to_bf16(y1);
        } else {
          float* c32 = reinterpret_cast<float*>(cache);
          c32[off] = y0;
          c32[off + half] = y1;
        }
      }
    }
  }
};

// Position check of the QKV epilogue: the position the token is written at
// must lie in the cache. Returns false (and flags the error once) if not.
__device__ __forceinline__ bool qkv_pos_ok(const GemvArgs& a, int& pos) {
  pos = *a.pos;
  if (pos < 0 || pos >= a.max_ctx) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.err, kErrPos);
    return false;
  }
  return true;
}

// One task is NP row pairs (NR = 2 NP rows): a RoPE pair (i, i + d/2) of a
// head (QKV), a gate row and an up row (gated FFN), or two consecutive rows.
// PF: the next task's weights are requested before the current task is
// reduced (more bytes in flight per wave, more registers).
// Resident waves per SIMD the compiler must keep for bf16 weights (a
// register budget that holds without spills; the lane's input slice of
// NJ * 8 floats dominates the register use). Other weight types are left to
// the compiler.
template <class T, int NJ, int KS, int EPI>
constexpr int gemv_min_waves() {
  if (T::ID != 1) return 1;
  if (NJ <= 2) return (EPI == EPI_RESIDUAL || EPI == EPI_QKV) ? 4 : 5;
  if (NJ <= 6) return (KS == 4 && EPI != EPI_QKV) ? 3 : 2;
  return 2;
}

template <class T, int NJ, int KS, int EPI, int NP, bool PF>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(gemv_min_waves<T, NJ, KS, EPI>())))
void gemv_kernel(GemvArgs a) {
  constexpr int GE = T::GE;
  constexpr int NR = 2 * NP;  // rows per task
  constexpr bool NORM = epi_has_norm(EPI);
  using PE = PairEpi<EPI>;
  constexpr bool PAIRED = PE::PAIRED;
  constexpr int TPW = kWaves / KS;  // tasks per workgroup iteration

  if (a.null_kernel) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform: row addresses stay scalar
  const int ks = wv % KS;
  const int slot = wv / KS;

  const int G = a.cols / GE;  // granules per row
  const size_t row_bytes = size_t(a.cols) * (T::ID == 0 ? 4 : 2);
  const int npairs = PE::npairs(a);
  const uint8_t* Wa = reinterpret_cast<const uint8_t*>(a.W);
  const uint8_t* Wb = PAIRED ? reinterpret_cast<const uint8_t*>(a.W2) : Wa;

  // weights of a task's rows. Loads are never
  // predicated: a granule past the row end reads the row's last granule
  // (its input values are zero) and a row past the matrix reads the last row
  // (its result is never stored).
  auto load_task = [&](int task, u32x4 (&wq)[NR][NJ]) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      int p = task * NP + q;
      p = p < npairs ? p : npairs - 1;
      int r0, r1;
      PE::rows(a, p, r0, r1);
      r0 = r0 < a.rows ? r0 : a.rows - 1;
      r1 = r1 < a.rows ? r1 : a.rows - 1;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        int gi = (j * KS + ks) * kWave + lane;
        gi = gi < G ? gi : G - 1;
        wq[2 * q][j] = ldg16(Wa + size_t(r0) * row_bytes + size_t(gi) * 16);
        wq[2 * q + 1][j] = ldg16(Wb + size_t(r1) * row_bytes + size_t(gi) * 16);
      }
    }
  };

  // the first task's weights do not depend on the input: fetch them while
  // the prologue reads and normalizes the input vector
  const int stride = gridDim.x * TPW;
  u32x4 wq[NR][NJ];
  load_task(blockIdx.x * TPW + slot, wq);


  // ---- prologue: this lane's slice of the input vector, in registers. The
  // norm weights are requested together with it when they fit in registers
  // (they do not depend on the sum of squares).
  // In the QKV kernel with bf16 weights the norm weights arrive as raw bits
  // (16 bytes of bf16 or 32 bytes of f32 per granule) from unconditional
  // loads and are converted after the sum of squares: converted at the load,
  // inside a branch on their type, each granule made the compiler wait for
  // every load in flight (the first task's weights included) before the next
  // input granule was requested (9B-shaped QKV 10.4 -> 9.5 us). The gated
  // FFN keeps the conversion at the load: with everything requested at once
  // it ended 0.2-0.3 us later (measured on the 7B/9B shapes).
  constexpr bool EARLY_NORM = NORM && NJ * GE <= 32;
  constexpr bool RAW_NORM = EARLY_NORM && GE == 8 && EPI == EPI_QKV;
  float u[NJ][GE];
  float gw[EARLY_NORM && !RAW_NORM ? NJ : 1][EARLY_NORM && !RAW_NORM ? GE : 1];
  u32x4 nr[RAW_NORM ? NJ : 1][2];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int gi = (j * KS + ks) * kWave + lane;
    const bool ok = gi < G;
    const int gc = ok ? gi : G - 1;
#pragma unroll
    for (int e = 0; e < GE; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(a.in + size_t(gc) * GE + e);
      u[j][e] = ok ? v.x : 0.0f; u[j][e + 1] = ok ? v.y : 0.0f;
      u[j][e + 2] = ok ? v.z : 0.0f; u[j][e + 3] = ok ? v.w : 0.0f;
    }
    if constexpr (RAW_NORM) {
      const uint8_t* nb = reinterpret_cast<const uint8_t*>(a.norm);
      const bool bf = a.ntype == 1;
      const size_t o0 = size_t(gc) * (bf ? 16 : 32);
      nr[j][0] = *reinterpret_cast<const u32x4*>(nb + o0);
      nr[j][1] = *reinterpret_cast<const u32x4*>(nb + o0 + (bf ? 0 : 16));
    } else if constexpr (EARLY_NORM) {
      load_norm_granule<GE>(a.norm, a.ntype, gc, gw[j]);
    }
  }
  if constexpr (NORM) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < GE; ++e) ss = fmaf(u[j][e], u[j][e], ss);
  }
  constexpr int kBatch = 16;  // tasks per LDS batch (column-split waves)
  static_assert(kBatch * NP <= kWave, "one batch item per lane of the finishing wave");
  __shared__ float red[KS > 1 ? kWaves : 1][KS > 1 ? kBatch : 1][NR];
  __shared__ float ssq[kWaves];
  if constexpr (NORM) {
    ss = wave_sum(ss);
    if constexpr (KS > 1) {
      if (lane == 0) ssq[wv] = ss;
      __syncthreads();
      ss = 0.0f;
#pragma unroll
      for (int k = 0; k < KS; ++k) ss += ssq[slot * KS + k];
    }
    const float r = 1.0f / sqrtf(ss / float(a.cols) + a.eps);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int gi = (j * KS + ks) * kWave + lane;
      float g[GE];
      if constexpr (RAW_NORM) {
        const u32x4 w0 = nr[j][0], w1 = nr[j][1];
        if (a.ntype == 1) {
          g[0] = bf_lo(w0.x); g[1] = bf_hi(w0.x); g[2] = bf_lo(w0.y); g[3] = bf_hi(w0.y);
          g[4] = bf_lo(w0.z); g[5] = bf_hi(w0.z); g[6] = bf_lo(w0.w); g[7] = bf_hi(w0.w);
        } else {
          g[0] = __uint_as_float(w0.x); g[1] = __uint_as_float(w0.y);
          g[2] = __uint_as_float(w0.z); g[3] = __uint_as_float(w0.w);
          g[4] = __uint_as_float(w1.x); g[5] = __uint_as_float(w1.y);
          g[6] = __uint_as_float(w1.z); g[7] = __uint_as_float(w1.w);
        }
      } else if constexpr (EARLY_NORM) {
#pragma unroll
        for (int e = 0; e < GE; ++e) g[e] = gw[j][e];
      } else {
        load_norm_granule<GE>(a.norm, a.ntype, gi < G ? gi : G - 1, g);
      }
#pragma unroll
      for (int e = 0; e < GE; ++e) u[j][e] = (u[j][e] * r) * g[e];   // u is 0 past the row end
    }
  }
  // the position (QKV epilogue) is checked once the first task's weights and
  // the input slice are requested: read first, its round trip delayed every
  // load of the workgroup
  int pos = 0;
  if constexpr (EPI == EPI_QKV) {
    if (!qkv_pos_ok(a, pos)) return;
  }
  auto epi_inputs = [&](int p, float& e0, float& e1) { PE::inputs(a, pos, p, e0, e1); };
  auto epilogue = [&](int p, float y0, float y1, float e0, float e1) { PE::finish(a, pos, p, y0, y1, e0, e1); };

  // ---- tasks: this wave slot handles task, task + stride, ...
  int nb = 0;                         // tasks in the current LDS batch
  int batch_base = blockIdx.x * TPW;  // base of its first task
  constexpr bool EPI_IN = (EPI == EPI_RESIDUAL || EPI == EPI_QKV);
  // Epilogue inputs of the pair this lane finishes (ex) and of the next
  // task's (exn). They are requested one task ahead, together with that
  // task's weights, so the wait for the weights covers them: requested at
  // the start of their own task, the wait for the weights right after would
  // wait for them too, an L2 round trip per task.
  float ex0 = 0.0f, ex1 = 0.0f, exn0 = 0.0f, exn1 = 0.0f;
  // the lane that finishes pair q of task t (batch item bi) requests its inputs
  auto epi_request = [&](int t, int bi) {
    if constexpr (KS == 1) {
      if (lane < NP && t < a.ntask) epi_inputs(t * NP + lane, exn0, exn1);
    } else {
      const int q = lane - bi * NP;
      if (ks == 0 && q >= 0 && q < NP && t < a.ntask) epi_inputs(t * NP + q, exn0, exn1);
    }
  };
  if constexpr (EPI_IN) epi_request(blockIdx.x * TPW + slot, 0);
  for (int base = blockIdx.x * TPW; base < a.ntask; base += stride) {
    const int task = base + slot;
    const bool more = base + stride < a.ntask;
    // a lane's exn holds the inputs of the batch item it finishes next; for
    // every other lane exn and ex are already equal
    if constexpr (EPI_IN) {
      ex0 = exn0;
      ex1 = exn1;
    }
    // batch item of the next task (KS > 1: a batch is finished after kBatch tasks)
    const int nb_next = (KS > 1 && nb + 1 == kBatch) ? 0 : nb + 1;
    u32x4 wn[PF ? NR : 1][NJ];
    if constexpr (PF) {
      if (more) {
        load_task(task + stride, wn);
        if constexpr (EPI_IN) epi_request(task + stride, nb_next);
      }
    }

    float acc[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[k] = granule_dot<T>(wq[k][j], u[j], acc[k]);
    if constexpr (PF) {
      if (more) {
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
          for (int j = 0; j < NJ; ++j) wq[k][j] = wn[k][j];
      }
    } else {
      if (more) {
        load_task(task + stride, wq);
        if constexpr (EPI_IN) epi_request(task + stride, nb_next);
      }
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) acc[k] = wave_sum(acc[k]);
    if constexpr (KS == 1) {
      if (lane < NP) {
        // lane q finishes pair q of the task
        float y0 = acc[0], y1 = acc[1];
#pragma unroll
        for (int q = 1; q < NP; ++q)
          if (lane == q) { y0 = acc[2 * q]; y1 = acc[2 * q + 1]; }
        if (task < a.ntask) epilogue(task * NP + lane, y0, y1, ex0, ex1);
      }
    } else {
      // partial sums of the KS waves meet in LDS; finished in batches so the
      // waves do not meet at a barrier for every task
      if (lane == 0) {
#pragma unroll
        for (int k = 0; k < NR; ++k) red[wv][nb][k] = acc[k];
      }
      ++nb;
      if (nb == kBatch || !more) {
        __syncthreads();
        if (ks == 0 && lane < nb * NP) {   // nb * NP <= kBatch * 2 < kWave: one item per lane
          const int bi = lane / NP, q = lane % NP;
          const int t = batch_base + bi * stride + slot;
          float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            s0 += red[slot * KS + k][bi][2 * q];
            s1 += red[slot * KS + k][bi][2 * q + 1];
          }
          if (t < a.ntask) epilogue(t * NP + q, s0, s1, ex0, ex1);
        }
        __syncthreads();
        nb = 0;
        batch_base = base + stride;
      }
    }
  }
}

// Workgroups that one kernel keeps resident on the current device
// (occupancy x compute units) for a block size and dynamic LDS size, cached
// per (device, kernel, LDS size): every instantiation has its own register
// use and so its own occupancy.
template <class K>
inline int resident_blocks(K kernel, int block = kBlock, int lds = 0) {
  struct Entry { const void* fn; int dev; int lds; int cap; };
  static thread_local Entry cache[256];
  static thread_local int used = 0;
  const void* fn = reinterpret_cast<const void*>(kernel);
  int dev = 0;
  (void)hipGetDevice(&dev);
  for (int i = 0; i < used; ++i)
    if (cache[i].fn == fn && cache[i].dev == dev && cache[i].lds == lds) return cache[i].cap;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  const int cap = per_cu * cus;
  if (used < 256) cache[used++] = Entry{fn, dev, lds, cap};
  return cap;
}

// Compute units of the current device (cached per device).
inline int device_cus() {
  static thread_local int cache[64] = {0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// Workgroups for `groups` task groups of a GEMV. Workgroup b takes groups b,
// b + grid, ...; consecutive workgroups land on different compute units, so
// with a grid that is a whole number of workgroups per compute unit every
// compute unit gets the same number of groups to within one.
//   per_cu > 0: at most per_cu workgroups per compute unit (and at most the
//               resident occupancy);
//   per_cu = 0: the resident occupancy;
//   per_cu < 0: the resident occupancy cut down so that every workgroup has
//               the same number of groups.
// Measured per kernel on the 1B/7B/9B layer shapes (last workgroup's end):
// residual GEMVs over long rows finish sooner with one (<= 8192 columns) or
// two workgroups per compute unit (9B down projection 19.1 -> 18.0 us, 7B
// 18.9 -> 17.7, 1B 8.0 -> 6.9), the gated FFN with the whole occupancy as a
// whole number per compute unit (7B 30.1 -> 28.4 us, 9B 30.8 -> 30.2), the
// QKV projection with equal groups per workgroup.
template <class K>
inline int gemv_grid(K kernel, int groups, int per_cu) {
  int cap = resident_blocks(kernel);
  if (per_cu < 0) {
    const int per_wg = (groups + cap - 1) / cap;
    return (groups + per_wg - 1) / per_wg;
  }
  if (per_cu > 0 && per_cu * device_cus() < cap) cap = per_cu * device_cus();
  return groups < cap ? groups : cap;
}

// workgroups per compute unit of a GEMV launch (see gemv_grid)
template <int EPI>
inline int gemv_per_cu(int cols) {
  if constexpr (EPI == EPI_QKV) return -1;
  if constexpr (EPI == EPI_RESIDUAL) return cols <= 8192 ? 1 : 2;
  return 0;
}

}  // namespace dec
