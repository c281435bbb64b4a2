// Small kernels: the per-op (unfused) steps of a layer, the RoPE table, and
// the per-token embedding gather and position advance.
#include "dec_device.h"
#include "dec_internal.h"
#include "dec_q4mfma.h"

namespace dec {

// RMSNorm of x (optionally times the norm weight) into `out`, one workgroup.
// The sum of squares is accumulated in the same lane order as the prologue
// of the fused kernels for the same weight type (f32/bf16: granules of `ge`
// elements, `ks` waves per row; 4-bit: the matrix-core kernel's order), so
// the per-op path rounds exactly like the fused one.
__global__ __launch_bounds__(kBlock) void rmsnorm_kernel(const float* x, const void* g, int ntype,
                                                         float* out, int n, float eps, int ge,
                                                         int ks, int with_weight, int null_kernel) {
  if (null_kernel) return;
  __shared__ float ssq[kWaves];
  __shared__ float rs;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  if (ge == 32) {
    const float ss = q4mfma_sumsq_part(reinterpret_cast<const float4*>(x), n / 4, threadIdx.x);
    if (lane == 0) ssq[wv] = ss;
    ks = kWaves;
  } else {
    const int G = n / ge;
    if (wv < ks) {
      float ss = 0.0f;
      for (int j = 0;; ++j) {
        const int gi = (j * ks + wv) * kWave + lane;
        if ((j * ks + wv) * kWave >= G) break;
        if (gi < G)
          for (int e = 0; e < ge; ++e) {
            const float v = x[gi * ge + e];
            ss = fmaf(v, v, ss);
          }
      }
      ss = wave_sum(ss);
      if (lane == 0) ssq[wv] = ss;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float ss;
    if (ks == 1) {
      ss = ssq[0];
    } else {
      ss = 0.0f;
      for (int k = 0; k < ks; ++k) ss += ssq[k];
    }
    rs = 1.0f / sqrtf(ss / float(n) + eps);
  }
  __syncthreads();
  const float r = rs;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    float v = x[i] * r;
    if (with_weight)
      v = v * (ntype == 1 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(g)[i])
                          : reinterpret_cast<const float*>(g)[i]);
    out[i] = v;
  }
}

__global__ void mul_kernel(float* u, const void* g, int ntype, int n, int null_kernel) {
  if (null_kernel) return;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n)
    u[i] = u[i] * (ntype == 1 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(g)[i])
                              : reinterpret_cast<const float*>(g)[i]);
}

// RoPE on q and k heads of y = Wqkv u, q written out, k and v appended.
__global__ void rope_append_kernel(const float* y, float* q, void* kc, void* vc,
                                   const int32_t* pos_p, const float* rope, uint32_t* err, int nq,
                                   int nkv, int d, int max_ctx, int kvtype, float* dbg_kv, int null_kernel) {
  if (null_kernel) return;
  const int pos = *pos_p;
  if (pos < 0 || pos >= max_ctx) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, kErrPos);
    return;
  }
  const int half = d / 2;
  const int task = blockIdx.x * blockDim.x + threadIdx.x;
  if (task >= (nq + 2 * nkv) * half) return;
  const int head = task / half, i = task % half;
  const int r0 = head * d + i;
  float y0 = y[r0], y1 = y[r0 + half];
  if (head < nq + nkv) {
    const float c = rope[(size_t(pos) * half + i) * 2];
    const float s = rope[(size_t(pos) * half + i) * 2 + 1];
    rope_rotate(y0, y1, c, s);
  }
  if (head < nq) {
    q[r0] = y0;
    q[r0 + half] = y1;
    return;
  }
  const bool isk = head < nq + nkv;
  const int j = isk ? head - nq : head - nq - nkv;
  if (dbg_kv) {   // the rows before rounding (debug export)
    float* dk = dbg_kv + (isk ? 0 : nkv * d) + j * d + i;
    dk[0] = y0;
    dk[half] = y1;
  }
  const size_t off = (size_t(j) * max_ctx + pos) * d + i;
  void* cache = isk ? kc : vc;
  if (kvtype == 2) {   // int8 cache: the row is staged as float, the attention appends it
    float* st = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(cache) + kv_i8_stage_off(nkv, max_ctx, d)) +
                size_t(j) * d + i;
    st[0] = y0;
    st[half] = y1;
  } else if (kvtype == 1) {
    uint16_t* c16 = reinterpret_cast<uint16_t*>(cache);
    c16[off] = f32_to_bf16(y0);
    c16[off + half] = f32_to_bf16(y1);
  } else {
    float* c32 = reinterpret_cast<float*>(cache);
    c32[off] = y0;
    c32[off + half] = y1;
  }
}

__global__ void swiglu_kernel(const float* g, const float* u, float* h, int n, int null_kernel) {
  if (null_kernel) return;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) h[i] = swiglu(g[i], u[i]);
}

// table[p][i] = (cos(p w_i), sin(p w_i)), w_i = theta^(-2i/d), in float64.
__global__ void rope_table_kernel(double theta, int d, int max_ctx, float* table) {
  const int half = d / 2;
  const long idx = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= long(max_ctx) * half) return;
  const int p = int(idx / half), i = int(idx % half);
  const double w = pow(theta, -2.0 * double(i) / double(d));
  const double phi = double(p) * w;
  table[idx * 2] = float(cos(phi));
  table[idx * 2 + 1] = float(sin(phi));
}

__global__ void embed_kernel(const float* embed, int vocab, int hidden, const int32_t* token,
                             float* x, uint32_t* err) {
  const int t = *token;
  const bool ok = t >= 0 && t < vocab;
  if (!ok && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, kErrToken);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < hidden; i += gridDim.x * blockDim.x)
    x[i] = ok ? embed[size_t(t) * hidden + i] : 0.0f;
}

__global__ void advance_kernel(int32_t* pos, int pos_lo, int pos_hi, const int32_t* tokens,
                               int32_t* token) {
  if (threadIdx.x != 0) return;
  int p = *pos + 1;
  if (p < pos_lo || p >= pos_hi) p = pos_lo;
  *pos = p;
  if (tokens) *token = tokens[p - pos_lo];
}

// Index of the largest value (the lowest index among equal maxima), one
// workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* v, int n, int32_t* out) {
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float x = v[i];
    if (x > best || (x == best && i < bi)) { best = x; bi = i; }
  }
  // wave reduction, then across the 16 waves in LDS
  for (int off = 32; off >= 1; off >>= 1) {
    const float ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  __shared__ float sb[16];
  __shared__ int si[16];
  const int wv = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) { sb[wv] = best; si[wv] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x / kWave); ++w)
      if (sb[w] > best || (sb[w] == best && si[w] < bi)) { best = sb[w]; bi = si[w]; }
    *out = bi;
  }
}

hipError_t launch_argmax(const float* v, int n, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3(1), dim3(1024), 0, s, v, n, out);
  return hipGetLastError();
}

static int ge_of(int wtype) { return wtype == 0 ? 4 : wtype == 1 ? 8 : 32; }

hipError_t launch_rmsnorm_like(const float* x, const void* g, int ntype, float* out, int n,
                               float eps, int wtype, int with_weight, int null_kernel,
                               hipStream_t s) {
  const int ge = ge_of(wtype);
  const int ks = gemv_ks(n, ge);
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(1), dim3(kBlock), 0, s, x, g, ntype, out, n, eps, ge, ks,
                     with_weight, null_kernel);
  return hipGetLastError();
}

hipError_t launch_mul(float* u, const void* g, int ntype, int n, int null_kernel, hipStream_t s) {
  hipLaunchKernelGGL(mul_kernel, dim3((n + 255) / 256), dim3(256), 0, s, u, g, ntype, n, null_kernel);
  return hipGetLastError();
}

hipError_t launch_rope_append(const float* y, float* q, void* kc, void* vc, const int32_t* pos,
                              const float* rope, uint32_t* err, int nq, int nkv, int d, int max_ctx,
                              int kvtype, float* dbg_kv, int null_kernel, hipStream_t s) {
  const int n = (nq + 2 * nkv) * d / 2;
  hipLaunchKernelGGL(rope_append_kernel, dim3((n + 255) / 256), dim3(256), 0, s, y, q, kc, vc, pos,
                     rope, err, nq, nkv, d, max_ctx, kvtype, dbg_kv, null_kernel);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* g, const float* u, float* h, int n, int null_kernel,
                         hipStream_t s) {
  hipLaunchKernelGGL(swiglu_kernel, dim3((n + 255) / 256), dim3(256), 0, s, g, u, h, n, null_kernel);
  return hipGetLastError();
}

hipError_t launch_rope_table(double theta, int d, int max_ctx, float* table, hipStream_t s) {
  const long n = long(max_ctx) * (d / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, theta, d,
                     max_ctx, table);
  return hipGetLastError();
}

hipError_t launch_embed(const float* embed, int vocab, int hidden, const int32_t* token, float* x,
                        uint32_t* err, hipStream_t s) {
  const int blocks = (hidden + 255) / 256;
  hipLaunchKernelGGL(embed_kernel, dim3(blocks), dim3(256), 0, s, embed, vocab, hidden, token, x, err);
  return hipGetLastError();
}

hipError_t launch_advance(int32_t* pos, int pos_lo, int pos_hi, const int32_t* tokens,
                          int32_t* token, hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, pos, pos_lo, pos_hi, tokens, token);
  return hipGetLastError();
}

}  // namespace dec
