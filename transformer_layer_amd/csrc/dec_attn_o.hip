// Attention combine fused into the output projection (bf16 weights and
// cache): x += Wo a, where a is combined here from the split-K attention's
// partials instead of by the attention kernel's last workgroups.
//
// Workgroup (cb, rb) owns column block cb of Wo (C columns: C / d whole
// query heads of one kv head j's group) and a block of R output rows. It
// requests, in this order, the (max, sum) partials of its heads' splits,
// their unnormalized outputs for its columns, and its Wo block (R rows x C
// columns), so that waiting for the partials never waits for the weights
// (loads complete in order). It then forms its heads' attention output
//   a_c = sum_s w_s o_s,c,  w_s = exp2(m_s - M) / sum_s' exp2(m_s' - M) l_s'
// (M the largest split max of the head, scores in log2 units) in LDS, takes
// the dot products of its rows with it, and adds them to x with float
// atomics: the column blocks of a row add in no fixed order. The combine's
// latency is spent while the weights stream, instead of as a chain of round
// trips at the end of the attention kernel.
#include "dec_device.h"
#include "dec_internal.h"

namespace dec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int C, int NL, int NO>
__global__ __launch_bounds__(512) void attn_o_kernel(AttnOArgs a) {
  constexpr int NW = 8, NT = 512;
  constexpr int LPR = C / 8;             // lanes per Wo row (bf16 granules of 8 columns)
  constexpr int RPW = 64 / LPR;          // rows per wave load
  constexpr int R = NL * RPW * NW;       // rows per workgroup
  constexpr int CG = C / 4;              // float4 column groups of the block
  constexpr int SL = NT / CG;            // threads per column group (each a subset of the splits)
  // NO partial-output loads per thread: NO * SL >= the plan's split count
  static_assert(LPR >= 8 && LPR <= 64 && SL >= 1 && NO >= 1 && NO * SL <= kAttnOSplits, "shape");

  if (a.null_kernel) return;
  const int ncb = a.cols / C;            // column blocks
  const int cb = blockIdx.x % ncb;
  const int rb = blockIdx.x / ncb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int g = a.nq / a.nkv;            // query heads per kv head
  const int Cg = g * a.d;                // columns of a kv head's group
  const int c0 = cb * C;                 // first column of the block
  const int j = c0 / Cg;                 // its kv head
  const int co = c0 - j * Cg;            // offset inside the group
  const int hb = co / a.d;               // first head of the block inside the group
  const int HB = C / a.d;                // heads in the block
  const int last = a.nsplit - 1;

  // (max, sum) of split s for head hb + h: thread t takes (h, s) =
  // (t / 32, t % 32) (threads past HB*32 repeat a valid pair, unused)
  const float* pml = a.part + size_t(a.nkv) * a.nsplit * Cg + size_t(j) * a.nsplit * g * 2;
  const int ml_t = tid % (HB * kAttnOSplits);
  const int ml_h = ml_t / kAttnOSplits, ml_s = ml_t % kAttnOSplits;
  const float2 ml = *reinterpret_cast<const float2*>(pml + (size_t(min(ml_s, last)) * g + hb + ml_h) * 2);

  // unnormalized outputs: thread t takes column group t % CG and splits
  // t / CG, + SL, ... (clamped to the splits the buffer holds)
  const int cg = tid % CG, sl = tid / CG;
  const float* po = a.part + size_t(j) * a.nsplit * Cg + co;
  float4 ov[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int s = min(sl + k * SL, last);
    ov[k] = *reinterpret_cast<const float4*>(po + size_t(s) * Cg + cg * 4);
  }

  // this workgroup's Wo rows: lane (sub, li) of wave wv takes rows
  // r0 + wv*NL*RPW + u*RPW + sub, columns c0 + li*8 .. +7 (c0 = cb*C)
  const int sub = lane / LPR, li = lane % LPR;
  const int r0 = rb * R + wv * NL * RPW + sub;
  const uint8_t* W = reinterpret_cast<const uint8_t*>(a.W);
  u32x4 wq[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int r = min(r0 + u * RPW, a.rows - 1);
    wq[u] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(W + (size_t(r) * a.cols + c0 + li * 8) * 2));
  }

  // the position decides which splits hold cache rows
  const int pos = *a.pos;
  if (pos < 0 || pos >= a.max_ctx) return;   // the attention kernel flagged it and wrote nothing
  int ns = (pos + a.chunk) / a.chunk;        // splits over positions 0..pos
  if (a.drop_last && ns > 1) --ns;           // (tests of the parity gates: the last split left out)

  __shared__ float wts[8][kAttnOSplits];      // per head and split: exp2(m - M) / den
  __shared__ float4 red[NT];
  __shared__ float av[C];

  // weights: groups of 32 lanes hold one head's splits
  {
    const bool ok = ml_s < ns;
    const float m = ok ? ml.x : -INFINITY;
    const float M = group_max<32>(m);
    const float w = ok ? exp2f(ml.x - M) : 0.0f;
    const float den = group_sum<32>(ok ? w * ml.y : 0.0f);  // >= 1: the split holding M adds l >= 1
    if (tid < HB * kAttnOSplits) wts[ml_h][ml_s] = w / den;
  }
  __syncthreads();
  {
    const int h = (cg * 4) / a.d;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < NO; ++k) {
      // splits past ns hold whatever an earlier token (or nothing) left
      // there: skipped, so that no stale value reaches the sum as 0 * inf
      const bool live = sl + k * SL < ns;
      const float w = live ? wts[h][sl + k * SL] : 0.0f;
      const float4 o = live ? ov[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      acc.x = fmaf(w, o.x, acc.x); acc.y = fmaf(w, o.y, acc.y);
      acc.z = fmaf(w, o.z, acc.z); acc.w = fmaf(w, o.w, acc.w);
    }
    red[tid] = acc;
  }
  __syncthreads();
  if (tid < CG) {
    float4 s4 = red[tid];
#pragma unroll
    for (int k = 1; k < SL; ++k) {
      const float4 v = red[k * CG + tid];
      s4.x += v.x; s4.y += v.y; s4.z += v.z; s4.w += v.w;
    }
    av[tid * 4] = s4.x; av[tid * 4 + 1] = s4.y; av[tid * 4 + 2] = s4.z; av[tid * 4 + 3] = s4.w;
  }
  __syncthreads();

  // dot products of this lane's rows with its eight columns, summed over the
  // row's lanes, staged in LDS (the workgroup's rows are contiguous) and
  // added to x by consecutive threads, so that the atomics coalesce
  __shared__ float rsum[R];
  float u8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) u8[e] = av[li * 8 + e];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const u32x4 w = wq[u];
    float acc = 0.0f;
    acc = fmaf(bf_lo(w.x), u8[0], acc); acc = fmaf(bf_hi(w.x), u8[1], acc);
    acc = fmaf(bf_lo(w.y), u8[2], acc); acc = fmaf(bf_hi(w.y), u8[3], acc);
    acc = fmaf(bf_lo(w.z), u8[4], acc); acc = fmaf(bf_hi(w.z), u8[5], acc);
    acc = fmaf(bf_lo(w.w), u8[6], acc); acc = fmaf(bf_hi(w.w), u8[7], acc);
    acc = group_sum<LPR>(acc);
    if (li == 0) rsum[wv * NL * RPW + u * RPW + sub] = acc;
  }
  __syncthreads();
  for (int i = tid; i < R; i += NT) {
    const int r = rb * R + i;
    if (r < a.rows) atomicAdd(a.x + r, rsum[i]);
  }
}

// rows per lane: the most (16, 8 or 4) that still gives every CU one
// workgroup, or two for column blocks of at most 128 columns. Every
// workgroup re-reads its block's partials (nsplit x C floats), so halving
// the row block pays only where those are small next to the weights:
// 7B-shaped layer (128 columns, 22 splits) 374.7 -> 377.1 tokens/s with two,
// 9B-shaped with 512-column blocks 311.0 -> 302.8 (same-box A/B).
static int attn_o_nl(int rows, int ncb, int C) {
  const int rpw = 64 / (C / 8);
  const int want = C <= 128 ? 512 : 256;
  for (int nl : {16, 8, 4}) {
    const int per_wg = nl * rpw * 8;
    if (ncb * ((rows + per_wg - 1) / per_wg) >= want) return nl;
  }
  return 4;
}

// columns per workgroup: one query head when heads are 128+ wide, else the
// kv head's whole group. Narrow blocks re-read fewer partials per
// workgroup but add more atomics per x element: one 128-wide head instead
// of the 512-column group, 9B-shaped layer 314.8 -> 318.0 tokens/s; one
// 64-wide head instead of the 256-column group, 1B-shaped 1692 -> 1655
// (same-box A/B).
static int attn_o_cols(int n_q, int n_kv, int head_dim) {
  return head_dim >= 128 ? head_dim : (n_q / n_kv) * head_dim;
}

bool attn_o_supported(int n_q, int n_kv, int head_dim, int nsplit) {
  if (n_kv <= 0 || n_q % n_kv || nsplit > kAttnOSplits) return false;
  const int g = n_q / n_kv, C = attn_o_cols(n_q, n_kv, head_dim);
  return (C == 64 || C == 128 || C == 256 || C == 512) && (g * head_dim) % C == 0 && C / head_dim <= 8;
}

template <int C, int NL, int NO>
static void go_attn_o_no(const AttnOArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_o_kernel<C, NL, NO>), grid, dim3(512), 0, s, a);
}

// partial-output loads per thread: the fewest that cover the plan's splits
// (splits past the last would only re-read it)
template <int C, int NL>
static hipError_t go_attn_o_nl(const AttnOArgs& a, dim3 grid, hipStream_t s) {
  constexpr int SL = 512 / (C / 4);
  const int no = (a.nsplit + SL - 1) / SL;
  switch (no) {
    case 1: go_attn_o_no<C, NL, 1>(a, grid, s); break;
    case 2: if constexpr (2 * SL <= kAttnOSplits) { go_attn_o_no<C, NL, 2>(a, grid, s); break; } return hipErrorInvalidValue;
    case 3: if constexpr (3 * SL <= kAttnOSplits) { go_attn_o_no<C, NL, 3>(a, grid, s); break; } return hipErrorInvalidValue;
    case 4: if constexpr (4 * SL <= kAttnOSplits) { go_attn_o_no<C, NL, 4>(a, grid, s); break; } return hipErrorInvalidValue;
    case 5: if constexpr (5 * SL <= kAttnOSplits) { go_attn_o_no<C, NL, 5>(a, grid, s); break; } return hipErrorInvalidValue;
    case 6: if constexpr (6 * SL <= kAttnOSplits) { go_attn_o_no<C, NL, 6>(a, grid, s); break; } return hipErrorInvalidValue;
    case 7: if constexpr (7 * SL <= kAttnOSplits) { go_attn_o_no<C, NL, 7>(a, grid, s); break; } return hipErrorInvalidValue;
    case 8: if constexpr (8 * SL <= kAttnOSplits) { go_attn_o_no<C, NL, 8>(a, grid, s); break; } return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int C>
static hipError_t go_attn_o(const AttnOArgs& a, hipStream_t s) {
  const int ncb = a.cols / C;
  const int nl = attn_o_nl(a.rows, ncb, C);
  const int rpw = 64 / (C / 8);
  const int per_wg = nl * rpw * 8;
  const dim3 grid(ncb * ((a.rows + per_wg - 1) / per_wg));
  if (nl == 16) return go_attn_o_nl<C, 16>(a, grid, s);
  if (nl == 8) return go_attn_o_nl<C, 8>(a, grid, s);
  return go_attn_o_nl<C, 4>(a, grid, s);
}

hipError_t launch_attn_o(const AttnOArgs& a, hipStream_t s) {
  if (!attn_o_supported(a.nq, a.nkv, a.d, a.nsplit)) return hipErrorInvalidValue;
  switch (attn_o_cols(a.nq, a.nkv, a.d)) {
    case 64: return go_attn_o<64>(a, s);
    case 128: return go_attn_o<128>(a, s);
    case 256: return go_attn_o<256>(a, s);
    case 512: return go_attn_o<512>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec
