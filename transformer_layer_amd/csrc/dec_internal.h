// Internal launch interface between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dec {

constexpr uint32_t kErrPos = 0x1u;
constexpr uint32_t kErrToken = 0x2u;
constexpr uint32_t kErrSync = 0x4u;
constexpr int kCounterStride = 16;  // uint32 words between two kv heads' arrival counters (64 bytes)

// Test-only arithmetic faults of the QKV epilogue (GemvArgs::fault): the
// kernels still run to completion and store in bounds, but the numbers are
// wrong, so a parity test must fail under each.
constexpr int kFaultSkipRope = 0x1;    // q and k left unrotated
constexpr int kFaultAppendNext = 0x2;  // k, v stored at position pos + 1 (pos itself when pos + 1 is past the cache)

// Sections of an int8 cache allocation (256-byte aligned): codes
// [nkv][max_ctx][d], one float scale per row [nkv][max_ctx], the newest row
// [nkv][d] as float (the QKV step writes it, the attention appends it).
__host__ __device__ constexpr size_t kv_align256(size_t n) { return (n + 255) / 256 * 256; }
__host__ __device__ constexpr size_t kv_i8_scale_off(int nkv, int max_ctx, int d) {
  return kv_align256(size_t(nkv) * max_ctx * d);
}
__host__ __device__ constexpr size_t kv_i8_stage_off(int nkv, int max_ctx, int d) {
  return kv_align256(kv_i8_scale_off(nkv, max_ctx, d) + size_t(nkv) * max_ctx * 4);
}
__host__ __device__ constexpr size_t kv_i8_bytes(int nkv, int max_ctx, int d) {
  return kv_i8_stage_off(nkv, max_ctx, d) + size_t(nkv) * d * 4;
}

// Arguments of the GEMV-core kernels (passed by value).
struct GemvArgs {
  const void* W;       // first matrix (elements)
  const void* S;       // its fp16 block scales (4-bit weights only)
  const void* W2;      // second matrix (gate/up pair) or null
  const void* S2;
  int rows;            // rows of the matrix / matrices
  int cols;            // input length
  int ntask;           // row pairs (the launcher turns them into tasks)
  const float* in;     // input vector [cols]
  const void* norm;    // RMSNorm weight [cols] (norm prologue only)
  int ntype;           // 0 f32, 1 bf16
  float eps;
  float* y;            // outputs, by epilogue
  float* y2;
  float* x;
  // QKV epilogue
  int nq, nkv, d, max_ctx, kvtype;   // kvtype 0 f32, 1 bf16, 2 int8 (staged as float)
  const int32_t* pos;
  const float* rope;
  void* kc;
  void* vc;
  uint32_t* err;
  int null_kernel;
  int fault;           // kFault* bits (tests of the parity gates only)
  float* dbg_kv;       // QKV epilogue: k [nkv][d] then v [nkv][d] as float32 before rounding, or null
};

// Granules (16-byte weight groups) per lane for a row of `cols` elements
// whose columns are split over `ks` waves.
inline int gemv_nj(int cols, int ge, int ks) {
  const int G = cols / ge;
  return (G + 64 * ks - 1) / (64 * ks);
}

// Waves that share one row (1, 2 or 4): the fewest that keep a lane's slice
// of the input vector within 16 registers; four when none does. The fused
// f32/bf16 kernels and the per-op RMSNorm both follow this rule, so they
// accumulate in the same order.
inline int gemv_ks(int cols, int ge) {
  for (int ks = 1; ks <= 4; ks *= 2)
    if (gemv_nj(cols, ge, ks) * ge <= 16) return ks;
  return 4;
}

// Four-bit GEMV on the matrix cores: waves per workgroup (4, or 8 when the
// projection has few 16-row tiles, so that more waves share each tile's
// steps of four 32-element blocks) and steps per wave (rounded up to 4, 8,
// 12 or 16). False when a wave would need more than 16 steps (cols > 16384).
inline bool q4mfma_plan(int cols, int ntiles, int* nw, int* spw) {
  const int steps = (cols / 32 + 3) / 4;
  int w = ntiles < 1024 ? 8 : 4;
  int per = (steps + w - 1) / w;
  if (per > 16 && w == 4) {
    w = 8;
    per = (steps + w - 1) / w;
  }
  if (per > 16) return false;
  *nw = w;
  *spw = per <= 4 ? 4 : per <= 8 ? 8 : per <= 12 ? 12 : 16;
  return true;
}

enum GemvEpi { kEpiStore = 0, kEpiResidual = 1, kEpiQkv = 2, kEpiSwiglu = 3, kEpiStore2 = 4, kEpiNormStore = 5 };

// The gated FFN with the down projection folded in (4-bit weights,
// dec_ffn_down.hip): f as for the gated FFN, dn as for the down projection
// (input f.y = h); bar = two zeroed counter words. Check: hipSuccess if the
// kernel can run the shape with every workgroup resident on this device,
// hipErrorInvalidValue for a shape outside its plans,
// hipErrorInvalidConfiguration when the workgroups would not all fit.
constexpr int kFfnDownBarWord = 2;   // words 2 and 3 of the first counter line
hipError_t ffn_down_q4_check(const GemvArgs& f, const GemvArgs& dn);
hipError_t launch_ffn_down_q4(const GemvArgs& f, const GemvArgs& dn, uint32_t* bar, int no_wait, hipStream_t s);

// Launch the GEMV core for weight type wtype (0 f32, 1 bf16, 2 q4).
hipError_t launch_gemv_f32(int epi, const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_bf16(int epi, const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_q4(int epi, const GemvArgs& a, hipStream_t s);

struct AttnArgs {
  const float* q;      // [n_q d]
  const void* kc;      // [n_kv][max_ctx][d]
  const void* vc;
  float* part;         // o [n_kv][S][g][d], then (m, l) [n_kv][S][g][2]
  uint32_t* counters;  // [n_kv * kCounterStride]
  float* out;          // [n_q d]
  const int32_t* pos;
  uint32_t* err;
  int nq, nkv, d, max_ctx, chunk, nsplit, kvtype;   // kvtype 0 f32, 1 bf16, 2 int8 rows + scales
  int waves;           // waves per workgroup (4 or 8)
  int kind;            // kAttnBatched, kAttnStream or kAttnLocal: which kernel runs
  int no_wait;         // combiners give up at once when splits are missing (failure-path tests)
  int partials_only;   // write the splits' partials and stop (the output projection combines them)
  int drop_last;       // test-only fault: the combine leaves out the last split (two or more splits)
  int null_kernel;
};

// The attention kernels: batched (dec_attn.hip: rows in registers in
// batches, one softmax per workgroup through LDS), streaming
// (dec_attn_stream.hip: keys scored as they arrive, values staged in LDS)
// and wave-local (dec_attn_local.hip: every row requested at launch, a
// softmax per wave, bf16 caches).
constexpr int kAttnDefault = -1, kAttnBatched = 0, kAttnStream = 1, kAttnLocal = 2;

// Attention chunk (positions per split), split count, waves per workgroup
// and kernel for a shape. kind_req picks the kernel (kAttnDefault: the
// library's choice for the shape), chunk_req the chunk (0: the kernel's
// default). False if the requested kernel cannot run the shape or chunk.
bool attn_plan(int n_q, int n_kv, int head_dim, int kvtype, int max_ctx, int chunk_req, int kind_req, int* chunk,
               int* nsplit, int* waves, int* kind);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);

// The wave-local kernel: kLocalWaves waves per workgroup, each with at most
// kLocalMaxSteps row loads of keys and of values in flight per lane.
constexpr int kLocalWaves = 8;
constexpr int kLocalMaxSteps = 9;
int attn_local_max_chunk(int head_dim, int kvtype);
hipError_t launch_attn_local(const AttnArgs& a, hipStream_t s);

// The streaming attention kernel: eight waves per workgroup; the longest
// chunk (a multiple of its row step) whose values, scores and scratch fit in
// one workgroup's LDS (0 if none does); planned for about kLdsTargetGroups
// workgroups (one per compute unit of an MI355X).
constexpr int kLdsWaves = 8;
constexpr int kLdsTargetGroups = 256;
constexpr int kStreamMinRows = 64;    // default chunks outside [min, max] rows
constexpr int kStreamMaxRows = 160;   // take the batched kernel
constexpr int kLdsBudget = 163840;   // LDS one workgroup may use on gfx950
int attn_lds_max_chunk(int n_q, int n_kv, int head_dim, int kvtype);
hipError_t launch_attn_lds(const AttnArgs& a, hipStream_t s);

// Attention combine fused into the output projection (bf16): x += Wo a, a
// combined from the partials of at most kAttnOSplits splits per kv head.
constexpr int kAttnOSplits = 32;
struct AttnOArgs {
  const float* part;   // the attention kernel's partials (layout of AttnArgs::part)
  const void* W;       // Wo, bf16 [rows][cols]
  float* x;            // [rows], updated with float atomics
  const int32_t* pos;
  int nq, nkv, d, rows, cols, nsplit, chunk, max_ctx;
  int drop_last;       // test-only fault: the combine leaves out the last split (two or more splits)
  int null_kernel;
};
bool attn_o_supported(int n_q, int n_kv, int head_dim, int nsplit);
hipError_t launch_attn_o(const AttnOArgs& a, hipStream_t s);

// small per-op and per-token kernels
// RMSNorm (optionally times its weight) with the fused kernels' summation
// order for weight type `wtype`.
hipError_t launch_rmsnorm_like(const float* x, const void* g, int ntype, float* out, int n,
                               float eps, int wtype, int with_weight, int null_kernel,
                               hipStream_t s);
hipError_t launch_mul(float* u, const void* g, int ntype, int n, int null_kernel, hipStream_t s);
hipError_t launch_rope_append(const float* y, float* q, void* kc, void* vc, const int32_t* pos,
                              const float* rope, uint32_t* err, int nq, int nkv, int d, int max_ctx,
                              int kvtype, float* dbg_kv, int null_kernel, hipStream_t s);
hipError_t launch_swiglu(const float* g, const float* u, float* h, int n, int null_kernel,
                         hipStream_t s);
hipError_t launch_rope_table(double theta, int d, int max_ctx, float* table, hipStream_t s);
hipError_t launch_embed(const float* embed, int vocab, int hidden, const int32_t* token, float* x,
                        uint32_t* err, hipStream_t s);
hipError_t launch_argmax(const float* v, int n, int32_t* out, hipStream_t s);
hipError_t launch_advance(int32_t* pos, int pos_lo, int pos_hi, const int32_t* tokens,
                          int32_t* token, hipStream_t s);

}  // namespace dec
