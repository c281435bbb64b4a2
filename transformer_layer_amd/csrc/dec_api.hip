// C ABI of libdec: argument checks, launch planning, error reporting.
// Every entry point validates on the host, then only enqueues kernels on the
// caller's stream: no allocation, no synchronization, no device reads.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/dec_api.h"
#include "dec_internal.h"

namespace {

thread_local char g_err[256] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DEC_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return DEC_OK;
}

int64_t pad4(int64_t n) { return (n + 3) / 4 * 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// the kernels' cache type: 0 f32, 1 bf16, 2 int8 rows with a scale each
int kv_kind(const dec_layer_desc* d) { return d->kvtype == DEC_BF16 ? 1 : d->kvtype == DEC_I8 ? 2 : 0; }

int ge_of(int wtype) { return wtype == DEC_F32 ? 4 : wtype == DEC_BF16 ? 8 : 32; }

// The attention plan of a layer shape: the kernel DEC_ATTN_* in its flags
// asks for (the library's choice without one) and its chunk, split count
// and waves. Every entry point plans through here, so the partials' layout,
// the kernel and the output projection's combine always agree.
bool attn_plan_of(const dec_layer_desc* d, int* chunk, int* ns, int* nw, int* kind) {
  int req = dec::kAttnDefault;
  switch (d->flags & DEC_ATTN_KERNEL_MASK) {
    case DEC_ATTN_BATCHED: req = dec::kAttnBatched; break;
    case DEC_ATTN_STREAM: req = dec::kAttnStream; break;
    case DEC_ATTN_LOCAL: req = dec::kAttnLocal; break;
    default: break;
  }
  return dec::attn_plan(d->n_q_heads, d->n_kv_heads, d->head_dim, kv_kind(d), d->max_ctx,
                        d->attn_chunk, req, chunk, ns, nw, kind);
}

int check_desc(const dec_layer_desc* d) {
  if (!d) return fail(DEC_E_NULL, "desc is NULL");
  if (d->wtype < DEC_F32 || d->wtype > DEC_Q4) return fail(DEC_E_DTYPE, "wtype %d", d->wtype);
  if (d->ntype != DEC_F32 && d->ntype != DEC_BF16) return fail(DEC_E_DTYPE, "ntype %d", d->ntype);
  if (d->kvtype != DEC_F32 && d->kvtype != DEC_BF16 && d->kvtype != DEC_I8) return fail(DEC_E_DTYPE, "kvtype %d", d->kvtype);
  if (d->head_dim != 64 && d->head_dim != 128) return fail(DEC_E_SHAPE, "head_dim %d (64 or 128)", d->head_dim);
  if (d->kvtype == DEC_I8 && d->head_dim != 128)
    return fail(DEC_E_SHAPE, "int8 cache needs head_dim 128 (got %d)", d->head_dim);
  if (d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->n_q_heads % d->n_kv_heads)
    return fail(DEC_E_SHAPE, "heads %d/%d", d->n_q_heads, d->n_kv_heads);
  const int g = d->n_q_heads / d->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return fail(DEC_E_SHAPE, "group %d (1, 2, 4 or 8)", g);
  const int ge = ge_of(d->wtype);
  const int qd = d->n_q_heads * d->head_dim;
  for (int c : {d->hidden, d->ffn, qd})
    if (c <= 0 || c % ge || c > 16384) return fail(DEC_E_SHAPE, "length %d (multiple of %d, <= 16384)", c, ge);
  if (d->max_ctx <= 0 || d->max_ctx > (1 << 20)) return fail(DEC_E_SHAPE, "max_ctx %d", d->max_ctx);
  if (!(d->rms_eps >= 0.0f)) return fail(DEC_E_SHAPE, "rms_eps");
  if (d->attn_chunk < 0 || d->attn_chunk > 256) return fail(DEC_E_SHAPE, "attn_chunk %d (0..256)", d->attn_chunk);
  int chunk, ns, nw, kind;
  if (!attn_plan_of(d, &chunk, &ns, &nw, &kind)) {
    if (ns > 256) return fail(DEC_E_SHAPE, "max_ctx %d needs %d splits (max 256)", d->max_ctx, ns);
    return fail(DEC_E_SHAPE, "attention kernel %d cannot run chunk %d of this shape", kind, chunk);
  }
  return DEC_OK;
}

int check_mat(const dec_layer_desc* d, dec_mat m, const char* name) {
  if (!m.w) return fail(DEC_E_NULL, "%s is NULL", name);
  if (!aligned16(m.w)) return fail(DEC_E_ALIGN, "%s not 16-byte aligned", name);
  if (d->wtype == DEC_Q4 && !m.scales) return fail(DEC_E_NULL, "%s scales are NULL", name);
  return DEC_OK;
}

hipError_t gemv(int wtype, int epi, const dec::GemvArgs& a, hipStream_t s) {
  switch (wtype) {
    case DEC_F32: return dec::launch_gemv_f32(epi, a, s);
    case DEC_BF16: return dec::launch_gemv_bf16(epi, a, s);
    default: return dec::launch_gemv_q4(epi, a, s);
  }
}

dec::GemvArgs base_args(const dec_layer_desc* d) {
  dec::GemvArgs a;
  memset(&a, 0, sizeof a);
  a.ntype = d->ntype == DEC_BF16 ? 1 : 0;
  a.eps = d->rms_eps;
  a.nq = d->n_q_heads;
  a.nkv = d->n_kv_heads;
  a.d = d->head_dim;
  a.max_ctx = d->max_ctx;
  a.kvtype = kv_kind(d);
  a.null_kernel = (d->flags & DEC_NULL_KERNELS) ? 1 : 0;
  a.fault = ((d->flags & DEC_TEST_SKIP_ROPE) ? dec::kFaultSkipRope : 0) |
            ((d->flags & DEC_TEST_APPEND_NEXT) ? dec::kFaultAppendNext : 0);
  return a;
}

// Float offset of the DEC_DEBUG_EXPORT_KV rows in the scratch buffer: after
// the per-op path's u, y, and the two FFN vectors.
int64_t kv_export_off(const dec_layer_desc* d) {
  const int64_t nqkv = int64_t(d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  return pad4(d->hidden) + pad4(nqkv) + 2 * pad4(d->ffn);
}

float* kv_export(const dec_layer_desc* d, const dec_layer_state* st) {
  return (d->flags & DEC_DEBUG_EXPORT_KV) ? st->scratch + kv_export_off(d) : nullptr;
}

int qkv_launch(const dec_layer_desc* d, const dec_layer_weights* w, const dec_layer_state* st,
               hipStream_t s) {
  dec::GemvArgs a = base_args(d);
  a.dbg_kv = kv_export(d, st);
  a.W = w->wqkv.w;
  a.S = w->wqkv.scales;
  a.rows = (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  a.cols = d->hidden;
  a.ntask = a.rows / 2;
  a.in = st->x;
  a.norm = w->attn_norm;
  a.y = st->q;
  a.pos = st->pos;
  a.rope = st->rope;
  a.kc = st->k_cache;
  a.vc = st->v_cache;
  a.err = st->err;
  return launched(gemv(d->wtype, dec::kEpiQkv, a, s), "rmsnorm_gemv_qkv_rope");
}

int attn_launch(const dec_layer_desc* d, const dec_layer_state* st, hipStream_t s, bool partials_only = false) {
  dec::AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = st->q;
  a.kc = st->k_cache;
  a.vc = st->v_cache;
  a.part = st->part;
  a.counters = st->counters;
  a.out = st->attn;
  a.pos = st->pos;
  a.err = st->err;
  a.nq = d->n_q_heads;
  a.nkv = d->n_kv_heads;
  a.d = d->head_dim;
  a.max_ctx = d->max_ctx;
  a.kvtype = kv_kind(d);
  a.null_kernel = (d->flags & DEC_NULL_KERNELS) ? 1 : 0;
  a.no_wait = (d->flags & DEC_TEST_NO_WAIT) ? 1 : 0;
  a.drop_last = (d->flags & DEC_TEST_DROP_SPLIT) ? 1 : 0;
  a.partials_only = partials_only ? 1 : 0;
  attn_plan_of(d, &a.chunk, &a.nsplit, &a.waves, &a.kind);
  return launched(dec::launch_attn(a, s), "attn_splitk");
}

// The combine inside the output projection: bf16 weights and cache and a
// split count it supports.
bool attn_o_possible(const dec_layer_desc* d) {
  if (d->wtype != DEC_BF16 || (d->kvtype != DEC_BF16 && d->kvtype != DEC_I8)) return false;
  int chunk, ns, nw, kind;
  attn_plan_of(d, &chunk, &ns, &nw, &kind);
  return dec::attn_o_supported(d->n_q_heads, d->n_kv_heads, d->head_dim, ns);
}

// The fused layer takes that path unless a flag turns it off (the failure
// test of the in-kernel combine needs the in-kernel combine).
bool attn_o_path(const dec_layer_desc* d) {
  const uint32_t off = DEC_UNFUSED | DEC_NO_FUSE_ATTN_O | DEC_DETERMINISTIC | DEC_TEST_NO_WAIT;
  return !(d->flags & off) && attn_o_possible(d);
}

int attn_o_launch(const dec_layer_desc* d, dec_mat wo, const dec_layer_state* st, hipStream_t s) {
  dec::AttnOArgs a;
  memset(&a, 0, sizeof a);
  a.part = st->part;
  a.W = wo.w;
  a.x = st->x;
  a.pos = st->pos;
  a.nq = d->n_q_heads;
  a.nkv = d->n_kv_heads;
  a.d = d->head_dim;
  a.rows = d->hidden;
  a.cols = d->n_q_heads * d->head_dim;
  a.max_ctx = d->max_ctx;
  a.null_kernel = (d->flags & DEC_NULL_KERNELS) ? 1 : 0;
  a.drop_last = (d->flags & DEC_TEST_DROP_SPLIT) ? 1 : 0;
  int nw, kind;
  attn_plan_of(d, &a.chunk, &a.nsplit, &nw, &kind);
  return launched(dec::launch_attn_o(a, s), "attn_o");
}

int residual_launch(const dec_layer_desc* d, dec_mat w, int rows, int cols, const float* in,
                    float* x, hipStream_t s) {
  dec::GemvArgs a = base_args(d);
  a.W = w.w;
  a.S = w.scales;
  a.rows = rows;
  a.cols = cols;
  a.ntask = (rows + 1) / 2;
  a.in = in;
  a.x = x;
  return launched(gemv(d->wtype, dec::kEpiResidual, a, s), "gemv_residual");
}

int ffn_launch(const dec_layer_desc* d, const void* norm, dec_mat wg, dec_mat wu, const float* x,
               float* h, hipStream_t s) {
  dec::GemvArgs a = base_args(d);
  a.W = wg.w;
  a.S = wg.scales;
  a.W2 = wu.w;
  a.S2 = wu.scales;
  a.rows = d->ffn;
  a.cols = d->hidden;
  a.ntask = d->ffn;
  a.in = x;
  a.norm = norm;
  a.y = h;
  return launched(gemv(d->wtype, dec::kEpiSwiglu, a, s), "gated_ffn");
}

// The gated FFN and the down projection in one launch (4-bit weights).
void ffn_down_args(const dec_layer_desc* d, const dec_layer_weights* w, const dec_layer_state* st,
                   dec::GemvArgs* f, dec::GemvArgs* dn) {
  *f = base_args(d);
  f->W = w->wgate.w;
  f->S = w->wgate.scales;
  f->W2 = w->wup.w;
  f->S2 = w->wup.scales;
  f->rows = d->ffn;
  f->cols = d->hidden;
  f->ntask = d->ffn;
  f->in = st->x;
  f->norm = w->ffn_norm;
  f->y = st->h;
  f->err = st->err;
  *dn = base_args(d);
  dn->W = w->wdown.w;
  dn->S = w->wdown.scales;
  dn->rows = d->hidden;
  dn->cols = d->ffn;
  dn->ntask = (d->hidden + 1) / 2;
  dn->in = st->h;
  dn->x = st->x;
  dn->err = st->err;
}

// DEC_OK if the fused FFN + down kernel runs this shape on the current device.
int ffn_down_possible(const dec_layer_desc* d) {
  if (d->wtype != DEC_Q4) return fail(DEC_E_UNSUPPORTED, "the gated FFN with down folded in needs 4-bit weights");
  dec_layer_weights w;
  dec_layer_state st;
  memset(&w, 0, sizeof w);
  memset(&st, 0, sizeof st);
  dec::GemvArgs f, dn;
  ffn_down_args(d, &w, &st, &f, &dn);
  const hipError_t e = dec::ffn_down_q4_check(f, dn);
  if (e == hipErrorInvalidConfiguration)
    return fail(DEC_E_SHAPE, "gated FFN + down: %d workgroups would not all be resident at once",
                (d->hidden + 15) / 16);
  if (e != hipSuccess) return fail(DEC_E_SHAPE, "gated FFN + down: no plan for hidden %d, ffn %d", d->hidden, d->ffn);
  return DEC_OK;
}

int ffn_down_launch(const dec_layer_desc* d, const dec_layer_weights* w, const dec_layer_state* st,
                    hipStream_t s) {
  dec::GemvArgs f, dn;
  ffn_down_args(d, w, st, &f, &dn);
  const int no_wait = (d->flags & DEC_TEST_NO_WAIT) ? 1 : 0;
  return launched(dec::launch_ffn_down_q4(f, dn, st->counters + dec::kFfnDownBarWord, no_wait, s),
                  "gated_ffn_down");
}

// The first fused kernel as its four per-op kernels (rmsnorm, weight
// multiply, QKV projection, RoPE + append), through `scratch`.
int qkv_unfused(const dec_layer_desc* d, const dec_layer_weights* w, const dec_layer_state* st, hipStream_t s) {
  const int H = d->hidden;
  const int nullk = (d->flags & DEC_NULL_KERNELS) ? 1 : 0;
  const int ntype = d->ntype == DEC_BF16 ? 1 : 0;
  const int nqkv = (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  float* u = st->scratch;
  float* y = u + pad4(H);
  int rc;
  if ((rc = launched(dec::launch_rmsnorm_like(st->x, nullptr, ntype, u, H, d->rms_eps, d->wtype, 0, nullk, s),
                     "rmsnorm")))
    return rc;
  if ((rc = launched(dec::launch_mul(u, w->attn_norm, ntype, H, nullk, s), "mul"))) return rc;
  dec::GemvArgs a = base_args(d);
  a.W = w->wqkv.w;
  a.S = w->wqkv.scales;
  a.rows = nqkv;
  a.cols = H;
  a.ntask = (nqkv + 1) / 2;
  a.in = u;
  a.y = y;
  if ((rc = launched(gemv(d->wtype, dec::kEpiStore, a, s), "gemv_qkv"))) return rc;
  return launched(dec::launch_rope_append(y, st->q, st->k_cache, st->v_cache, st->pos, st->rope, st->err,
                                          d->n_q_heads, d->n_kv_heads, d->head_dim, d->max_ctx,
                                          kv_kind(d), kv_export(d, st), nullk, s),
                  "rope_append");
}

// The gated FFN as its three per-op kernels (rmsnorm with multiply, gate/up
// projection, SwiGLU), through `scratch`.
int ffn_unfused(const dec_layer_desc* d, const dec_layer_weights* w, const dec_layer_state* st, hipStream_t s) {
  const int H = d->hidden, F = d->ffn;
  const int nullk = (d->flags & DEC_NULL_KERNELS) ? 1 : 0;
  const int ntype = d->ntype == DEC_BF16 ? 1 : 0;
  const int nqkv = (d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  float* u = st->scratch;
  float* gate = u + pad4(H) + pad4(nqkv);
  float* up = gate + pad4(F);
  int rc;
  if ((rc = launched(dec::launch_rmsnorm_like(st->x, w->ffn_norm, ntype, u, H, d->rms_eps, d->wtype, 1, nullk, s),
                     "rmsnorm_mul")))
    return rc;
  dec::GemvArgs a = base_args(d);
  a.W = w->wgate.w;
  a.S = w->wgate.scales;
  a.W2 = w->wup.w;
  a.S2 = w->wup.scales;
  a.rows = F;
  a.cols = H;
  a.ntask = F;
  a.in = u;
  a.y = gate;
  a.y2 = up;
  if ((rc = launched(gemv(d->wtype, dec::kEpiStore2, a, s), "gemv_gate_up"))) return rc;
  return launched(dec::launch_swiglu(gate, up, st->h, F, nullk, s), "swiglu");
}

int check_state(const dec_layer_state* st, bool scratch) {
  if (!st) return fail(DEC_E_NULL, "state is NULL");
  if (!st->x || !st->q || !st->attn || !st->h || !st->part || !st->counters || !st->k_cache ||
      !st->v_cache || !st->pos || !st->rope || !st->err)
    return fail(DEC_E_NULL, "a state pointer is NULL");
  if (scratch && !st->scratch)
    return fail(DEC_E_NULL, "scratch is NULL (needed by DEC_UNFUSED, DEC_NO_FUSE_QKV, DEC_NO_FUSE_FFN, DEC_DEBUG_EXPORT_KV)");
  for (const void* p : {(const void*)st->x, (const void*)st->q, (const void*)st->attn,
                        (const void*)st->h, (const void*)st->part, (const void*)st->k_cache,
                        (const void*)st->v_cache})
    if (!aligned16(p)) return fail(DEC_E_ALIGN, "state buffer not 16-byte aligned");
  if (scratch && !aligned16(st->scratch)) return fail(DEC_E_ALIGN, "scratch not 16-byte aligned");
  return DEC_OK;
}

int check_weights(const dec_layer_desc* d, const dec_layer_weights* w) {
  if (!w) return fail(DEC_E_NULL, "weights are NULL");
  if (!w->attn_norm || !w->ffn_norm) return fail(DEC_E_NULL, "norm weight is NULL");
  int rc;
  if ((rc = check_mat(d, w->wqkv, "wqkv")) || (rc = check_mat(d, w->wo, "wo")) ||
      (rc = check_mat(d, w->wgate, "wgate")) || (rc = check_mat(d, w->wup, "wup")) ||
      (rc = check_mat(d, w->wdown, "wdown")))
    return rc;
  return DEC_OK;
}

// ---- the library's own scratch (dec_layer_step_static): attention arrival
// counters at offset 0, split partials from kStaticPartOffset, per-op
// intermediates after them. A file-scope device array: every GPU the library
// runs on holds its own copy until the process ends. Host code must not pass
// `scratch` itself to a kernel (on the host it is a stand-in, not a device
// address): the address comes from hipGetSymbolAddress, per device.
constexpr size_t kStaticBytes = DEC_STATIC_SCRATCH_BYTES;
constexpr size_t kStaticCounterWords = 16384;                 // 256 kv heads x DEC_COUNTER_STRIDE
constexpr size_t kStaticPartOffset = kStaticCounterWords * 4;   // 64 KiB
static __device__ __align__(256) uint8_t scratch[kStaticBytes];

__global__ void clear_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_addr[kMaxDevices];      // the array's address on each device (null: not looked up yet)
bool g_static_cleared[kMaxDevices];    // counters cleared by a launch that has run outside a capture

// The array's address on the current device, looked up once per device;
// the first call enqueues a clear of the counter words on `s` (a kernel, not
// a memset, so that a capturing caller records it as an ordinary node).
int static_scratch(hipStream_t s, uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DEC_E_LAUNCH, "no current device for the static scratch");
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(DEC_E_LAUNCH, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_static_addr[dev] = p;
  }
  uint8_t* base = static_cast<uint8_t*>(g_static_addr[dev]);
  if (!g_static_cleared[dev]) {
    hipLaunchKernelGGL(clear_words, dim3(64), dim3(256), 0, s, reinterpret_cast<uint32_t*>(base),
                       int(kStaticCounterWords));
    int rc;
    if ((rc = launched(hipGetLastError(), "clear static counters"))) return rc;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) g_static_cleared[dev] = true;
  }
  *out = base;
  return DEC_OK;
}

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

}  // namespace

extern "C" {

int dec_abi_version(void) { return DEC_ABI_VERSION; }

const char* dec_last_error(void) { return g_err; }

int64_t dec_attn_part_floats(const dec_layer_desc* d) {
  if (check_desc(d)) return -1;
  int chunk, ns, nw, kind;
  attn_plan_of(d, &chunk, &ns, &nw, &kind);
  return int64_t(d->n_q_heads) * ns * (d->head_dim + 2);
}

int64_t dec_cache_bytes(const dec_layer_desc* d) {
  if (check_desc(d)) return -1;
  if (d->kvtype == DEC_I8) return int64_t(dec::kv_i8_bytes(d->n_kv_heads, d->max_ctx, d->head_dim));
  return int64_t(d->n_kv_heads) * d->max_ctx * d->head_dim * (d->kvtype == DEC_BF16 ? 2 : 4);
}

int64_t dec_cache_scale_offset(const dec_layer_desc* d) {
  if (check_desc(d)) return -1;
  if (d->kvtype != DEC_I8) return fail(DEC_E_DTYPE, "scales: the cache is not int8"), -1;
  return int64_t(dec::kv_i8_scale_off(d->n_kv_heads, d->max_ctx, d->head_dim));
}

int64_t dec_cache_stage_offset(const dec_layer_desc* d) {
  if (check_desc(d)) return -1;
  if (d->kvtype != DEC_I8) return fail(DEC_E_DTYPE, "stage: the cache is not int8"), -1;
  return int64_t(dec::kv_i8_stage_off(d->n_kv_heads, d->max_ctx, d->head_dim));
}

int64_t dec_scratch_floats(const dec_layer_desc* d) {
  if (check_desc(d)) return -1;
  const int64_t kv = (d->flags & DEC_DEBUG_EXPORT_KV) ? pad4(2 * int64_t(d->n_kv_heads) * d->head_dim) : 0;
  return kv_export_off(d) + kv;
}

int64_t dec_scratch_kv_offset(const dec_layer_desc* d) {
  if (check_desc(d)) return -1;
  return kv_export_off(d);
}

int dec_rmsnorm_gemv_qkv_rope(const dec_layer_desc* d, const dec_layer_weights* w,
                              const dec_layer_state* st, void* stream) {
  int rc;
  if ((rc = check_desc(d)) || (rc = check_state(st, (d->flags & DEC_DEBUG_EXPORT_KV) != 0))) return rc;
  if (!w) return fail(DEC_E_NULL, "weights are NULL");
  if (!w->attn_norm) return fail(DEC_E_NULL, "attn_norm is NULL");
  if ((rc = check_mat(d, w->wqkv, "wqkv"))) return rc;
  return qkv_launch(d, w, st, hipStream_t(stream));
}

int dec_attn_splitk(const dec_layer_desc* d, const dec_layer_state* st, void* stream) {
  int rc;
  if ((rc = check_desc(d)) || (rc = check_state(st, false))) return rc;
  return attn_launch(d, st, hipStream_t(stream));
}

int dec_attn_partials(const dec_layer_desc* d, const dec_layer_state* st, void* stream) {
  int rc;
  if ((rc = check_desc(d)) || (rc = check_state(st, false))) return rc;
  return attn_launch(d, st, hipStream_t(stream), true);
}

int dec_attn_o_residual(const dec_layer_desc* d, dec_mat wo, const dec_layer_state* st, void* stream) {
  int rc;
  if ((rc = check_desc(d)) || (rc = check_state(st, false)) || (rc = check_mat(d, wo, "wo"))) return rc;
  if (d->flags & DEC_DETERMINISTIC)
    return fail(DEC_E_UNSUPPORTED, "the combine inside the output projection adds with float atomics");
  if (!attn_o_possible(d))
    return fail(DEC_E_UNSUPPORTED, "needs bf16 weights and cache and at most %d attention splits",
                dec::kAttnOSplits);
  return attn_o_launch(d, wo, st, hipStream_t(stream));
}

int dec_gemv_residual(const dec_layer_desc* d, dec_mat w, int32_t rows, int32_t cols,
                      const float* in, float* x, void* stream) {
  int rc;
  if ((rc = check_desc(d)) || (rc = check_mat(d, w, "w"))) return rc;
  if (!in || !x) return fail(DEC_E_NULL, "in/x is NULL");
  if (!aligned16(in)) return fail(DEC_E_ALIGN, "in not 16-byte aligned");
  const int ge = ge_of(d->wtype);
  if (rows <= 0 || cols <= 0 || cols % ge || cols > 16384)
    return fail(DEC_E_SHAPE, "rows %d cols %d (cols a multiple of %d, <= 16384)", rows, cols, ge);
  const char* xb = reinterpret_cast<const char*>(x);
  const char* ib = reinterpret_cast<const char*>(in);
  if (xb < ib + size_t(cols) * 4 && ib < xb + size_t(rows) * 4) return fail(DEC_E_SHAPE, "in and x overlap");
  return residual_launch(d, w, rows, cols, in, x, hipStream_t(stream));
}

int dec_gated_ffn(const dec_layer_desc* d, const void* ffn_norm, dec_mat wgate, dec_mat wup,
                  const float* x, float* h, void* stream) {
  int rc;
  if ((rc = check_desc(d)) || (rc = check_mat(d, wgate, "wgate")) || (rc = check_mat(d, wup, "wup")))
    return rc;
  if (!ffn_norm || !x || !h) return fail(DEC_E_NULL, "ffn_norm/x/h is NULL");
  if (!aligned16(x)) return fail(DEC_E_ALIGN, "x not 16-byte aligned");
  return ffn_launch(d, ffn_norm, wgate, wup, x, h, hipStream_t(stream));
}

int dec_gated_ffn_down(const dec_layer_desc* d, const dec_layer_weights* w, const dec_layer_state* st,
                       void* stream) {
  int rc;
  if ((rc = check_desc(d)) || (rc = check_state(st, false))) return rc;
  if (!w) return fail(DEC_E_NULL, "weights are NULL");
  if (!w->ffn_norm) return fail(DEC_E_NULL, "ffn_norm is NULL");
  if ((rc = check_mat(d, w->wgate, "wgate")) || (rc = check_mat(d, w->wup, "wup")) ||
      (rc = check_mat(d, w->wdown, "wdown")))
    return rc;
  if ((rc = ffn_down_possible(d))) return rc;
  return ffn_down_launch(d, w, st, hipStream_t(stream));
}

int dec_layer_step(const dec_layer_desc* d, const dec_layer_weights* w, const dec_layer_state* st,
                   void* stream) {
  int rc;
  const uint32_t f = d ? d->flags : 0u;
  const bool split_qkv = f & (DEC_UNFUSED | DEC_NO_FUSE_QKV);
  const bool split_ffn = f & (DEC_UNFUSED | DEC_NO_FUSE_FFN);
  const bool fuse_down = (f & DEC_FUSE_DOWN) && !split_ffn;
  const bool scratch = split_qkv || split_ffn || (f & DEC_DEBUG_EXPORT_KV);
  if ((rc = check_desc(d)) || (rc = check_weights(d, w)) || (rc = check_state(st, scratch))) return rc;
  if (fuse_down && (rc = ffn_down_possible(d))) return rc;
  hipStream_t s = hipStream_t(stream);
  const int H = d->hidden, F = d->ffn, qd = d->n_q_heads * d->head_dim;
  if ((rc = split_qkv ? qkv_unfused(d, w, st, s) : qkv_launch(d, w, st, s))) return rc;
  if (attn_o_path(d)) {
    if ((rc = attn_launch(d, st, s, true))) return rc;
    if ((rc = attn_o_launch(d, w->wo, st, s))) return rc;
  } else {
    if ((rc = attn_launch(d, st, s))) return rc;
    if ((rc = residual_launch(d, w->wo, H, qd, st->attn, st->x, s))) return rc;
  }
  if (fuse_down) return ffn_down_launch(d, w, st, s);
  if ((rc = split_ffn ? ffn_unfused(d, w, st, s) : ffn_launch(d, w->ffn_norm, w->wgate, w->wup, st->x, st->h, s)))
    return rc;
  return residual_launch(d, w->wdown, H, F, st->h, st->x, s);
}

int dec_layer_step_static(const dec_layer_desc* d, const dec_layer_weights* w, const dec_layer_state* st,
                          void* stream) {
  int rc;
  if ((rc = check_desc(d))) return rc;
  if (!st) return fail(DEC_E_NULL, "state is NULL");
  if (d->flags & DEC_DEBUG_EXPORT_KV)
    return fail(DEC_E_UNSUPPORTED, "DEC_DEBUG_EXPORT_KV writes to st->scratch, which the static step does not use");
  const int64_t part = pad64(dec_attn_part_floats(d));
  const int64_t ops = dec_scratch_floats(d);
  if (int64_t(d->n_kv_heads) * DEC_COUNTER_STRIDE > int64_t(kStaticCounterWords) ||
      int64_t(kStaticPartOffset) + 4 * (part + ops) > int64_t(kStaticBytes))
    return fail(DEC_E_SHAPE, "static scratch of %zu bytes is too small: %lld partial and %lld per-op floats",
                kStaticBytes, (long long)part, (long long)ops);
  hipStream_t s = hipStream_t(stream);
  uint8_t* base = nullptr;
  if ((rc = static_scratch(s, &base))) return rc;
  dec_layer_state in = *st;
  in.counters = reinterpret_cast<uint32_t*>(base);
  in.part = reinterpret_cast<float*>(base + kStaticPartOffset);
  in.scratch = in.part + part;
  return dec_layer_step(d, w, &in, stream);
}

int dec_lm_head(const dec_layer_desc* d, int32_t head_type, const void* final_norm, dec_mat head,
                int32_t vocab, const float* x, float* logits, int32_t* token, void* stream) {
  int rc;
  if ((rc = check_desc(d))) return rc;
  if (head_type < DEC_F32 || head_type > DEC_Q4) return fail(DEC_E_DTYPE, "head_type %d", head_type);
  if (!final_norm || !x || !logits || !token) return fail(DEC_E_NULL, "final_norm/x/logits/token is NULL");
  if (!head.w) return fail(DEC_E_NULL, "head is NULL");
  if (!aligned16(head.w) || !aligned16(x)) return fail(DEC_E_ALIGN, "head/x not 16-byte aligned");
  if (head_type == DEC_Q4 && !head.scales) return fail(DEC_E_NULL, "head scales are NULL");
  if (vocab <= 0) return fail(DEC_E_SHAPE, "vocab %d", vocab);
  if (d->hidden % ge_of(head_type)) return fail(DEC_E_SHAPE, "hidden %d vs head type", d->hidden);
  hipStream_t s = hipStream_t(stream);
  dec::GemvArgs a = base_args(d);
  a.W = head.w;
  a.S = head.scales;
  a.rows = vocab;
  a.cols = d->hidden;
  a.ntask = (vocab + 1) / 2;
  a.in = x;
  a.norm = final_norm;
  a.y = logits;
  if ((rc = launched(gemv(head_type, dec::kEpiNormStore, a, s), "lm_head"))) return rc;
  return launched(dec::launch_argmax(logits, vocab, token, s), "argmax");
}

int dec_rope_table(double theta, int32_t head_dim, int32_t max_ctx, float* table, void* stream) {
  if (!table) return fail(DEC_E_NULL, "table is NULL");
  if (!(theta > 0.0) || head_dim <= 0 || head_dim % 2 || max_ctx <= 0)
    return fail(DEC_E_SHAPE, "theta/head_dim/max_ctx");
  return launched(dec::launch_rope_table(theta, head_dim, max_ctx, table, hipStream_t(stream)), "rope_table");
}

int dec_embed(const float* embed, int32_t vocab, int32_t hidden, const int32_t* token, float* x,
              uint32_t* err, void* stream) {
  if (!embed || !token || !x || !err) return fail(DEC_E_NULL, "embed/token/x/err is NULL");
  if (vocab <= 0 || hidden <= 0) return fail(DEC_E_SHAPE, "vocab/hidden");
  return launched(dec::launch_embed(embed, vocab, hidden, token, x, err, hipStream_t(stream)), "embed");
}

int dec_advance(int32_t* pos, int32_t pos_lo, int32_t pos_hi, const int32_t* tokens, int32_t* token,
                void* stream) {
  if (!pos) return fail(DEC_E_NULL, "pos is NULL");
  if (tokens && !token) return fail(DEC_E_NULL, "token is NULL");
  if (pos_lo < 0 || pos_hi <= pos_lo) return fail(DEC_E_SHAPE, "pos_lo/pos_hi");
  return launched(dec::launch_advance(pos, pos_lo, pos_hi, tokens, token, hipStream_t(stream)), "advance");
}

}  // extern "C"
