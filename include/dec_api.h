/*
 * dec_api.h - C ABI of libdec, a batch-1 decoder-layer engine for AMD MI355X
 * (gfx950, wave64).
 *
 * One decode step of a pre-norm decoder layer, for a single token, follows
 * the chain "RDNA4 Decode Kernel Fusion: Pipeline Barriers, Not Launches, Are
 * the Win" lists in section "Decode is where the bubble has nowhere to go":
 * input RMSNorm, QKV projection, RoPE on Q and K, attention against the KV
 * cache, output projection, post-attention RMSNorm, gate and up projections,
 * SwiGLU, down projection; the residual stream x is updated after the output
 * projection and after the down projection. The same page's section "Fusion
 * removes the barrier by removing the write" (and its opening questions)
 * names the three fusions this library implements: RMSNorm and its weight
 * multiply in the preamble of the following projection, RoPE folded into the
 * QKV projection's epilogue, and gate, up and SwiGLU as one gated-FFN kernel
 * whose wide intermediate never reaches memory. A fused layer is five
 * kernels: dec_rmsnorm_gemv_qkv_rope, the attention (dec_attn_splitk, or
 * dec_attn_partials with bf16 weights and cache), the output projection with
 * the residual add (dec_gemv_residual, or dec_attn_o_residual, which also
 * combines the attention's partials), dec_gated_ffn, dec_gemv_residual (down
 * projection); dec_layer_step runs them in order.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *    stated otherwise. The library never allocates, frees or synchronizes,
 *    and reads no device memory from the host; every call only enqueues
 *    kernels on `stream` (a hipStream_t passed as void*; NULL is the null
 *    stream), so every call may be captured into a HIP graph. The caller
 *    keeps every buffer alive until the enqueued work has finished.
 *  - Return value: DEC_OK (0), or a negative DEC_E_* code; nothing is
 *    enqueued when the code is negative. dec_last_error() returns a
 *    thread-local text for the last failure on the calling thread.
 *  - Matrices are row-major [rows][cols]: y = W u means
 *    y[r] = sum_c W[r][c] u[c]. Element types:
 *      DEC_F32  float32
 *      DEC_BF16 bfloat16 bit patterns (uint16)
 *      DEC_Q4   4-bit blocks: `w` is [rows][cols/2] bytes, element 2i in the
 *               low nibble of byte i and 2i+1 in the high nibble, each a
 *               two's-complement code in [-8, 7]; `scales` is fp16
 *               [rows][cols/32]; weight = scale[r][c/32] * code[r][c].
 *    Each matrix base pointer is 16-byte aligned; cols is a multiple of 4
 *    (f32), 8 (bf16) or 32 (q4), and at most 16384.
 *  - Activations (x, q, attention output, h) are float32. Arithmetic is
 *    float32 with float32 accumulation.
 *  - The position of the token being decoded is a device int32 (`pos`), so a
 *    captured graph replays unchanged from token to token. A position outside
 *    [0, max_ctx) makes the kernels that read it set bit DEC_ERR_POS in the
 *    device word `err` and store nothing.
 */
#ifndef DEC_API_H
#define DEC_API_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DEC_ABI_VERSION 7

enum dec_dtype { DEC_F32 = 0, DEC_BF16 = 1, DEC_Q4 = 2, DEC_I8 = 3 };

enum dec_status {
  DEC_OK = 0,
  DEC_E_NULL = -1,        /* a required pointer is NULL */
  DEC_E_SHAPE = -2,       /* sizes violate the contract above */
  DEC_E_DTYPE = -3,       /* unsupported element type for this argument */
  DEC_E_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  DEC_E_LAUNCH = -5,      /* the HIP runtime rejected a launch */
  DEC_E_UNSUPPORTED = -6  /* valid request the library does not implement */
};

/* uint32 words per kv head in dec_layer_state.counters: kv head j uses words
   j * DEC_COUNTER_STRIDE (+0 arrivals, +1 finished combiners), alone on
   their 64-byte line; words 2 and 3 of the first line count the grid-wide
   arrivals and departures of dec_gated_ffn_down */
#define DEC_COUNTER_STRIDE 16

/* bits of the device error word */
#define DEC_ERR_POS 0x1u
#define DEC_ERR_TOKEN 0x2u
#define DEC_ERR_SYNC 0x4u  /* an attention combiner stopped waiting for the other
                              splits of its kv head (that output slice is not
                              written), or a dec_gated_ffn_down workgroup stopped
                              waiting for the others (its 16 rows of x not updated) */

/* dec_layer_desc.flags.
   Fusion controls, global and per fused operation ("backend-specific kernel
   fusion", sections "A practical engineering example" and "What you can do
   this week": every fused path can be switched off on its own and all of
   them at once, and the unfused path computes the same arithmetic): */
#define DEC_UNFUSED 0x1u        /* all three below: dec_layer_step runs the ten per-op kernels */
#define DEC_NULL_KERNELS 0x2u   /* same launches, every kernel body returns at once */
#define DEC_NO_FUSE_QKV 0x4u    /* the first kernel as rmsnorm, weight multiply, QKV projection,
                                   RoPE + append (four kernels) */
#define DEC_NO_FUSE_FFN 0x8u    /* the gated FFN as rmsnorm with multiply, gate/up projection,
                                   SwiGLU (three kernels) */
#define DEC_NO_FUSE_ATTN_O 0x10u /* the attention combines its own splits and the output
                                    projection is a plain dec_gemv_residual */
#define DEC_DETERMINISTIC 0x20u /* no float atomics on the path, so repeated runs give the
                                   same bits (takes the DEC_NO_FUSE_ATTN_O path) */
#define DEC_FUSE_DOWN 0x40u     /* 4-bit weights: the gated FFN and the down projection as one
                                   kernel (dec_gated_ffn_down), four kernels per layer; ignored
                                   with DEC_UNFUSED or DEC_NO_FUSE_FFN */

/* Which attention kernel runs (a two-bit field; 0 = the library's choice
   for the shape). All three compute the same split-K reduction ("RDNA4
   Decode Kernel Fusion...", section "Where fusion stops"); they differ in
   how a workgroup's rows reach the softmax. A kernel that cannot run the
   shape or attn_chunk makes every entry point return DEC_E_SHAPE. */
#define DEC_ATTN_KERNEL_MASK 0x3000u
#define DEC_ATTN_BATCHED 0x1000u /* rows in registers in batches, one softmax per workgroup
                                    through LDS (any cache type; chunks up to 256) */
#define DEC_ATTN_STREAM 0x2000u  /* keys scored as they arrive, values staged in LDS
                                    (chunks whose values fit in LDS; int8 caches: at
                                    most 256, at most four query heads per kv head) */
#define DEC_ATTN_LOCAL 0x3000u   /* every row requested at launch, a softmax per wave,
                                    waves rescaled once (bf16 cache; chunks up to 9 row
                                    steps of eight waves: 288 positions at d = 128) */
/* Tests only. DEC_TEST_NO_WAIT exercises a failure path: an attention
   combiner that finds splits of its kv head still missing gives up at once
   (DEC_ERR_SYNC, its output slice not written) instead of polling. The
   three faults below make the fused kernels' numbers wrong on purpose
   (every kernel still completes and stores in bounds), so a parity test can
   show that it fails on a wrong kernel ("Kernel fusion and block bridging",
   section "What it keeps": the gates are run against violations). */
#define DEC_TEST_NO_WAIT 0x100u
#define DEC_TEST_SKIP_ROPE 0x200u   /* the fused QKV kernel leaves q and k unrotated */
#define DEC_TEST_APPEND_NEXT 0x400u /* the fused QKV kernel stores k, v at position p + 1
                                       (at p when p + 1 is past the cache) */
#define DEC_TEST_DROP_SPLIT 0x800u  /* attention combines leave out the last split
                                       (when there are two or more) */
/* Debugging: the QKV step (fused or per-op) also writes the token's rotated
   k and plain v rows as float32, before they are rounded to the cache type,
   to st->scratch from float offset dec_scratch_kv_offset(desc): k [n_kv][d],
   then v [n_kv][d]. A test can then check every appended cache value
   against its own float32 source bit for bit. Needs st->scratch. */
#define DEC_DEBUG_EXPORT_KV 0x80u

/* Static shape of one decoder layer (identical for every layer of a stack). */
typedef struct {
  int32_t hidden;      /* H */
  int32_t n_q_heads;   /* query heads */
  int32_t n_kv_heads;  /* key/value heads; n_q_heads % n_kv_heads == 0, ratio <= 8 */
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t ffn;         /* F */
  int32_t max_ctx;     /* cache positions per (layer, kv head) */
  float rms_eps;       /* RMSNorm epsilon, added to mean(x^2) inside the root */
  int32_t wtype;       /* projection weights: DEC_F32 | DEC_BF16 | DEC_Q4 */
  int32_t ntype;       /* norm weights: DEC_F32 | DEC_BF16 */
  int32_t kvtype;      /* KV cache: DEC_F32 | DEC_BF16 | DEC_I8 (int8 rows with a float
                          scale each, head_dim 128; layout at dec_cache_bytes) */
  int32_t attn_chunk;  /* cache positions per attention split; 0 = library default */
  uint32_t flags;      /* DEC_* flags above */
} dec_layer_desc;

/* A weight matrix: `w` the elements, `scales` the per-block fp16 scales
   (DEC_Q4 only; NULL otherwise). */
typedef struct {
  const void* w;
  const void* scales;
} dec_mat;

/* One layer's weights (all device memory, caller-owned).
   attn_norm, ffn_norm: [H] in ntype.
   wqkv: [(n_q + 2 n_kv) d][H]; rows are the q heads, then the k heads, then
         the v heads, each head's d rows contiguous.
   wo: [H][n_q d]. wgate, wup: [F][H]. wdown: [H][F]. */
typedef struct {
  const void* attn_norm;
  dec_mat wqkv;
  dec_mat wo;
  const void* ffn_norm;
  dec_mat wgate;
  dec_mat wup;
  dec_mat wdown;
} dec_layer_weights;

/* One layer's activations, cache and bookkeeping (device memory, caller-owned). */
typedef struct {
  float* x;            /* [H] residual stream, read and updated in place */
  float* q;            /* [n_q d] rotated queries (written by the QKV kernel) */
  float* attn;         /* [n_q d] attention output, heads in order (the bf16
                          layer step combines inside the output projection
                          and leaves it untouched) */
  float* h;            /* [F] SwiGLU output, input of the down projection */
  float* part;         /* [dec_attn_part_floats(desc)] split partials, 16-byte
                          aligned; any contents between calls */
  uint32_t* counters;  /* [n_kv * DEC_COUNTER_STRIDE] arrival counters; zero
                          before first use, and the attention kernel leaves
                          them zero */
  void* k_cache;       /* this layer's keys   [n_kv][max_ctx][d] in kvtype
                          (DEC_I8: dec_cache_bytes(desc) bytes, see there) */
  void* v_cache;       /* this layer's values, same layout */
  const int32_t* pos;  /* position p of the token being decoded */
  const float* rope;   /* [max_ctx][d/2][2] (cos, sin) from dec_rope_table */
  uint32_t* err;       /* device error word (bits are OR-ed in) */
  float* scratch;      /* [dec_scratch_floats(desc)]; used by DEC_UNFUSED,
                          DEC_NO_FUSE_QKV, DEC_NO_FUSE_FFN and
                          DEC_DEBUG_EXPORT_KV only, may be NULL otherwise */
} dec_layer_state;

/* ---- sizes of caller-provided buffers ---------------------------------- */

/* floats needed by dec_layer_state.part for this shape (>= 1). */
int64_t dec_attn_part_floats(const dec_layer_desc* desc);
/* Bytes of one layer's k_cache (and of its v_cache), 256-byte aligned
   sections. DEC_F32/DEC_BF16: the rows [n_kv][max_ctx][d]. DEC_I8 (a leaner
   KV cache, "Vulkan Command Buffer Reuse vs CUDA Graphs...", section "What I
   am building next"; the scheme is this library's): int8 codes
   [n_kv][max_ctx][d], then at byte offset dec_cache_scale_offset one float
   scale per row [n_kv][max_ctx] (value = code * scale; scale = max|x| / 127,
   code = x * (127 / max|x|) rounded half to even, in float32), then at
   dec_cache_stage_offset the newest k (or v) row [n_kv][d] as float32: the
   QKV step writes it there and the attention quantizes it into slot p. */
int64_t dec_cache_bytes(const dec_layer_desc* desc);
int64_t dec_cache_scale_offset(const dec_layer_desc* desc);
int64_t dec_cache_stage_offset(const dec_layer_desc* desc);
/* floats needed by dec_layer_state.scratch for the per-op path (with
   DEC_DEBUG_EXPORT_KV in desc->flags, also for the exported k and v rows). */
int64_t dec_scratch_floats(const dec_layer_desc* desc);
/* float offset in st->scratch of the rows DEC_DEBUG_EXPORT_KV writes (after
   every per-op intermediate, so a layer step does not overwrite them). */
int64_t dec_scratch_kv_offset(const dec_layer_desc* desc);

/* ---- the five kernels of a fused layer -------------------------------- */

/* Input RMSNorm + QKV projection + RoPE + KV-cache append, one kernel.
   Passages: "RDNA4 Decode Kernel Fusion..." opening questions and section
   "Fusion removes the barrier by removing the write" (RMSNorm and its multiply
   in the projection's preamble; RoPE in the QKV projection's epilogue);
   "Kernel fusion and block bridging", section "Fusion" (q's rotation, k's
   rotation into its cache slot and v's copy into its slot in one launch).
   Computes u = x / sqrt(mean(x^2) + eps) * attn_norm, y = Wqkv u, rotates
   each q and k head by RoPE at position p (pairs (i, i + d/2), cos/sin from
   the table), writes q (float32) and stores k, v rounded to kvtype
   (nearest even) at cache position p of every kv head (DEC_I8: as float32
   rows in the cache's stage section; the attention appends them).
   Reads: x, weights, rope, pos. Writes: q, k_cache[:, p], v_cache[:, p], err. */
int dec_rmsnorm_gemv_qkv_rope(const dec_layer_desc* desc, const dec_layer_weights* w,
                              const dec_layer_state* st, void* stream);

/* Decode attention of the token's queries over cache positions 0..p,
   split along the positions ("split-K"): each workgroup reduces one chunk of
   one kv head for all of its query heads into (max, sum, unnormalized
   output) partials, and the last workgroups of a kv head to arrive (up to
   eight, each a slice of the head group's outputs) combine them with a
   log-sum-exp rescale. Passage: "RDNA4 Decode Kernel Fusion...",
   sections "Decode is where the bubble has nowhere to go" (attention against
   the KV cache) and "Where fusion stops" (attention stays its own kernel).
   Query head h uses kv head h / (n_q/n_kv); scores are scaled by 1/sqrt(d).
   The last arrivals of a kv head combine in a fixed order (each output
   element sums its splits in split order), so repeated runs give the same
   bits. DEC_I8 caches: the workgroup whose split holds p quantizes the
   staged k and v rows into slot p and scores the token from them. Reads:
   q, caches, pos. Writes: attn, part, counters (left zero), err (and the
   int8 cache's slot p). */
int dec_attn_splitk(const dec_layer_desc* desc, const dec_layer_state* st, void* stream);

/* The attention's first half on its own: the same split-K reduction as
   dec_attn_splitk, stopping once every split's partials are in `part`
   (o [n_kv][splits][g][d] unnormalized, then (m, l) [n_kv][splits][g][2]
   with m in log2 units); nothing is combined and attn, counters are left
   as they were. Passage: "RDNA4 Decode Kernel Fusion...", section "Where
   fusion stops" (attention is the one step that stays its own kernel; what
   follows it is the output projection). Reads: q, caches, pos. Writes:
   part, err. */
int dec_attn_partials(const dec_layer_desc* desc, const dec_layer_state* st, void* stream);

/* The attention's combine fused into the output projection with its
   residual add: x += Wo a, where a is formed inside this kernel from the
   partials dec_attn_partials left in st->part (a log-sum-exp rescale per
   head and split), so the attention output never reaches memory. Passage:
   "RDNA4 Decode Kernel Fusion...", sections "Where fusion stops" (the
   output projection after attention) and "Fusion removes the barrier by
   removing the write" (an intermediate that is not written needs no
   barrier). Each workgroup owns one column block of Wo (one query head,
   or a kv head's whole group of 64-wide heads) and a block of rows, and
   adds its rows' share to x with float atomics: repeated runs agree within
   float32 rounding, not bit for bit. Requires bf16 weights and cache and at
   most 32 attention splits for desc (DEC_E_UNSUPPORTED otherwise, and under
   DEC_DETERMINISTIC). Reads: part, wo, pos. Writes: x. */
int dec_attn_o_residual(const dec_layer_desc* desc, dec_mat wo, const dec_layer_state* st, void* stream);

/* x += W in: a projection fused with the residual add ("RDNA4 Decode Kernel
   Fusion...", section "Decode is where the bubble has nowhere to go": output
   projection and down projection). `w` is [rows][cols] in desc->wtype, `in`
   is float32 [cols], `x` float32 [rows]. `in` and `x` must not overlap. */
int dec_gemv_residual(const dec_layer_desc* desc, dec_mat w, int32_t rows, int32_t cols,
                      const float* in, float* x, void* stream);

/* Post-attention RMSNorm + gate and up projections + SwiGLU, one kernel
   ("RDNA4 Decode Kernel Fusion...", section "Fusion removes the barrier by
   removing the write": gate, up and SwiGLU collapse into one gated-FFN
   kernel). u = x / sqrt(mean(x^2) + eps) * ffn_norm;
   h[j] = silu(wgate[j] . u) * (wup[j] . u), silu(z) = z / (1 + exp(-z)).
   The gate and up values stay in registers; only h (float32 [F]) is written. */
int dec_gated_ffn(const dec_layer_desc* desc, const void* ffn_norm, dec_mat wgate, dec_mat wup,
                  const float* x, float* h, void* stream);

/* The gated FFN and the down projection with the residual add, in one
   launch: x += wdown . h, h as dec_gated_ffn computes it from x ("RDNA4
   Decode Kernel Fusion: Pipeline Barriers, Not Launches, Are the Win",
   section "Fusion removes the barrier by removing the write": the figure's
   four-kernel layer folds the down projection into the FFN). 4-bit weights
   only (others: DEC_E_UNSUPPORTED). Reads w->ffn_norm, w->wgate, w->wup,
   w->wdown and st->x; writes st->h (float32 [F]) and st->x; uses words 2
   and 3 of st->counters (zero before the first call; every call leaves
   them zero) and st->err. One workgroup per 16 rows of x; every workgroup
   computes its share of h, then waits at a grid-wide counter until all
   have, so all of them must be resident on the GPU at once: a shape whose
   workgroups would not all fit on the current device, or whose rows exceed
   the kernel's plans, returns DEC_E_SHAPE. A wait that does not
   end within its bound sets DEC_ERR_SYNC and leaves that workgroup's rows
   of x unchanged. h differs from dec_gated_ffn's in the last bits (its
   sums are split over eight waves instead of four); x is within float32
   rounding of dec_gated_ffn followed by dec_gemv_residual. */
int dec_gated_ffn_down(const dec_layer_desc* desc, const dec_layer_weights* w, const dec_layer_state* st,
                       void* stream);

/* One whole decoder layer for the token at position *pos, in the order
   "RDNA4 Decode Kernel Fusion: Pipeline Barriers, Not Launches, Are the Win"
   gives in section "Decode is where the bubble has nowhere to go" (norm,
   QKV projection, RoPE, attention, output projection, norm, gate/up,
   SwiGLU, down), with the fusions of its section "Fusion removes the
   barrier by removing the write" and of its opening questions (norm in the
   projection's preamble, RoPE in the QKV epilogue, gate, up and SwiGLU in
   one kernel). Pre-norm residual structure: x += O(attention(norm(x))),
   then x += down(ffn(norm(x))).
   Five kernels: dec_rmsnorm_gemv_qkv_rope, the attention, the output
   projection with the residual add, dec_gated_ffn, dec_gemv_residual
   (down). With bf16 weights and cache (and at most 32 attention splits)
   the attention is dec_attn_partials and the output projection
   dec_attn_o_residual (the combine inside the projection, float atomics
   into x); otherwise dec_attn_splitk and dec_gemv_residual.
   Flags: DEC_NO_FUSE_QKV, DEC_NO_FUSE_FFN and DEC_NO_FUSE_ATTN_O switch off
   one fused operation each (DEC_DETERMINISTIC takes the atomics-free
   path); DEC_UNFUSED switches off all three: ten per-op kernels (rmsnorm,
   weight multiply, QKV projection, RoPE + append, attention, output
   projection + residual, rmsnorm with multiply, gate/up projection,
   SwiGLU, down projection + residual), whose f32 and 4-bit results equal
   the fused ones bit for bit. st->scratch is needed when DEC_UNFUSED,
   DEC_NO_FUSE_QKV or DEC_NO_FUSE_FFN is set. DEC_FUSE_DOWN (4-bit
   weights) runs dec_gated_ffn_down in place of the last two kernels. */
int dec_layer_step(const dec_layer_desc* desc, const dec_layer_weights* w,
                   const dec_layer_state* st, void* stream);

/* ---- the same step without caller-provided scratch ----------------------- */

/* Bytes of the library's static device scratch (per GPU, held until the
   process ends). */
#define DEC_STATIC_SCRATCH_BYTES (4u << 20)

/* dec_layer_step for callers that cannot allocate device memory: code under
   HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
   The attention's split partials, its arrival counters and the per-op
   intermediates live in a static device array of the library instead of
   st->part, st->counters and st->scratch, which are not read (they may be
   NULL); every other field of st is used as in dec_layer_step. The array
   holds DEC_STATIC_SCRATCH_BYTES per GPU: a shape whose 64 KiB of counter
   words, partials (dec_attn_part_floats) and per-op intermediates
   (dec_scratch_floats, floats) do not fit returns DEC_E_SHAPE. The first
   call on a GPU looks up the array's address there and enqueues a clear of
   the counters on `stream`; nothing is allocated, copied or synchronized.
   Every call on one GPU shares that GPU's array, which keeps the last call's
   contents, so calls that overlap on one GPU (other streams, other threads)
   race and must be serialized by the caller. DEC_DEBUG_EXPORT_KV is
   refused (DEC_E_UNSUPPORTED): its rows would land in the static array. */
int dec_layer_step_static(const dec_layer_desc* desc, const dec_layer_weights* w,
                          const dec_layer_state* st, void* stream);

/* ---- LM head ------------------------------------------------------------- */

/* Final RMSNorm, LM head and greedy choice of the next token: the "LM head +
   sampling" segment of the per-token budget in "RDNA4 Decode Kernel Fusion:
   Pipeline Barriers, Not Launches, Are the Win" (section "What it does to
   the token"); sampling is greedy. u = x / sqrt(mean(x^2) + eps) * final_norm
   (norm weight in desc->ntype), logits = W_head u with W_head [vocab][H] in
   head_type (DEC_F32 | DEC_BF16 | DEC_Q4), *token = argmax logits (the lowest
   index among equal maxima). Writes logits (float32 [vocab]) and *token.
   Two kernels: the GEMV with the norm prologue, and a one-workgroup argmax. */
int dec_lm_head(const dec_layer_desc* desc, int32_t head_type, const void* final_norm, dec_mat head,
                int32_t vocab, const float* x, float* logits, int32_t* token, void* stream);

/* ---- per-token bookkeeping --------------------------------------------- */

/* RoPE table: table[p][i] = (cos(p w_i), sin(p w_i)), w_i = theta^(-2i/d),
   for p < max_ctx and i < d/2; the angle and both functions are evaluated in
   float64 on the device and rounded to float32. */
int dec_rope_table(double theta, int32_t head_dim, int32_t max_ctx, float* table, void* stream);

/* x = embed[*token] (float32 table [vocab][hidden]). A token outside
   [0, vocab) sets bit DEC_ERR_TOKEN in err and writes zeros to x. */
int dec_embed(const float* embed, int32_t vocab, int32_t hidden, const int32_t* token,
              float* x, uint32_t* err, void* stream);

/* Advance to the next token: p = *pos + 1, replaced by pos_lo when it falls
   outside [pos_lo, pos_hi); *pos = p; if `tokens` is not NULL, *token = tokens[p - pos_lo]
   (a teacher-forced list of pos_hi - pos_lo entries). One tiny kernel. */
int dec_advance(int32_t* pos, int32_t pos_lo, int32_t pos_hi, const int32_t* tokens,
                int32_t* token, void* stream);

/* ---- misc --------------------------------------------------------------- */
const char* dec_last_error(void);
int dec_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DEC_API_H */
