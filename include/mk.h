/*
 * mk -- a fused batch-1 speculative-decode verify step for a DeepSeek-style
 * mixture-of-experts decoder layer on AMD Instinct MI355X (gfx950).
 *
 * One call of mk_decode_step runs one whole layer as ONE persistent kernel
 * launch: RMSNorm, Q and latent-KV projections with RoPE and KV insert, latent
 * attention over the KV cache for T verify rows, router softmax/top-k, routed
 * and shared SwiGLU experts, and both residual adds.  What the layer computes
 * follows "Why one GB300 doesn't beat 4x RTX PRO 6000 at single-stream
 * decode" (section "Where the 11.2 ms goes": the per-kernel table of one
 * verify step; section "Tier 2: the fusion program": norm -> gate -> top-k ->
 * shared expert fused per layer; section "Corrections to things we said": one
 * persistent kernel per decoder layer, tiled for at most 8 rows) and the
 * multi-head latent attention of the DeepSeek-V2 paper (section 2.1).  The
 * fused one-launch-per-layer design answers that report's finding that about a
 * thousand sub-10-microsecond kernels per step cost 40% of the step.
 *
 * Conventions
 *  - Every function returns MK_OK (0) or a negative mk_status; no exceptions
 *    cross this boundary.  mk_last_error() gives a message for the calling
 *    thread's last failure.
 *  - There is no fallback path: an unsupported device or shape is an error,
 *    never a slower kernel ("DeepSeek-V4.1-Flash breaks 1,000 tokens per second
 *    for one user", section "What NVIDIA shipped, and why B300 was refused":
 *    the plugin refuses rather than falling back silently).
 *  - The caller allocates every device buffer (packed weights, KV rows, layer
 *    state, workspace, inputs, outputs), sized with the *_bytes queries.  The
 *    library keeps borrowed pointers until mk_layer_destroy / mk_model_destroy
 *    and allocates no device memory.
 *  - Step calls are asynchronous on the caller's HIP stream (a hipStream_t
 *    passed as void*, NULL = default stream).  A device-side failure (a grid
 *    barrier that timed out) is reported by mk_sync_status after the stream
 *    has been synchronised.
 *  - Calls that use the same workspace, state or KV rows must not overlap in
 *    time (issue them on one stream).  Two persistent launches running at once
 *    on one GPU can starve each other of compute units; the bounded barrier
 *    wait then reports MK_ERR_TIMEOUT rather than hanging.
 */
#ifndef MK_H
#define MK_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 4
#define MK_MAX_T 8           /* verify rows per step: k drafts + 1, at most 8 */
#define MK_STATIC_SCRATCH_BYTES (32u << 20)   /* scratch of mk_decode_step_static, per GPU */

typedef enum mk_status {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = -1,       /* null pointer, T out of range, capacity too small, ... */
  MK_ERR_ABI_MISMATCH = -2,      /* config.abi_version != MK_ABI_VERSION */
  MK_ERR_UNSUPPORTED_DEVICE = -3,/* not gfx950 */
  MK_ERR_NOT_CORESIDENT = -4,    /* the persistent grid cannot be resident at once */
  MK_ERR_HIP = -5,               /* a HIP runtime call failed */
  MK_ERR_TIMEOUT = -6,           /* a grid barrier wait exceeded its bound */
  MK_ERR_DEVICE_FAULT = -7,      /* the device reported another failure */
  MK_ERR_UNSUPPORTED_SHAPE = -8  /* dimensions the kernels are not built for */
} mk_status;

/* Storage formats.  FP8_B128: OCP E4M3 ("FN": bias 7, max 448) codes with one
 * fp32 scale per 128x128 block of the [rows][cols] matrix (value = code * scale).
 * MXFP4: OCP Microscaling (MX v1.0) FP4 -- E2M1 codes, two per byte (element 2j
 * in the low nibble of byte j), one E8M0 scale byte per 32 consecutive elements
 * of a row (value = E2M1(code) * 2^(scale - 127)); the expert format the pages'
 * serving stack uses ("DeepSeek-V4.1-Flash breaks 1,000 tokens per second for
 * one user", section "Appendix: method").
 * FP8_ROW (KV cache only): per cache row, its d_latent + d_rope E4M3 codes (with
 * sparse attention also its idx_dim index-key codes, under the same scale), then
 * the row's scale as an fp32, then zero bytes up to a multiple of 16
 * (value = E4M3(code) * scale).  The same page names an fp8 E4M3 KV cache for
 * that stack without a scale layout; the scale written by a step is the
 * smallest power of two 2^e with max|row| <= 448 * 2^e (1 for a zero row),
 * codes round to nearest even, so the stored value is exact in bf16. */
typedef enum mk_format {
  MK_FMT_F32 = 0, MK_FMT_BF16 = 1, MK_FMT_FP8_B128 = 2, MK_FMT_MXFP4 = 3, MK_FMT_FP8_ROW = 4
} mk_format;

/* Layer shape.  Canonical weight layouts (row-major) that mk_pack_* consume:
 *   W_Q   [n_heads*(d_head+d_rope)][d_model]  head h owns rows h*(d_head+d_rope)..:
 *                                             first d_head -> q^C, last d_rope -> q^R
 *   W_DKV [d_latent+d_rope][d_model]          first d_latent -> latent c, last d_rope -> shared key
 *   W_UK  [n_heads][d_head][d_latent]         k^C_h = W_UK[h] c   (used absorbed: q~ = W_UK[h]^T q^C)
 *   W_UV  [n_heads][d_head][d_latent]         o_h = W_UV[h] z_h
 *   W_O   [d_model][n_heads*d_head]
 *   W_R   [n_experts][d_model]                router; optional bias [n_experts] fp32
 *   W1,W3 [d_ff][d_model], W2 [d_model][d_ff] per expert (SwiGLU: W2 (silu(W1 x) * W3 x))
 * attn_format applies to W_Q, W_DKV, W_UK, W_UV, W_O, W_R (F32 or BF16);
 * expert_format to W1, W3, W2 (F32, BF16, FP8_B128 or MXFP4); kv_format to the
 * cache (F32, BF16 or FP8_ROW).
 * Supported shapes: d_model, d_ff multiples of 128; d_head, d_latent multiples
 * of 32, d_head <= 128, n_heads <= 128; d_rope a multiple of 32; n_experts a multiple of 16 and <= 1024;
 * top_k <= 16; d_model <= 4096; n_heads*d_head and d_ff <= 4608.
 * Formats must be all F32, or attention BF16 with a BF16 or FP8_ROW cache and
 * experts BF16, FP8_B128 or MXFP4. */
typedef struct mk_layer_config {
  int32_t abi_version;       /* must be MK_ABI_VERSION */
  int32_t d_model;
  int32_t n_heads;
  int32_t d_head;
  int32_t d_latent;
  int32_t d_rope;
  int32_t n_experts;
  int32_t top_k;
  int32_t n_shared;          /* 0 or 1 */
  int32_t d_ff;
  int32_t attn_format;
  int32_t expert_format;
  int32_t kv_format;
  int32_t has_router_bias;
  float rms_eps;             /* RMSNorm epsilon */
  float rope_base;           /* RoPE base (angles formed in double on the device) */
  int32_t q_lora_rank;       /* 0: one W_Q.  > 0: low-rank query of this rank (a multiple of 32,
                                <= d_model; bf16 attention): c^Q = W_DQ x, q-norm (RMSNorm of c^Q
                                with gain gamma_q), q = W_UQ norm(c^Q) -- the low-rank query of
                                the DeepSeek-V2 paper, section 2.1, with the q-norm of the pages'
                                q-norm-rope-insert kernel ("Why one GB300 doesn't beat 4x RTX PRO
                                6000 at single-stream decode", section "Where the 11.2 ms goes") */
  int32_t kv_norm;           /* 1: RMSNorm (gain gamma_kv) of the latent c before it is cached
                                (the RoPE key is not normalised); with q_lora_rank > 0 only */
  /* Sparse attention (idx_topk > 0): the pages' sparse attention mode with an indexer ("Why one
   * GB300 ...", sections "Where the 11.2 ms goes" and "Corrections to things we said"), as the
   * lightning indexer of the DeepSeek-V3.2 report.  Per verify row t: q^I = W_IQ x [idx_heads]
   * [idx_dim], w^I = W_IW x [idx_heads], the row's index key k^I = W_IK x (x: the RMSNorm-1
   * output), cached after the RoPE key (a cache row holds d_latent + d_rope + idx_dim values);
   * score of cache row s <= L + t: sum_j w^I_j max(0, q^I_j . k^I_s); the row attends to its
   * idx_topk highest-scoring rows (ties to the lower row; every row when L + t + 1 <= idx_topk).
   * Needs bf16 attention, a bf16 or FP8_ROW cache, n_heads a multiple of 16, idx_heads a multiple of 16,
   * idx_dim a multiple of 32 and <= 128, idx_heads * idx_dim <= 8192, idx_topk <= 8192. */
  int32_t idx_heads;
  int32_t idx_dim;
  int32_t idx_topk;
  int32_t idx_max_rows;      /* sparse: the largest L + T a step may use, a multiple of 8 (sizes
                                the workspace's index scores); a step past it is refused */
  int32_t kv_max_rows;       /* the largest L + T the caller expects (0: not stated).  With the bf16
                                cache and the 512 + 64 latent shape (dense attention), 16,384 or more
                                sizes the workspace for the four-tile attention units that long
                                contexts use ("Why one GB300 doesn't beat 4x RTX PRO 6000 at
                                single-stream decode", section "The decomposition": step time
                                against context); steps of any length stay allowed */
} mk_layer_config;

typedef struct mk_device_info {
  int32_t hip_device;
  int32_t is_gfx950;
  int32_t n_cus;             /* compute units the device reports (never assumed) */
  int32_t wgs_per_cu;        /* co-resident workgroups of the layer kernel per CU */
  int32_t grid_wgs;          /* persistent grid size used */
  int32_t threads_per_wg;
  int32_t lds_bytes_per_wg;
  int32_t pad;
  int64_t hbm_bytes;
  char arch_name[64];
} mk_device_info;

/* Packed tensors (pre-tiled for coalesced streaming; opaque layout). */
typedef enum mk_tensor {
  MK_T_WQ = 0, MK_T_WDKV = 1, MK_T_WUK = 2, MK_T_WUV = 3, MK_T_WO = 4, MK_T_WR = 5,
  MK_T_EXPERT = 6,           /* W1, W3, W2 (and fp8 or MXFP4 scales) of one expert in one block */
  MK_T_WDQ = 7,              /* W_DQ [q_lora_rank][d_model] (q_lora_rank > 0) */
  MK_T_WUQ = 8,              /* W_UQ [n_heads*(d_head+d_rope)][q_lora_rank], rows as W_Q's */
  MK_T_WIDX = 9              /* sparse attention: [W_IQ; W_IW; W_IK] rows [idx_heads*idx_dim +
                                idx_heads + idx_dim][d_model] (W_IQ row j*idx_dim + m = head j, dim m) */
} mk_tensor;

/* Packed layer weights (device pointers). */
typedef struct mk_layer_weights {
  const float* gamma1;       /* [d_model] fp32 RMSNorm gain before attention */
  const float* gamma2;       /* [d_model] fp32 RMSNorm gain before the MoE block */
  const void* wq;
  const void* wdkv;
  const void* wuk;
  const void* wuv;
  const void* wo;
  const void* wr;
  const float* router_bias;  /* [n_experts] fp32, non-NULL iff has_router_bias */
  const void* const* experts;/* HOST array of n_experts + n_shared device pointers to packed
                                expert blocks; slot n_experts + s is shared expert s.  Blocks
                                may be shared between layers. */
  const void* wdq;           /* q_lora_rank > 0: packed W_DQ and W_UQ (wq is then unused and may be */
  const void* wuq;           /*   NULL), gamma_q [q_lora_rank] fp32; NULL otherwise                  */
  const float* gamma_q;
  const float* gamma_kv;     /* kv_norm: [d_latent] fp32; NULL otherwise */
  const void* widx;          /* sparse attention: packed MK_T_WIDX; NULL otherwise */
} mk_layer_weights;

/* KV cache of one layer: `capacity` rows in kv_format (mk_kv_bytes gives the
 * size; an FP8_ROW row takes its values' count + 4 bytes rounded up to 16), row
 * j = latent c_j followed by its RoPE-rotated key (and with sparse attention its
 * index key).  A step reads rows
 * [0, length) plus its own new rows and writes rows [length, length+T); it does
 * not change `length` (the caller commits accepted rows). */
typedef struct mk_kv_cache {
  void* rows;
  int32_t capacity;
  int32_t length;
} mk_kv_cache;

typedef struct mk_stats {
  int64_t steps;             /* mk_decode_step calls that launched */
  int64_t launches;          /* kernel launches issued by those calls (one per step) */
  int32_t grid_wgs;
  int32_t threads_per_wg;
  int32_t barriers_per_step; /* grid-wide barriers inside one launch */
  int32_t trace_enabled;
  int64_t device_launches;   /* launches that reached the expert phase (read from the device) */
  int64_t expert_blocks_sum; /* sum over those launches of expert weight blocks streamed
                                (distinct routed experts + shared experts) */
} mk_stats;

typedef struct mk_layer mk_layer;
typedef struct mk_model mk_model;

/* ---- version, device, sizes ------------------------------------------------ */
/* The library's MK_ABI_VERSION.  A caller compares it with the header it was
 * built against before any other call: a caller of an older interface must
 * fail, not run on quietly ("DeepSeek-V4.1-Flash breaks 1,000 tokens per
 * second for one user", section "Before you try it: two traps and a tip",
 * Trap 1: a caller of the old plugin interface started without error and
 * served at the old speed).  Every mk_layer_config also carries the version
 * and is refused with MK_ERR_ABI_MISMATCH when it differs.  No errors. */
int mk_abi_version(void);
/* Message of the calling thread's last failed call (thread-local; the pointer
 * stays valid until that thread's next failing call).  Never NULL. */
const char* mk_last_error(void);
/* Fills `out` (caller's host memory) for `hip_device`: architecture, compute
 * units and the persistent grid the layer kernel would use (one resident
 * workgroup per compute unit, matched to the device rather than assumed).
 * MK_ERR_UNSUPPORTED_DEVICE if the device is not gfx950 (refused at start-up,
 * no fallback: "DeepSeek-V4.1-Flash breaks 1,000 tokens per second for one
 * user", section "What NVIDIA shipped, and why B300 was refused", where the
 * plugin refuses a GPU with fewer SMs than it keeps resident work blocks for,
 * and section "A small patch", item 1: the resident block count set to the
 * GPU's SM count); MK_ERR_NOT_CORESIDENT if the grid cannot be resident;
 * MK_ERR_INVALID_ARG for a null `out` or a device index out of range. */
int mk_query_device(int hip_device, mk_device_info* out);
/* Validates a config (ABI version, formats, supported shape). */
int mk_check_config(const mk_layer_config* cfg);
int mk_packed_bytes(const mk_layer_config* cfg, int tensor, size_t* bytes);
int mk_kv_bytes(const mk_layer_config* cfg, int32_t capacity, size_t* bytes);
/* Per-layer device state (expert table, counters, trace); one per mk_layer. */
int mk_layer_state_bytes(const mk_layer_config* cfg, int hip_device, size_t* bytes);
/* Scratch shared by layers that run one after another on one stream. */
int mk_layer_workspace_bytes(const mk_layer_config* cfg, int hip_device, size_t* bytes);

/* ---- packing (asynchronous on `stream`) ------------------------------------ */
/* src: canonical device tensor in the tensor's format (layouts above). */
int mk_pack_tensor(const mk_layer_config* cfg, int tensor, const void* src, void* dst, void* stream);
/* One expert: canonical W1, W3 [d_ff][d_model], W2 [d_model][d_ff] in expert_format
 * (MXFP4: bytes [rows][cols/2]); for FP8_B128 the three fp32 scale arrays
 * [ceil(rows/128)][ceil(cols/128)], for MXFP4 the three E8M0 scale byte arrays
 * [rows][cols/32] (passed through the same pointers), else NULL. */
int mk_pack_expert(const mk_layer_config* cfg, const void* w1, const void* w3, const void* w2,
                   const float* s1, const float* s3, const float* s2, void* dst, void* stream);

/* ---- layer ------------------------------------------------------------------- */
/* Checks the device (gfx950, co-residency of the persistent grid: one
 * workgroup per compute unit, all resident at once, as the pages' plugin keeps
 * one resident work block per SM -- "DeepSeek-V4.1-Flash breaks 1,000 tokens
 * per second for one user", sections "What NVIDIA shipped, and why B300 was
 * refused" and "A small patch"), copies the expert table into `state`, clears
 * its counters (synchronously).  `w` and its arrays are read during the call
 * only; the device buffers it points to (and `state_dev`, `workspace_dev`) are
 * borrowed until mk_layer_destroy.  On failure *out is NULL and nothing is
 * kept.  Errors: MK_ERR_INVALID_ARG (null pointers, a router bias given iff
 * the config says so), the config's errors, the device errors of
 * mk_query_device, MK_ERR_HIP. */
int mk_layer_init(const mk_layer_config* cfg, const mk_layer_weights* w, void* state_dev,
                  void* workspace_dev, int hip_device, mk_layer** out);
/* One verify step: hidden_in [T][d_model] fp32 (device) -> hidden_out [T][d_model]
 * fp32 (device; may not alias hidden_in); writes KV rows [length, length+T).
 * MK_ERR_INVALID_ARG if T is not in [1, MK_MAX_T] or length + T > capacity. */
int mk_decode_step(mk_layer* layer, const float* hidden_in, int T, const mk_kv_cache* kv,
                   float* hidden_out, void* stream);
/* For callers that cannot allocate device memory at step time (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same step as mk_decode_step, with the same kernels and results, but its
 * scratch (activations, attention partials, expert rows: everything the layer's
 * workspace holds) is a device array inside the library, of
 * MK_STATIC_SCRATCH_BYTES per GPU, held by every GPU the library runs on until
 * the process ends; the workspace given to mk_layer_init is not touched.  The
 * caller still passes inputs, outputs and the KV rows, and the layer keeps its
 * own state.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams, or layers of different
 * threads) race and give wrong results; issue them on one stream.  Nothing in
 * the array needs clearing between calls.  Errors: those of mk_decode_step,
 * and MK_ERR_UNSUPPORTED_SHAPE when the layer's workspace
 * (mk_layer_workspace_bytes) exceeds MK_STATIC_SCRATCH_BYTES, MK_ERR_HIP when
 * the array's device address could not be found at mk_layer_init. */
int mk_decode_step_static(mk_layer* layer, const float* hidden_in, int T, const mk_kv_cache* kv,
                          float* hidden_out, void* stream);
/* Copies the step's intermediate results from the workspace to host memory
 * (synchronises `stream`).  tap: 0 = Q [T][n_h][d_h+d_r] (q^R rotated),
 * 1 = absorbed query q~ [T][n_h][d_latent], 2 = attention latent z [T][n_h][d_latent],
 * 3 = o [T][n_h*d_head] (fp32 for F32 layers, else bf16 bit patterns: it is kept
 * in the matrix-core operand format), 4 = post-attention hidden [T][d_model],
 * 5 = router logits [T][n_experts], 6 = selected experts int32 [T][top_k],
 * 7 = gates [T][top_k]; sparse attention: 8 = kept cache rows int32 [T][idx_topk]
 * (ascending; row t keeps min(idx_topk, L + t + 1)), 9 = index scores fp32
 * [T][idx_max_rows] (row t: columns 0 .. L + T - 1 written).
 * Valid only after a step on this layer and before another layer reuses the workspace
 * (the workspace that step used: the layer's own, or the static scratch). */
int mk_debug_tap(mk_layer* layer, int tap, void* host_dst, size_t bytes, void* stream);
/* Synchronous: the launch count kept by the host and the counters the kernel
 * kept on the device (launches that reached the expert phases, expert blocks
 * streamed), so a caller can check that the fused path actually ran and how
 * much it streamed ("DeepSeek-V4.1-Flash breaks 1,000 tokens per second for
 * one user", section "Before you try it: two traps and a tip", Trap 2: a
 * setting that made the engine run stock code on every step unnoticed, hence
 * "check that the speed moved").  MK_ERR_INVALID_ARG for null arguments. */
int mk_get_stats(const mk_layer* layer, mk_stats* out);
/* Enables per-workgroup phase timestamps (written into the layer state);
 * enabling clears the trace buffer (synchronous). */
int mk_set_trace(mk_layer* layer, int enabled);
/* Copies the trace of the last step: int64 ticks of a 100 MHz clock,
 * [grid_wgs][2 + 2*barriers_per_step + 16]: start, (arrive, release) per barrier slot, end,
 * then 16 sub-phase stamps (0 where a workgroup did not reach the mark): 0-4 attention
 * (query tile staged, key chunks done, wave merge written, split counter, split merge
 * done), 5 projection input normalised, 6 output-projection input staged, 7 router
 * input normalised, 8 routing done, 9 first down-projection input staged.  Barrier
 * slots 0-7 follow the phases in launch order (0 after the first projection, 1 after
 * RoPE / cache insert / absorbed query, 2 attention, 3 merge and W_UV, 4 W_O, 5 router,
 * 6 gate/up when not fused, 7 experts); 8 follows the low-rank query's up-projection,
 * 9 the index scores and 10 the top-k of sparse attention; a slot a variant does not
 * use stays 0. */
int mk_read_trace(mk_layer* layer, int64_t* host_dst, size_t bytes, void* stream);
/* Barrier wait bound in microseconds (default 2,000,000). */
int mk_set_barrier_timeout_us(mk_layer* layer, int64_t us);
/* Synchronises nothing; reads the layer's device fault word (call after the
 * stream is synchronised).  Every wait inside a launch is bounded: past the
 * bound the fault word is set and all workgroups leave the launch, so a stuck
 * step becomes a visible error instead of a hang ("DeepSeek-V4.1-Flash breaks
 * 1,000 tokens per second for one user", section "The safety layer": the
 * watchdog that turns a possible hang into a fast, visible stop).  MK_OK,
 * MK_ERR_TIMEOUT if a bounded wait gave up, MK_ERR_INVALID_ARG if the device
 * KV length + T passed the capacity.  The word stays set (and every later
 * launch of the layer leaves at its first barrier) until mk_layer_reset. */
int mk_sync_status(mk_layer* layer);
/* Clears the barrier counters and the fault word (synchronous; no launch of
 * this layer may be in flight). */
int mk_layer_reset(mk_layer* layer);
void mk_layer_destroy(mk_layer* layer);

/* ---- stack ------------------------------------------------------------------- */
/* A stack of layers plus bf16 embedding and LM-head tables [vocab][d_model]
 * (the head packed with mk_pack_head, or fp8 with mk_pack_head_fp8) and a
 * final RMSNorm gain.  One step: embedding gather, every layer (one launch
 * each), final norm + LM head + argmax (ties to the lower id) + greedy
 * acceptance (or sampled verification, mk_model_set_sampling), all on the
 * device with the KV length kept in device memory (no host synchronisation). */
int mk_head_packed_bytes(int32_t vocab, int32_t d_model, size_t* bytes);
int mk_pack_head(int32_t vocab, int32_t d_model, const uint16_t* src_bf16, void* dst, void* stream);
/* An fp8 head (the fp8 head that "Why one GB300 doesn't beat 4x RTX PRO 6000 at
 * single-stream decode", section "Three readings", counts as a small item):
 * E4M3 codes [vocab][d_model] (device) with fp32 scales per 128x128 block
 * [ceil(vocab/128)][ceil(d_model/128)] (device), value = E4M3(code) * scale.
 * mk_head_packed_bytes_fmt gives the packed size for format MK_FMT_BF16 or
 * MK_FMT_FP8_B128 (MK_ERR_INVALID_ARG otherwise); mk_pack_head_fp8 repacks
 * into dst (the caller's device buffer of that size), asynchronously on
 * `stream`; the sources may be freed once the stream has passed the call. */
int mk_head_packed_bytes_fmt(int32_t vocab, int32_t d_model, int32_t format, size_t* bytes);
int mk_pack_head_fp8(int32_t vocab, int32_t d_model, const uint8_t* codes, const float* scales, void* dst,
                     void* stream);
int mk_model_state_bytes(int32_t n_layers, int32_t vocab, int hip_device, size_t* bytes);
/* layers: n_layers initialised layers sharing one config; kv_rows: HOST array of
 * n_layers device pointers, each [capacity][d_latent + d_rope]. */
int mk_model_init(mk_layer* const* layers, int32_t n_layers, const uint16_t* embedding,
                  const void* head_packed, const float* gamma_final, int32_t vocab,
                  void* const* kv_rows, int32_t capacity, void* state_dev, void* hidden_dev,
                  mk_model** out);
/* The same with the head's format: MK_FMT_BF16 (mk_pack_head) or
 * MK_FMT_FP8_B128 (mk_pack_head_fp8). */
int mk_model_init_ex(mk_layer* const* layers, int32_t n_layers, const uint16_t* embedding,
                     const void* head_packed, int32_t head_format, const float* gamma_final, int32_t vocab,
                     void* const* kv_rows, int32_t capacity, void* state_dev, void* hidden_dev, mk_model** out);
/* Verification mode of the following steps.  temperature 0 (the default):
 * greedy, as described at mk_model_step.  temperature > 0: sampled
 * verification with matched random draws ("DeepSeek-V4.1-Flash breaks 1,000
 * tokens per second for one user", section "The safety layer"): speculative
 * sampling with the drafts taken as point proposals.  Row i's target is
 * p_i = softmax(logits_i / temperature); draft i+1 is accepted when the row's
 * acceptance draw is below p_i(draft); the first rejection commits a draw from
 * p_i without the rejected draft, T-1 acceptances a draw from p_{T-1}.  Token
 * draws are Gumbel-max: argmax_v logits_iv / temperature - ln(-ln u_iv), ties
 * to the lower id.  The draws of the s-th step after this call (s = 0, 1, ...,
 * counted on the device by every step that commits) are SplitMix64 outputs:
 * key = mix(seed + (s+1) G), u(i) = ((mix(key + (i+1) G) >> 41) + 1/2) 2^-23
 * (G = 0x9E3779B97F4A7C15, mix = SplitMix64's output function), with
 * u_iv = u(i (vocab+1) + v) and the acceptance draw u(i (vocab+1) + vocab).
 * argmax_dev then receives each row's token draw.  Synchronous (resets the
 * device step counter); no step may be in flight.  MK_ERR_INVALID_ARG for a
 * negative or non-finite temperature. */
int mk_model_set_sampling(mk_model* m, float temperature, uint64_t seed);
/* Sets the committed KV length (synchronous copy). */
int mk_model_set_length(mk_model* m, int32_t length);
/* Device pointer to the committed KV length (int32). */
const int32_t* mk_model_length_ptr(const mk_model* m);
/* One verify step of the stack: T = k+1 rows, the last committed token and k
 * drafts, verified in one pass; tokens per step = accepted drafts + 1 ("Why
 * one GB300 doesn't beat 4x RTX PRO 6000 at single-stream decode", section
 * "The decomposition"), with greedy acceptance (the byte-for-byte greedy gate
 * of "DeepSeek-V4.1-Flash breaks 1,000 tokens per second for one user",
 * section "The safety layer").  Launches: embedding, one per layer, one for
 * the head, all asynchronous on `stream`; the host reads nothing back.
 * tokens_dev [T] (device int32): t0 then T-1 drafts.  a_i = argmax of row i's
 * logits (ties to the lower id); n = the largest n <= T-1 with draft_j ==
 * a_{j-1} for all j <= n; n+1 tokens are committed (drafts 1..n and a_n).
 * Writes argmax_dev [T], committed_dev [1 + T] (count, then the tokens),
 * advances the device KV length by n+1 and sets tokens_dev[0] = a_n; if
 * next_drafts_dev ([T-1]) is non-NULL it is copied into tokens_dev[1..T-1] for
 * the next step.  logits_dev ([T][vocab] fp32) may be NULL.
 * Device-side failures (a token id outside [0, vocab), KV length + T past the
 * capacity, a layer's bounded wait giving up) set the stack's fault word: the
 * remaining layers of the step do nothing and the head commits nothing
 * (committed_dev[0] = 0, argmax_dev = -1, KV length and tokens_dev unchanged);
 * mk_model_sync_status reports it.  Host-side errors: MK_ERR_INVALID_ARG (null
 * pointers, T outside [1, MK_MAX_T]), MK_ERR_HIP (a launch failed). */
int mk_model_step(mk_model* m, int32_t* tokens_dev, int T, const int32_t* next_drafts_dev,
                  int32_t* argmax_dev, int32_t* committed_dev, float* logits_dev, void* stream);
/* Reads the stack's device fault word (call after the stream is synchronised):
 * MK_OK, MK_ERR_INVALID_ARG (a token id outside [0, vocab), or KV length + T
 * past the capacity), MK_ERR_TIMEOUT (a layer's bounded wait gave up), as in
 * mk_sync_status ("The safety layer": a visible stop, not a silent one).  The
 * word stays set, and every later step commits nothing, until mk_model_reset. */
int mk_model_sync_status(mk_model* m);
/* Clears the stack's fault word and resets every layer (mk_layer_reset);
 * synchronous, no step may be in flight. */
int mk_model_reset(mk_model* m);
/* Diagnostics: with record_dev (device fp32 [n_layers + 1][MK_MAX_T][d_model],
 * the caller's) set, a step keeps every layer's input rows: the embedding
 * writes slot 0, layer l reads slot l and writes slot l + 1, the head reads
 * slot n_layers.  NULL returns to the two internal buffers.  Takes effect at
 * the next mk_model_step. */
int mk_model_set_hidden_record(mk_model* m, float* record_dev);
void mk_model_destroy(mk_model* m);

#ifdef __cplusplus
}
#endif
#endif
