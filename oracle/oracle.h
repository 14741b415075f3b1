/*
 * CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of one batch-1
 * speculative-decode verify step of a DeepSeek-style mixture-of-experts decoder
 * layer, and of the stack around it (embedding, final norm, LM head, greedy
 * acceptance).  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load or call it.  It shares no code with the GPU library.
 *
 * Sources of the computation:
 *  - Which operations make up the layer and in what order (RMSNorm, Q and
 *    latent-KV projections with RoPE and KV insert, latent attention over the
 *    KV cache for T = k+1 verify rows, router softmax/top-k, routed and shared
 *    SwiGLU experts, residual adds): "Why one GB300 doesn't beat 4x RTX PRO
 *    6000 at single-stream decode", section "Where the 11.2 ms goes" (the
 *    per-kernel table: norm/quant, q-norm-rope-insert, FlashMLA decode
 *    attention, top-k, prepare-megamoe, MegaMoE, lm_head, rejection kernel)
 *    and section "Tier 2: the fusion program" (norm -> gate -> top-k -> shared
 *    expert); the same report, section "The decomposition", for verify blocks
 *    of k drafts plus one row, tiled for at most 8 rows.
 *  - The multi-head latent attention algebra (latent KV cache c, decoupled
 *    RoPE key shared by all heads, absorbed query q~ = W_UK^T q^C): the
 *    DeepSeek-V2 paper, section 2.1 "Multi-Head Latent Attention"; the pages
 *    name FlashMLA as the attention kernel ("DeepSeek-V4.1-Flash breaks 1,000
 *    tokens per second for one user", section "Appendix: method").
 *  - RMSNorm (Zhang and Sennrich 2019), RoPE (Su et al., RoFormer, 2021,
 *    adjacent-pair form), SwiGLU (Shazeer 2020), softmax top-k gating with
 *    renormalised gates over the selected experts.
 *  - OCP 8-bit floating point specification (E4M3) for fp8 weights.
 *  - OCP Microscaling Formats (MX) specification v1.0 for MXFP4 expert weights
 *    (E2M1 elements, E8M0 block scales over 32 elements): "DeepSeek-V4.1-Flash
 *    breaks 1,000 tokens per second for one user", section "Appendix: method",
 *    names MXFP4 expert weights as the serving format, with an fp8 (E4M3) KV
 *    cache; the page gives no scale layout for the cache, and the reading taken
 *    is one power-of-two fp32 scale per cache row (orc_fp8_row_scale).
 *  - Verification: greedy (the byte-for-byte greedy gate of "DeepSeek-V4.1-Flash
 *    breaks 1,000 tokens per second for one user", section "The safety layer"),
 *    or sampled at a temperature with matched random draws (same section) and
 *    one rejection step per speculative step ("Why one GB300 ...", section
 *    "Where the 11.2 ms goes"): speculative sampling (Leviathan et al. 2023;
 *    Chen et al. 2023) with the drafts read as point proposals, token draws by
 *    the Gumbel-max trick, draws from SplitMix64 (Steele, Lea and Flood 2014).
 *    The LM head may be fp8 with 128x128 block scales (the fp8 head named as a
 *    small item in "Why one GB300 ...", section "Three readings").
 *
 *  - Layer variant: the low-rank query of the DeepSeek-V2 paper (section 2.1,
 *    c^Q = W_DQ x, q = W_UQ c^Q) with the q-norm named by the pages'
 *    "q-norm-rope-insert" kernel ("Why one GB300 ...", section "Where the
 *    11.2 ms goes") as an RMSNorm of c^Q with its own gain, and an RMSNorm of
 *    the latent before it is cached (the normalised compressed latents of the
 *    DeepSeek-V2 architecture); the RoPE key is not normalised.
 *
 *  - Sparse attention: the pages' sparse attention mode with an indexer
 *    ("Why one GB300 ...", sections "Where the 11.2 ms goes" and "Corrections
 *    to things we said") read as the lightning indexer and top-k selection of
 *    the DeepSeek-V3.2 report (index scores sum_j w_j relu(q_j . k_s), each
 *    query row attends to its top-k cache rows); no normalisation or RoPE of
 *    the index keys, which the cache rows carry after the RoPE key.
 *
 * Readings where the pages are silent (each listed in the design notes):
 * eps = 1e-6; softmax scale 1/sqrt(d_h + d_r); RoPE base 10000 with the angle
 * p * theta_j formed in double; selection by logit with ties to the lower
 * expert index; gates = softmax probabilities of the selected experts
 * renormalised to sum to 1; the shared expert is added with weight 1; new KV
 * rows are rounded to the cache's storage format and read back by attention.
 *
 * Arithmetic: weights are widened/dequantised exactly (fp8: (float)q * s;
 * MXFP4: E2M1(q) * 2^(e-127));
 * activations are fp32; every dot product accumulates in fp32 in increasing
 * index order.  The *_f64 entry points redo the layer in double precision in
 * the un-absorbed form (per-head keys and values expanded from the latent).
 */
#ifndef MK_ORACLE_H
#define MK_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8B128 = 2, ORC_MXFP4 = 3, ORC_FP8ROW = 4 };

typedef struct orc_cfg {
  int d;          /* hidden size */
  int n_h, d_h;   /* heads, per-head content dim */
  int d_c, d_r;   /* latent KV rank, decoupled RoPE dim (even) */
  int E, top_k;   /* routed experts, experts picked per token */
  int n_shared;   /* shared experts (always applied, weight 1) */
  int f;          /* expert FFN width */
  int attn_fmt;   /* ORC_F32 | ORC_BF16: W_Q, W_DKV, W_UK, W_UV, W_O, W_R */
  int exp_fmt;    /* ORC_F32 | ORC_BF16 | ORC_FP8B128 | ORC_MXFP4: W1, W3, W2 */
  int kv_fmt;     /* ORC_F32 | ORC_BF16 | ORC_FP8ROW (see orc_kv_row_bytes) */
  float eps;      /* RMSNorm epsilon */
  double rope_base;
  int q_lora;     /* 0: one W_Q; > 0: low-rank query of this rank, c^Q = W_DQ x,
                     q-norm (RMSNorm with gain gamma_q), q = W_UQ norm(c^Q) */
  int kv_norm;    /* 1: RMSNorm with gain gamma_kv on the latent c before it is cached */
  int idx_heads;  /* sparse attention (idx_topk > 0): indexer heads H_I, index key dim d_I,   */
  int idx_dim;    /*   keys kept per query row k; each cache row then holds its index key    */
  int idx_topk;   /*   after the latent and the RoPE key (d_c + d_r + d_I values; an fp8     */
                  /*   row holds them as d_c + d_r + d_I codes under the row's one scale)   */
} orc_cfg;

/* Canonical (row-major) weights.  Expert slot e in [0, E) is routed expert e,
 * slot E + s is shared expert s.  A NULL expert pointer is allowed for experts
 * no token selects; using one is an error (-3).
 *   W_Q   [n_h*(d_h+d_r)][d]   head h owns rows h*(d_h+d_r) ...: first d_h = q^C, last d_r = q^R
 *   W_DKV [d_c+d_r][d]         first d_c rows -> latent c, last d_r -> pre-RoPE shared key
 *   W_UK  [n_h][d_h][d_c]      k^C_h = W_UK[h] c
 *   W_UV  [n_h][d_h][d_c]      v_h   = W_UV[h] c
 *   W_O   [d][n_h*d_h]
 *   W_R   [E][d], router_bias [E] or NULL
 *   W1,W3 [f][d], W2 [d][f]; fp8 scales [ceil(rows/128)][ceil(cols/128)] fp32
 *   q_lora > 0 (the low-rank query of the DeepSeek-V2 paper, section 2.1, with
 *   the q-norm of the pages' q-norm-rope-insert kernel): W_DQ [q_lora][d],
 *   W_UQ [n_h*(d_h+d_r)][q_lora] in place of W_Q; kv_norm: gain [d_c].
 *   Sparse attention (idx_topk > 0): the lightning indexer of the DeepSeek-V3.2
 *   report (the pages' SparseAttnFwdMode and indexer) -- per query row t,
 *   q^I = W_IQ x [H_I][d_I], w^I = W_IW x [H_I], its index key k^I = W_IK x
 *   (cached with the row); score of cache row s <= pos: sum_j w^I_j *
 *   max(0, q^I_j . k^I_s); the row attends to the idx_topk highest-scoring
 *   rows (ties to the lower row; all rows when pos + 1 <= idx_topk).
 *   MXFP4 (OCP Microscaling Formats spec v1.0: E2M1 elements, one E8M0 scale
 *   per block of 32 consecutive elements): W1, W3, W2 as bytes [rows][cols/2],
 *   element 2j in the low nibble of byte j and 2j+1 in the high nibble; the
 *   scales s1, s3, s2 as bytes [rows][cols/32]; element value = E2M1(code) *
 *   2^(scale - 127), exact in fp32.  cols must be a multiple of 32. */
typedef struct orc_weights {
  const float* gamma1;
  const float* gamma2;
  const void* wq;
  const void* wdkv;
  const void* wuk;
  const void* wuv;
  const void* wo;
  const void* wr;
  const float* router_bias;
  const void* const* w1;
  const void* const* w3;
  const void* const* w2;
  const void* const* s1;    /* fp8: const float* scales; MXFP4: const uint8_t* E8M0 codes */
  const void* const* s3;
  const void* const* s2;
  const void* wdq;          /* q_lora > 0: W_DQ [q_lora][d], W_UQ [n_h*(d_h+d_r)][q_lora] (attn_fmt), */
  const void* wuq;          /*   gamma_q [q_lora] (W_Q is then unused)                                */
  const float* gamma_q;
  const float* gamma_kv;    /* kv_norm: [d_c] */
  const void* widx;         /* sparse: [W_IQ; W_IW; W_IK] rows [H_I*d_I + H_I + d_I][d] (attn_fmt) */
  const int32_t* force_isel;/* sparse, optional: kept rows [T][idx_topk] to use instead of the
                               selection (the scores are still computed and tapped) */
} orc_weights;

/* Optional intermediate outputs (any pointer may be NULL). */
typedef struct orc_attn_taps {
  float* x;     /* [T][d]                 RMSNorm-1 output                        */
  float* q;     /* [T][n_h][d_h+d_r]      per-head q^C and RoPE-rotated q^R       */
  float* ckv;   /* [T][d_c+d_r]           latent c and RoPE-rotated key (unrounded) */
  float* qabs;  /* [T][n_h][d_c]          absorbed query q~                       */
  float* z;     /* [T][n_h][d_c]          attention-weighted latent               */
  float* o;     /* [T][n_h*d_h]           per-head value up-projection            */
  int32_t* sel; /* [T][idx_topk]          sparse: kept cache rows, ascending, -1 padded */
  float* iscore;/* [T][L+T]               sparse: index scores (row i: 0 .. L+i)   */
} orc_attn_taps;

typedef struct orc_moe_taps {
  float* xp;       /* [T][d]        RMSNorm-2 output                 */
  float* logits;   /* [T][E]        router logits (bias included)    */
  int32_t* sel;    /* [T][top_k]    selected experts, best first     */
  float* gate;     /* [T][top_k]    renormalised gate weights        */
  float* y_sel;    /* [T][top_k][d] expert outputs of the picks      */
  float* y_shared; /* [T][d]        sum of shared-expert outputs     */
} orc_moe_taps;

/* KV cache rows of kvw values (d_c+d_r, plus d_I with sparse attention).
 * ORC_F32 / ORC_BF16: kvw elements.  ORC_FP8ROW: the row's kvw E4M3 codes
 * (orc_f32_to_e4m3 of value / scale), then its scale as an
 * fp32 (orc_fp8_row_scale, a power of two), zero bytes up to a multiple of 16;
 * element value = E4M3(code) * scale, exact in fp32.  Bytes per row (-1 for an
 * unknown format): */
int orc_kv_row_bytes(int kv_fmt, int kvw);
/* Rows [0, nrows) of a cache as fp32 values [nrows][kvw]. */
int orc_kv_decode_rows(const void* kv, int kv_fmt, int kvw, int nrows, float* out);

/* Attention block: Hp = H + W_O(attention).  Writes KV rows [L, L+T) of `kv`
 * ([capacity] rows in kv_fmt) and reads rows [0, L+i] for verify row i.
 * Returns 0, or a negative code on bad arguments. */
int orc_attn_block(const orc_cfg* c, const orc_weights* w, const float* H, int T,
                   void* kv, int L, float* Hp, const orc_attn_taps* taps);

/* Router only: x' = RMSNorm(Hp)*gamma2, logits, top-k selection and gates. */
int orc_router(const orc_cfg* c, const orc_weights* w, const float* Hp, int T,
               float* xp, float* logits, int32_t* sel, float* gate);

/* MoE block: out = Hp + sum_t gate_t * expert_{sel_t}(x') + sum_s shared_s(x').
 * If force_sel is non-NULL ([T][top_k]) the selection is taken from it and the
 * gates are recomputed from the logits for those experts. */
int orc_moe_block(const orc_cfg* c, const orc_weights* w, const float* Hp, int T,
                  const int32_t* force_sel, float* out, const orc_moe_taps* taps);

/* Whole layer = attention block then MoE block. */
int orc_layer_step(const orc_cfg* c, const orc_weights* w, const float* H, int T,
                   void* kv, int L, float* out, const orc_attn_taps* at, const orc_moe_taps* mt);

/* Double-precision brute force of the whole layer, un-absorbed form.  Reads
 * KV rows [0, L) from `kv` (not modified); the new rows are rounded to kv_fmt
 * (as the cache stores them) and written to kv_new_f64 ([T][d_c+d_r], may be
 * NULL).  force_sel as in orc_moe_block.  Outputs in double. */
int orc_layer_step_f64(const orc_cfg* c, const orc_weights* w, const float* H, int T,
                       const void* kv, int L, const int32_t* force_sel,
                       double* out, double* hp_out, double* kv_new_f64, double* logits_out,
                       int32_t* sel_out);

/* Stack pieces (bf16 tables [V][d]).  h[i] = Emb[tokens[i]] widened to fp32. */
int orc_embed(const uint16_t* emb, int V, int d, const int32_t* tokens, int T, float* h);
/* logits[i] = W_head (RMSNorm(h_i) * gamma_f), fp32; argmax with ties to the lower id. */
int orc_head(const uint16_t* head, int V, int d, const float* gamma_f, float eps,
             const float* h, int T, float* logits, int32_t* argmax);
/* The same in a weight format: ORC_BF16 (scales NULL) or ORC_FP8B128 (E4M3
 * codes [V][d], fp32 scales [ceil(V/128)][ceil(d/128)]). */
int orc_head_fmt(const void* head, int fmt, const float* scales, int V, int d, const float* gamma_f, float eps,
                 const float* h, int T, float* logits, int32_t* argmax);
/* Sampled verification (temperature tau > 0) with the step's draws made from
 * a 64-bit key: see oracle.c.  tokens = t0, d_1 .. d_{T-1}.  Writes sample[T]
 * (row i's Gumbel-max draw from softmax(logits_i / tau)) and committed[1 + T]
 * (count n+1, then d_1..d_n and the final draw); returns n+1, or -1. */
int orc_verify_sampled(const float* logits, int V, int T, const int32_t* tokens, float tau, uint64_t key,
                       int32_t* sample, int32_t* committed);
uint64_t orc_splitmix64_mix(uint64_t z);
uint64_t orc_sample_key(uint64_t seed, uint32_t step);      /* mix(seed + (step + 1) gamma) */
float orc_sample_uniform(uint64_t key, uint64_t i);         /* ((mix(key + (i+1) gamma) >> 41) + 1/2) 2^-23 */
/* Greedy verification.  tokens = t0, d_1 .. d_{T-1}; a = argmax per row.
 * n = largest n <= T-1 with d_j == a_{j-1} for every j <= n.  Commits n+1 tokens
 * (d_1..d_n, a_n) into committed[0..n]; returns n+1. */
int orc_greedy_accept(const int32_t* tokens, const int32_t* a, int T, int32_t* committed);

/* Format helpers, exposed for the tests. */
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float x);
float orc_e4m3_to_f32(uint8_t q);
uint8_t orc_f32_to_e4m3(float x);      /* RNE, saturating at +-448, NaN -> 0x7F */
float orc_fp8_row_scale(const float* row, int n);   /* smallest 2^e >= amax / 448; 1 for a zero row */
float orc_e2m1_to_f32(uint8_t code);   /* low 4 bits: S.EE.M, bias 1 */
float orc_e8m0_to_f32(uint8_t e);      /* 2^(e-127); 255 is NaN */

#ifdef __cplusplus
}
#endif
#endif
