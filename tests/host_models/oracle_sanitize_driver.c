/* Drives the CPU oracle and the host build of the seeded generator through
 * every entry point on small shapes, in every storage format, plus their
 * argument checks -- built with AddressSanitizer and UndefinedBehaviorSanitizer
 * by tests/test_host_sanitizers.py (test infrastructure; the numbers are
 * checked elsewhere, here only that nothing reads or writes out of bounds or
 * hits undefined behaviour).  Exit status 0 when every call returned what it
 * should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"
#include "../../synth/synth.h"

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static const float kSigma = 0.02f;
static float sigma_c(float s) { return s * 1.7320508f / 65536.0f; }

/* a tensor of n elements in format fmt (0 f32, 1 bf16) */
static void* tensor(int fmt, size_t n, uint64_t stream, float sigma, float mean) {
  if (fmt == ORC_F32) {
    float* p = (float*)malloc(n * sizeof(float));
    mks_host_normal_f32(p, n, 0, stream, 0, sigma_c(sigma), mean);
    return p;
  }
  uint16_t* p = (uint16_t*)malloc(n * sizeof(uint16_t));
  mks_host_normal_bf16(p, n, 0, stream, 0, sigma_c(sigma), mean);
  return p;
}

/* one expert matrix [R][K] in the expert format, with its scales */
static void expert_matrix(int fmt, int R, int K, uint64_t stream, void** w, void** s) {
  *s = NULL;
  if (fmt == ORC_FP8B128) {
    const int nb = ((R + 127) / 128) * ((K + 127) / 128);
    *w = malloc((size_t)R * K);
    *s = malloc((size_t)nb * sizeof(float));
    mks_host_fp8_blocks((uint8_t*)*w, (float*)*s, R, K, 0, stream, sigma_c(kSigma));
  } else if (fmt == ORC_MXFP4) {
    *w = malloc((size_t)R * K / 2);
    *s = malloc((size_t)R * K / 32);
    mks_host_mxfp4_blocks((uint8_t*)*w, (uint8_t*)*s, R, K, 0, stream, sigma_c(kSigma));
  } else {
    *w = tensor(fmt, (size_t)R * K, stream, kSigma, 0.f);
  }
}

static void run_layer(int attn_fmt, int exp_fmt, int kv_fmt, int with_bias) {
  orc_cfg c;
  memset(&c, 0, sizeof c);
  c.d = 64; c.n_h = 2; c.d_h = 16; c.d_c = 32; c.d_r = 8; c.E = 4; c.top_k = 2; c.n_shared = 1; c.f = 64;
  c.attn_fmt = attn_fmt; c.exp_fmt = exp_fmt; c.kv_fmt = kv_fmt; c.eps = 1e-6f; c.rope_base = 10000.0;
  const int T = 3, L = 5, cap = L + T, kvw = c.d_c + c.d_r, NE = c.E + c.n_shared;
  orc_weights w;
  memset(&w, 0, sizeof w);
  uint64_t st = 1;
  w.gamma1 = (const float*)tensor(ORC_F32, c.d, st++, 0.1f, 1.f);
  w.gamma2 = (const float*)tensor(ORC_F32, c.d, st++, 0.1f, 1.f);
  w.wq = tensor(attn_fmt, (size_t)c.n_h * (c.d_h + c.d_r) * c.d, st++, kSigma, 0.f);
  w.wdkv = tensor(attn_fmt, (size_t)kvw * c.d, st++, kSigma, 0.f);
  w.wuk = tensor(attn_fmt, (size_t)c.n_h * c.d_h * c.d_c, st++, kSigma, 0.f);
  w.wuv = tensor(attn_fmt, (size_t)c.n_h * c.d_h * c.d_c, st++, kSigma, 0.f);
  w.wo = tensor(attn_fmt, (size_t)c.d * c.n_h * c.d_h, st++, kSigma, 0.f);
  w.wr = tensor(attn_fmt, (size_t)c.E * c.d, st++, kSigma, 0.f);
  float* bias = NULL;
  if (with_bias) {
    bias = (float*)tensor(ORC_F32, c.E, st++, 1.f, 0.f);
    w.router_bias = bias;
  }
  void* w1[8]; void* w3[8]; void* w2[8]; void* s1[8]; void* s3[8]; void* s2[8];
  for (int e = 0; e < NE; ++e) {
    expert_matrix(exp_fmt, c.f, c.d, st++, &w1[e], &s1[e]);
    expert_matrix(exp_fmt, c.f, c.d, st++, &w3[e], &s3[e]);
    expert_matrix(exp_fmt, c.d, c.f, st++, &w2[e], &s2[e]);
  }
  w.w1 = (const void* const*)w1; w.w3 = (const void* const*)w3; w.w2 = (const void* const*)w2;
  w.s1 = (const void* const*)s1; w.s3 = (const void* const*)s3; w.s2 = (const void* const*)s2;
  float* H = (float*)tensor(ORC_F32, (size_t)T * c.d, st++, 1.f, 0.f);
  void* kv = tensor(kv_fmt, (size_t)cap * kvw, st++, 1.f, 0.f);
  void* kv2 = malloc((size_t)cap * kvw * (kv_fmt == ORC_F32 ? 4 : 2));
  memcpy(kv2, kv, (size_t)cap * kvw * (kv_fmt == ORC_F32 ? 4 : 2));
  float* out = (float*)malloc((size_t)T * c.d * sizeof(float));
  float* taps[12];
  const size_t tsz[12] = {(size_t)T * c.d, (size_t)T * c.n_h * (c.d_h + c.d_r), (size_t)T * kvw,
                          (size_t)T * c.n_h * c.d_c, (size_t)T * c.n_h * c.d_c, (size_t)T * c.n_h * c.d_h,
                          (size_t)T * c.d, (size_t)T * c.E, (size_t)T * c.top_k, (size_t)T * c.top_k,
                          (size_t)T * c.top_k * c.d, (size_t)T * c.d};
  for (int i = 0; i < 12; ++i) taps[i] = (float*)malloc(tsz[i] * sizeof(float));
  orc_attn_taps at = {taps[0], taps[1], taps[2], taps[3], taps[4], taps[5]};
  orc_moe_taps mt = {taps[6], taps[7], (int32_t*)taps[8], taps[9], taps[10], taps[11]};
  CHECK(orc_layer_step(&c, &w, H, T, kv, L, out, &at, &mt) == 0);
  for (int i = 0; i < T * c.d; ++i) CHECK(isfinite(out[i]));
  /* the same step in double precision, with the oracle's selection forced */
  double* o64 = (double*)malloc((size_t)T * c.d * sizeof(double));
  double* hp64 = (double*)malloc((size_t)T * c.d * sizeof(double));
  double* kvn = (double*)malloc((size_t)T * kvw * sizeof(double));
  double* lg = (double*)malloc((size_t)T * c.E * sizeof(double));
  int32_t sel64[3 * 2];
  CHECK(orc_layer_step_f64(&c, &w, H, T, kv2, L, (const int32_t*)taps[8], o64, hp64, kvn, lg, sel64) == 0);
  /* router and MoE block on their own */
  float* xp = (float*)malloc((size_t)T * c.d * sizeof(float));
  float* logits = (float*)malloc((size_t)T * c.E * sizeof(float));
  int32_t sel[3 * 2];
  float gate[3 * 2];
  CHECK(orc_router(&c, &w, out, T, xp, logits, sel, gate) == 0);
  for (int t = 0; t < T; ++t) {
    float sg = 0.f;
    for (int k = 0; k < c.top_k; ++k) {
      CHECK(sel[t * c.top_k + k] >= 0 && sel[t * c.top_k + k] < c.E);
      sg += gate[t * c.top_k + k];
    }
    CHECK(fabsf(sg - 1.f) < 1e-5f);
  }
  CHECK(orc_moe_block(&c, &w, out, T, sel, xp, NULL) == 0);
  /* argument checks */
  CHECK(orc_layer_step(NULL, &w, H, T, kv, L, out, NULL, NULL) < 0);
  CHECK(orc_layer_step(&c, &w, H, 0, kv, L, out, NULL, NULL) == 0);   /* no rows: nothing to do */
  CHECK(orc_layer_step(&c, &w, H, -1, kv, L, out, NULL, NULL) < 0);
  CHECK(orc_layer_step(&c, &w, H, T, kv, -1, out, NULL, NULL) < 0);
  orc_weights w0 = w;
  w0.w1 = NULL;
  CHECK(orc_moe_block(&c, &w0, out, T, NULL, xp, NULL) < 0);
  for (int i = 0; i < 12; ++i) free(taps[i]);
  free(o64); free(hp64); free(kvn); free(lg); free(xp); free(logits);
  for (int e = 0; e < NE; ++e) { free(w1[e]); free(w3[e]); free(w2[e]); free(s1[e]); free(s3[e]); free(s2[e]); }
  free((void*)w.gamma1); free((void*)w.gamma2); free((void*)w.wq); free((void*)w.wdkv); free((void*)w.wuk);
  free((void*)w.wuv); free((void*)w.wo); free((void*)w.wr); free(bias); free(H); free(kv); free(kv2); free(out);
}

static void run_stack_pieces(void) {
  const int V = 48, d = 64, T = 4;
  uint16_t* emb = (uint16_t*)tensor(ORC_BF16, (size_t)V * d, 101, 0.02f, 0.f);
  uint16_t* head = (uint16_t*)tensor(ORC_BF16, (size_t)V * d, 102, 0.02f, 0.f);
  float* gf = (float*)tensor(ORC_F32, d, 103, 0.1f, 1.f);
  int32_t tokens[4] = {3, 17, 0, 47};
  float* h = (float*)malloc((size_t)T * d * sizeof(float));
  float* logits = (float*)malloc((size_t)T * V * sizeof(float));
  int32_t am[4], committed[5];
  CHECK(orc_embed(emb, V, d, tokens, T, h) == 0);
  CHECK(orc_head(head, V, d, gf, 1e-6f, h, T, logits, am) == 0);
  for (int t = 0; t < T; ++t) CHECK(am[t] >= 0 && am[t] < V);
  const int n = orc_greedy_accept(tokens, am, T, committed);
  CHECK(n >= 1 && n <= T);
  int32_t smp[4], com[5];
  const int ns = orc_verify_sampled(logits, V, T, tokens, 0.7f, orc_sample_key(5, 2), smp, com);
  CHECK(ns >= 1 && ns <= T && com[0] == ns);
  CHECK(orc_verify_sampled(logits, V, T, tokens, 0.f, 1, smp, com) < 0);
  uint8_t* codes = (uint8_t*)malloc((size_t)V * d);
  float scales[1] = {0.01f};
  for (int i = 0; i < V * d; ++i) codes[i] = (uint8_t)(i * 37 % 126);
  CHECK(orc_head_fmt(codes, ORC_FP8B128, scales, V, d, gf, 1e-6f, h, T, logits, am) == 0);
  CHECK(orc_head_fmt(codes, ORC_FP8B128, NULL, V, d, gf, 1e-6f, h, T, logits, am) < 0);
  free(codes);
  int32_t bad[1] = {V};
  CHECK(orc_embed(emb, V, d, bad, 1, h) < 0);
  free(emb); free(head); free(gf); free(h); free(logits);
}

static void run_generator(void) {
  uint64_t r[37];
  mks_host_raw_fill(r, 37, 5, 9, 123);
  CHECK(r[0] == mks_host_raw(5, 9, 123));
  /* ragged fp8 blocks and MXFP4 rows */
  const int shapes[4][2] = {{129, 1}, {1, 257}, {300, 200}, {17, 96}};
  for (int i = 0; i < 4; ++i) {
    const int R = shapes[i][0], K = shapes[i][1];
    const int nb = ((R + 127) / 128) * ((K + 127) / 128);
    uint8_t* q = (uint8_t*)malloc((size_t)R * K);
    float* s = (float*)malloc((size_t)nb * sizeof(float));
    mks_host_fp8_blocks(q, s, R, K, 0, 7, sigma_c(kSigma));
    for (int b = 0; b < nb; ++b) CHECK(s[b] > 0.f);
    free(q); free(s);
    if (K % 32 == 0) {
      uint8_t* c4 = (uint8_t*)malloc((size_t)R * K / 2);
      uint8_t* e8 = (uint8_t*)malloc((size_t)R * K / 32);
      mks_host_mxfp4_blocks(c4, e8, R, K, 0, 8, sigma_c(kSigma));
      free(c4); free(e8);
    }
  }
  /* encoders at special values */
  const float xs[] = {0.f, -0.f, 1e-30f, 448.f, 1e9f, -1e9f, 6.f, 7.f, NAN, INFINITY};
  for (unsigned i = 0; i < sizeof xs / sizeof xs[0]; ++i) {
    (void)mks_host_e4m3_encode(xs[i]);
    (void)mks_host_e2m1_encode(xs[i]);
    (void)mks_host_bf16_encode(xs[i]);
  }
  CHECK(mks_host_e2m1_encode(6.f) == 7);
  CHECK(mks_host_e2m1_encode(-6.f) == 15);
}

int main(void) {
  const int fmts[5][3] = {{ORC_F32, ORC_F32, ORC_F32}, {ORC_BF16, ORC_BF16, ORC_BF16},
                          {ORC_BF16, ORC_FP8B128, ORC_BF16}, {ORC_BF16, ORC_MXFP4, ORC_BF16},
                          {ORC_F32, ORC_FP8B128, ORC_BF16}};
  for (int i = 0; i < 5; ++i)
    for (int b = 0; b < 2; ++b) run_layer(fmts[i][0], fmts[i][1], fmts[i][2], b);
  run_stack_pieces();
  run_generator();
  printf(g_fail ? "FAILED %d\n" : "oracle and generator: all calls clean\n", g_fail);
  return g_fail ? 1 : 0;
}
