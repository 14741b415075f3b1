/*
 * CPU ORACLE -- TEST INFRASTRUCTURE ONLY (see oracle.h for what it computes,
 * the passages it follows and the readings it takes).  Plain loops; every dot
 * product accumulates in increasing index order.  OpenMP only splits
 * independent output elements across threads, so results do not depend on
 * the thread count.  Build with -ffp-contract=off.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ formats */
float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* round to nearest, ties to even */
uint16_t orc_f32_to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* OCP E4M3: bias 7; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN. */
float orc_e4m3_to_f32(uint8_t q) {
  int s = q >> 7, e = (q >> 3) & 0xF, m = q & 7;
  if (e == 15 && m == 7) return NAN;
  float v = (e == 0) ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return s ? -v : v;
}

/* OCP E4M3 ("FN") encoding, round to nearest with ties to even, saturating at
 * +-448 (the largest finite value; S.1111.111 is NaN); NaN -> 0x7F.  Written
 * from the definition: a normal value is (1 + m/8) 2^(e-7), e = 1..15, a
 * subnormal m 2^-9. */
uint8_t orc_f32_to_e4m3(float x) {
  if (isnan(x)) return 0x7F;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {                       /* subnormal range: steps of 2^-9 */
    const int m = (int)rint(a * 512.0);           /* m = 8 is the smallest normal, code 0x08 */
    return sign | (uint8_t)m;
  }
  int k;
  frexp(a, &k);                                   /* a = f 2^k, f in [0.5, 1) */
  int E = k - 1;                                  /* a in [2^E, 2^(E+1)) */
  int m = (int)rint((a / ldexp(1.0, E) - 1.0) * 8.0);
  if (m == 8) {
    m = 0;
    ++E;
  }
  if (E + 7 > 15 || (E + 7 == 15 && m == 7)) return sign | 0x7E;
  return sign | (uint8_t)(((E + 7) << 3) | m);
}

/* Scale of one fp8 KV row: the smallest power of two 2^e with amax <= 448 2^e
 * (1 when the row is all zeros), so that row / scale fits E4M3 without
 * saturating and code * scale is exact in fp32 (and in bf16). */
float orc_fp8_row_scale(const float* row, int n) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) amax = fmax(amax, fabs((double)row[i]));
  if (amax == 0.0) return 1.0f;
  int e = ilogb(amax) - 8;
  while (amax > ldexp(448.0, e)) ++e;
  while (amax <= ldexp(448.0, e - 1)) --e;
  return ldexpf(1.0f, e);
}

int orc_kv_row_bytes(int kv_fmt, int kvw) {
  if (kv_fmt == ORC_F32) return 4 * kvw;
  if (kv_fmt == ORC_BF16) return 2 * kvw;
  if (kv_fmt == ORC_FP8ROW) return (kvw + 4 + 15) / 16 * 16;
  return -1;
}

/* OCP MX E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field
 * 0 is subnormal (m * 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
float orc_e2m1_to_f32(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  float v = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
  return s ? -v : v;
}

/* OCP MX E8M0 scale: 2^(e - 127); the code 255 is NaN. */
float orc_e8m0_to_f32(uint8_t e) { return e == 255 ? NAN : ldexpf(1.0f, (int)e - 127); }

static float e4m3_lut[256];
static float e2m1_lut[16];
static float e8m0_lut[256];
static int e4m3_lut_ready = 0;
static void lut_init(void) {
  if (!e4m3_lut_ready) {
    for (int i = 0; i < 256; ++i) e4m3_lut[i] = orc_e4m3_to_f32((uint8_t)i);
    for (int i = 0; i < 16; ++i) e2m1_lut[i] = orc_e2m1_to_f32((uint8_t)i);
    for (int i = 0; i < 256; ++i) e8m0_lut[i] = orc_e8m0_to_f32((uint8_t)i);
    e4m3_lut_ready = 1;
  }
}

/* A weight matrix in one of the storage formats. */
typedef struct {
  const void* p;
  int fmt;
  const void* s; /* fp8: fp32 block scales; MXFP4: E8M0 codes */
  long rows, cols;
} wmat;

static wmat mk_wmat(const void* p, int fmt, const void* s, long rows, long cols) {
  wmat m = {p, fmt, s, rows, cols};
  return m;
}

/* element (r, k) widened to fp32 exactly (fp8: fp32 product of code and scale;
 * MXFP4: E2M1 value times a power of two) */
static inline float wat(const wmat* m, long r, long k) {
  long i = r * m->cols + k;
  if (m->fmt == ORC_F32) return ((const float*)m->p)[i];
  if (m->fmt == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)m->p)[i]);
  if (m->fmt == ORC_MXFP4) {
    uint8_t b = ((const uint8_t*)m->p)[r * (m->cols / 2) + k / 2];
    uint8_t code = (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
    return e2m1_lut[code] * e8m0_lut[((const uint8_t*)m->s)[r * (m->cols / 32) + k / 32]];
  }
  long nbk = (m->cols + 127) / 128;
  return e4m3_lut[((const uint8_t*)m->p)[i]] * ((const float*)m->s)[(r / 128) * nbk + k / 128];
}
static inline double wat64(const wmat* m, long r, long k) {
  if (m->fmt == ORC_MXFP4) return (double)wat(m, r, k);     /* exact in fp32 */
  long i = r * m->cols + k;
  if (m->fmt == ORC_F32) return (double)((const float*)m->p)[i];
  if (m->fmt == ORC_BF16) return (double)orc_bf16_to_f32(((const uint16_t*)m->p)[i]);
  long nbk = (m->cols + 127) / 128;
  return (double)e4m3_lut[((const uint8_t*)m->p)[i]] * (double)((const float*)m->s)[(r / 128) * nbk + k / 128];
}

/* y = W x, fp32, sequential over k */
static void matvec(const wmat* m, const float* x, float* y) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < m->rows; ++r) {
    float acc = 0.0f;
    if (m->fmt == ORC_F32) {
      const float* w = (const float*)m->p + r * m->cols;
      for (long k = 0; k < m->cols; ++k) acc += w[k] * x[k];
    } else if (m->fmt == ORC_BF16) {
      const uint16_t* w = (const uint16_t*)m->p + r * m->cols;
      for (long k = 0; k < m->cols; ++k) acc += orc_bf16_to_f32(w[k]) * x[k];
    } else {
      for (long k = 0; k < m->cols; ++k) acc += wat(m, r, k) * x[k];
    }
    y[r] = acc;
  }
}

static void matvec64(const wmat* m, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < m->rows; ++r) {
    double acc = 0.0;
    for (long k = 0; k < m->cols; ++k) acc += wat64(m, r, k) * x[k];
    y[r] = acc;
  }
}

/* ------------------------------------------------------------------ pieces */
/* RMSNorm: x_k = (h_k * (1/sqrt(mean(h^2) + eps))) * gamma_k */
static void rmsnorm(const float* h, const float* gamma, int d, float eps, float* x) {
  float ss = 0.0f;
  for (int k = 0; k < d; ++k) ss += h[k] * h[k];
  float r = 1.0f / sqrtf(ss / (float)d + eps);
  for (int k = 0; k < d; ++k) x[k] = (h[k] * r) * gamma[k];
}
static void rmsnorm64(const float* h, const float* gamma, int d, double eps, double* x) {
  double ss = 0.0;
  for (int k = 0; k < d; ++k) ss += (double)h[k] * (double)h[k];
  double r = 1.0 / sqrt(ss / (double)d + eps);
  for (int k = 0; k < d; ++k) x[k] = ((double)h[k] * r) * (double)gamma[k];
}
static void rmsnorm64d(const double* h, const float* gamma, int d, double eps, double* x) {
  double ss = 0.0;
  for (int k = 0; k < d; ++k) ss += h[k] * h[k];
  double r = 1.0 / sqrt(ss / (double)d + eps);
  for (int k = 0; k < d; ++k) x[k] = (h[k] * r) * (double)gamma[k];
}

/* RoPE, adjacent pairs: theta_j = base^(-2j/d_r), angle p*theta_j in double. */
static void rope(float* v, int d_r, long pos, double base) {
  for (int j = 0; j < d_r / 2; ++j) {
    double th = pow(base, -2.0 * (double)j / (double)d_r);
    double a = (double)pos * th;
    float c = (float)cos(a), s = (float)sin(a);
    float v0 = v[2 * j], v1 = v[2 * j + 1];
    v[2 * j] = v0 * c - v1 * s;
    v[2 * j + 1] = v0 * s + v1 * c;
  }
}
static void rope64(double* v, int d_r, long pos, double base) {
  for (int j = 0; j < d_r / 2; ++j) {
    double th = pow(base, -2.0 * (double)j / (double)d_r);
    double a = (double)pos * th;
    double c = cos(a), s = sin(a);
    double v0 = v[2 * j], v1 = v[2 * j + 1];
    v[2 * j] = v0 * c - v1 * s;
    v[2 * j + 1] = v0 * s + v1 * c;
  }
}

/* element m of cache row `row` (kvw elements per row) */
static inline float kv_get(const void* kv, int fmt, int kvw, long row, int m) {
  if (fmt == ORC_F32) return ((const float*)kv)[row * kvw + m];
  if (fmt == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)kv)[row * kvw + m]);
  const uint8_t* r = (const uint8_t*)kv + row * orc_kv_row_bytes(fmt, kvw);
  float sc;
  memcpy(&sc, r + kvw, 4);
  return orc_e4m3_to_f32(r[m]) * sc;
}
/* stores one row (rounded to the cache's format: per element for fp32 / bf16,
 * with the row's scale for fp8) */
static void kv_put_row(void* kv, int fmt, int kvw, long row, const float* v) {
  if (fmt == ORC_F32) {
    memcpy((float*)kv + row * kvw, v, sizeof(float) * kvw);
  } else if (fmt == ORC_BF16) {
    for (int m = 0; m < kvw; ++m) ((uint16_t*)kv)[row * kvw + m] = orc_f32_to_bf16(v[m]);
  } else {
    uint8_t* r = (uint8_t*)kv + row * orc_kv_row_bytes(fmt, kvw);
    const float sc = orc_fp8_row_scale(v, kvw);
    for (int m = 0; m < kvw; ++m) r[m] = orc_f32_to_e4m3(v[m] / sc);
    memcpy(r + kvw, &sc, 4);
    memset(r + kvw + 4, 0, (size_t)(orc_kv_row_bytes(fmt, kvw) - kvw - 4));
  }
}
/* a row as the cache would give it back after storing it */
static void kv_round_row(int fmt, int kvw, const float* v, float* out) {
  if (fmt == ORC_F32) {
    memcpy(out, v, sizeof(float) * kvw);
  } else if (fmt == ORC_BF16) {
    for (int m = 0; m < kvw; ++m) out[m] = orc_bf16_to_f32(orc_f32_to_bf16(v[m]));
  } else {
    const float sc = orc_fp8_row_scale(v, kvw);
    for (int m = 0; m < kvw; ++m) out[m] = orc_e4m3_to_f32(orc_f32_to_e4m3(v[m] / sc)) * sc;
  }
}

int orc_kv_decode_rows(const void* kv, int kv_fmt, int kvw, int nrows, float* out) {
  if (!kv || !out || kvw <= 0 || nrows < 0 || orc_kv_row_bytes(kv_fmt, kvw) < 0) return -1;
  for (long j = 0; j < nrows; ++j)
    for (int m = 0; m < kvw; ++m) out[j * kvw + m] = kv_get(kv, kv_fmt, kvw, j, m);
  return 0;
}

static float silu(float u) { return u / (1.0f + expf(-u)); }
static double silu64(double u) { return u / (1.0 + exp(-u)); }

static int check_cfg(const orc_cfg* c, int T) {
  if (!c || T < 0 || c->d <= 0 || c->n_h <= 0 || c->d_h <= 0 || c->d_c <= 0 || c->d_r <= 0 ||
      (c->d_r & 1) || c->E <= 0 || c->top_k <= 0 || c->top_k > c->E || c->f <= 0 || c->n_shared < 0)
    return -1;
  if (c->exp_fmt == ORC_MXFP4 && (c->d % 32 || c->f % 32)) return -1;
  if (c->kv_fmt != ORC_F32 && c->kv_fmt != ORC_BF16 && c->kv_fmt != ORC_FP8ROW) return -1;
  if (c->q_lora < 0 || (c->kv_norm != 0 && c->kv_norm != 1)) return -1;
  return 0;
}
static int check_lowrank(const orc_cfg* c, const orc_weights* w) {
  if (c->idx_topk < 0 || (c->idx_topk > 0 && (c->idx_heads <= 0 || c->idx_dim <= 0 || !w->widx)))
    return -1;
  if (c->q_lora > 0 && (!w->wdq || !w->wuq || !w->gamma_q)) return -1;
  if (c->kv_norm && !w->gamma_kv) return -1;
  if (c->q_lora == 0 && !w->wq) return -1;
  return 0;
}

/* ------------------------------------------------------------------ sparse attention */
/* row `row` of a row-major [rows][cols] matrix in format fmt (fp32 or bf16) */
static const void* mat_row(const void* p, int fmt, long row, long cols) {
  return fmt == ORC_F32 ? (const void*)((const float*)p + row * cols) : (const void*)((const uint16_t*)p + row * cols);
}
typedef struct { double v; long i; } scored;
static int by_score_desc(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->v != y->v) return x->v > y->v ? -1 : 1;
  return x->i < y->i ? -1 : (x->i > y->i ? 1 : 0);
}
static int by_index(const void* a, const void* b) {
  const long x = *(const long*)a, y = *(const long*)b;
  return x < y ? -1 : (x > y ? 1 : 0);
}
/* The kept rows of a query row at position pos: all rows 0..pos when pos + 1 <= k,
 * else the k highest scores (ties to the lower row), in ascending row order.
 * Returns how many. */
static long select_rows(const double* score, long pos, int k, long* out) {
  const long n = pos + 1;
  if (n <= k) {
    for (long j = 0; j < n; ++j) out[j] = j;
    return n;
  }
  scored* a = malloc(sizeof(scored) * n);
  for (long j = 0; j < n; ++j) { a[j].v = score[j]; a[j].i = j; }
  qsort(a, (size_t)n, sizeof(scored), by_score_desc);
  for (int t = 0; t < k; ++t) out[t] = a[t].i;
  free(a);
  qsort(out, (size_t)k, sizeof(long), by_index);
  return k;
}

/* ------------------------------------------------------------------ attention */
int orc_attn_block(const orc_cfg* c, const orc_weights* w, const float* H, int T,
                   void* kv, int L, float* Hp, const orc_attn_taps* taps) {
  if (check_cfg(c, T) || !w || !H || !kv || !Hp || L < 0 || check_lowrank(c, w)) return -1;
  const int d = c->d, nh = c->n_h, dh = c->d_h, dc = c->d_c, dr = c->d_r, ql = c->q_lora;
  const int qw = dh + dr, kvw = dc + dr;
  wmat WQ = mk_wmat(w->wq, c->attn_fmt, NULL, (long)nh * qw, d);
  wmat WDQ = mk_wmat(w->wdq, c->attn_fmt, NULL, ql, d);
  wmat WUQ = mk_wmat(w->wuq, c->attn_fmt, NULL, (long)nh * qw, ql);
  wmat WD = mk_wmat(w->wdkv, c->attn_fmt, NULL, kvw, d);
  wmat WO = mk_wmat(w->wo, c->attn_fmt, NULL, d, (long)nh * dh);
  const float scale = (float)(1.0 / sqrt((double)(dh + dr)));

  float* cq = malloc(sizeof(float) * (ql > 0 ? ql : 1));
  float* cqn = malloc(sizeof(float) * (ql > 0 ? ql : 1));
  float* cn = malloc(sizeof(float) * dc);
  /* sparse attention: the indexer's projections and the row width with the index key */
  const int sparse = c->idx_topk > 0, HI = c->idx_heads, dI = c->idx_dim, KI = c->idx_topk;
  const int rw = kvw + (sparse ? dI : 0);
  wmat WIQ = mk_wmat(sparse ? w->widx : NULL, c->attn_fmt, NULL, (long)HI * dI, d);
  wmat WIW = mk_wmat(sparse ? mat_row(w->widx, c->attn_fmt, (long)HI * dI, d) : NULL, c->attn_fmt, NULL, HI, d);
  wmat WIK = mk_wmat(sparse ? mat_row(w->widx, c->attn_fmt, (long)HI * dI + HI, d) : NULL, c->attn_fmt, NULL, dI, d);
  float* qi = malloc(sizeof(float) * (sparse ? (long)HI * dI : 1));
  float* wi = malloc(sizeof(float) * (sparse ? HI : 1));
  double* isc = malloc(sizeof(double) * ((long)L + T));
  long* sel = malloc(sizeof(long) * ((long)L + T));
  float* x = malloc(sizeof(float) * d);
  float* q = malloc(sizeof(float) * nh * qw);
  float* ckv = malloc(sizeof(float) * rw);
  float* qa = malloc(sizeof(float) * nh * dc);
  float* z = malloc(sizeof(float) * nh * dc);
  float* o = malloc(sizeof(float) * nh * dh);
  float* att = malloc(sizeof(float) * d);
  lut_init();
  for (int i = 0; i < T; ++i) {
    const long pos = (long)L + i;
    rmsnorm(H + (long)i * d, w->gamma1, d, c->eps, x);
    if (ql > 0) {
      /* low-rank query: c^Q = W_DQ x, q-norm, q = W_UQ norm(c^Q) */
      matvec(&WDQ, x, cq);
      rmsnorm(cq, w->gamma_q, ql, c->eps, cqn);
      matvec(&WUQ, cqn, q);
    } else {
      matvec(&WQ, x, q);
    }
    matvec(&WD, x, ckv);
    if (c->kv_norm) {
      /* the latent is normalised before it is cached (the RoPE key is not) */
      rmsnorm(ckv, w->gamma_kv, dc, c->eps, cn);
      memcpy(ckv, cn, sizeof(float) * dc);
    }
    for (int h = 0; h < nh; ++h) rope(q + (long)h * qw + dh, dr, pos, c->rope_base);
    rope(ckv + dc, dr, pos, c->rope_base);
    if (sparse) matvec(&WIK, x, ckv + kvw);     /* the row's index key, cached with it */
    kv_put_row(kv, c->kv_fmt, rw, pos, ckv);
    /* the rows this query row attends to */
    long nsel = pos + 1;
    if (sparse) {
      matvec(&WIQ, x, qi);
      matvec(&WIW, x, wi);
#pragma omp parallel for schedule(static)
      for (long j = 0; j <= pos; ++j) {
        float sc = 0.0f;
        for (int hh = 0; hh < HI; ++hh) {
          float dot = 0.0f;
          for (int m = 0; m < dI; ++m) dot += qi[(long)hh * dI + m] * kv_get(kv, c->kv_fmt, rw, j, kvw + m);
          if (dot > 0.0f) sc += wi[hh] * dot;
        }
        isc[j] = (double)sc;
        if (taps && taps->iscore) taps->iscore[(long)i * (L + T) + j] = sc;
      }
      nsel = select_rows(isc, pos, KI, sel);
      if (w->force_isel)
        for (long u = 0; u < nsel; ++u) sel[u] = w->force_isel[(long)i * KI + u];
      if (taps && taps->sel)
        for (int t = 0; t < KI; ++t) taps->sel[(long)i * KI + t] = t < nsel ? (int32_t)sel[t] : -1;
    } else {
      for (long j = 0; j <= pos; ++j) sel[j] = j;
    }

    /* absorbed query: qa_h[m] = sum_e W_UK[h][e][m] q^C_h[e] */
    for (int h = 0; h < nh; ++h) {
      const float* qc = q + (long)h * qw;
      for (int m = 0; m < dc; ++m) {
        float acc = 0.0f;
        for (int e = 0; e < dh; ++e) {
          long wi = ((long)h * dh + e) * dc + m;
          float wv = c->attn_fmt == ORC_F32 ? ((const float*)w->wuk)[wi]
                                            : orc_bf16_to_f32(((const uint16_t*)w->wuk)[wi]);
          acc += wv * qc[e];
        }
        qa[(long)h * dc + m] = acc;
      }
    }
    /* attention over stored rows 0 .. pos, per head */
#pragma omp parallel for schedule(static)
    for (int h = 0; h < nh; ++h) {
      float* sh = malloc(sizeof(float) * nsel);
      const float* qah = qa + (long)h * dc;
      const float* qr = q + (long)h * qw + dh;
      float mx = -INFINITY;
      for (long u = 0; u < nsel; ++u) {
        const long j = sel[u];
        float acc = 0.0f;
        for (int m = 0; m < dc; ++m) acc += qah[m] * kv_get(kv, c->kv_fmt, rw, j, m);
        for (int r = 0; r < dr; ++r) acc += qr[r] * kv_get(kv, c->kv_fmt, rw, j, dc + r);
        sh[u] = acc * scale;
        if (sh[u] > mx) mx = sh[u];
      }
      float sum = 0.0f;
      for (long u = 0; u < nsel; ++u) { sh[u] = expf(sh[u] - mx); sum += sh[u]; }
      float* zh = z + (long)h * dc;
      for (int m = 0; m < dc; ++m) zh[m] = 0.0f;
      for (long u = 0; u < nsel; ++u) {
        float p = sh[u] / sum;
        for (int m = 0; m < dc; ++m) zh[m] += p * kv_get(kv, c->kv_fmt, rw, sel[u], m);
      }
      /* value up-projection: o_h[e] = sum_m W_UV[h][e][m] z_h[m] */
      for (int e = 0; e < dh; ++e) {
        float acc = 0.0f;
        for (int m = 0; m < dc; ++m) {
          long wi = ((long)h * dh + e) * dc + m;
          float wv = c->attn_fmt == ORC_F32 ? ((const float*)w->wuv)[wi]
                                            : orc_bf16_to_f32(((const uint16_t*)w->wuv)[wi]);
          acc += wv * zh[m];
        }
        o[(long)h * dh + e] = acc;
      }
      free(sh);
    }
    matvec(&WO, o, att);
    for (int k = 0; k < d; ++k) Hp[(long)i * d + k] = H[(long)i * d + k] + att[k];

    if (taps) {
      if (taps->x) memcpy(taps->x + (long)i * d, x, sizeof(float) * d);
      if (taps->q) memcpy(taps->q + (long)i * nh * qw, q, sizeof(float) * nh * qw);
      if (taps->ckv) memcpy(taps->ckv + (long)i * kvw, ckv, sizeof(float) * kvw);   /* without the index key */
      if (taps->qabs) memcpy(taps->qabs + (long)i * nh * dc, qa, sizeof(float) * nh * dc);
      if (taps->z) memcpy(taps->z + (long)i * nh * dc, z, sizeof(float) * nh * dc);
      if (taps->o) memcpy(taps->o + (long)i * nh * dh, o, sizeof(float) * nh * dh);
    }
  }
  free(x); free(q); free(ckv); free(qa); free(z); free(o); free(att); free(cq); free(cqn); free(cn);
  free(qi); free(wi); free(isc); free(sel);
  return 0;
}

/* ------------------------------------------------------------------ router */
/* top-k by value, descending; ties go to the lower index */
static void topk_desc(const float* v, int n, int k, int32_t* idx) {
  char* used = calloc((size_t)n, 1);
  for (int t = 0; t < k; ++t) {
    int best = -1;
    for (int e = 0; e < n; ++e)
      if (!used[e] && (best < 0 || v[e] > v[best])) best = e;
    used[best] = 1;
    idx[t] = best;
  }
  free(used);
}

static void router_token(const orc_cfg* c, const orc_weights* w, const float* hp, float* xp,
                         float* logits, float* prob) {
  wmat WR = mk_wmat(w->wr, c->attn_fmt, NULL, c->E, c->d);
  rmsnorm(hp, w->gamma2, c->d, c->eps, xp);
  matvec(&WR, xp, logits);
  if (w->router_bias)
    for (int e = 0; e < c->E; ++e) logits[e] = logits[e] + w->router_bias[e];
  float mx = -INFINITY;
  for (int e = 0; e < c->E; ++e) if (logits[e] > mx) mx = logits[e];
  float sum = 0.0f;
  for (int e = 0; e < c->E; ++e) { prob[e] = expf(logits[e] - mx); sum += prob[e]; }
  for (int e = 0; e < c->E; ++e) prob[e] = prob[e] / sum;
}

static void gates_of(const float* prob, const int32_t* sel, int k, float* gate) {
  float s = 0.0f;
  for (int t = 0; t < k; ++t) s += prob[sel[t]];
  for (int t = 0; t < k; ++t) gate[t] = prob[sel[t]] / s;
}

int orc_router(const orc_cfg* c, const orc_weights* w, const float* Hp, int T,
               float* xp, float* logits, int32_t* sel, float* gate) {
  if (check_cfg(c, T) || !w || !Hp || !w->wr) return -1;
  float* xb = malloc(sizeof(float) * c->d);
  float* lb = malloc(sizeof(float) * c->E);
  float* pb = malloc(sizeof(float) * c->E);
  int32_t* sb = malloc(sizeof(int32_t) * c->top_k);
  float* gb = malloc(sizeof(float) * c->top_k);
  for (int i = 0; i < T; ++i) {
    router_token(c, w, Hp + (long)i * c->d, xb, lb, pb);
    topk_desc(lb, c->E, c->top_k, sb);
    gates_of(pb, sb, c->top_k, gb);
    if (xp) memcpy(xp + (long)i * c->d, xb, sizeof(float) * c->d);
    if (logits) memcpy(logits + (long)i * c->E, lb, sizeof(float) * c->E);
    if (sel) memcpy(sel + (long)i * c->top_k, sb, sizeof(int32_t) * c->top_k);
    if (gate) memcpy(gate + (long)i * c->top_k, gb, sizeof(float) * c->top_k);
  }
  free(xb); free(lb); free(pb); free(sb); free(gb);
  return 0;
}

/* ------------------------------------------------------------------ experts */
/* y = W2 (silu(W1 x) * (W3 x)) for expert slot e */
static int expert_fwd(const orc_cfg* c, const orc_weights* w, int e, const float* x, float* y,
                      float* a, float* b) {
  if (!w->w1 || !w->w3 || !w->w2 || !w->w1[e] || !w->w3[e] || !w->w2[e]) return -3;
  int sc = c->exp_fmt == ORC_FP8B128 || c->exp_fmt == ORC_MXFP4;
  if (sc && (!w->s1 || !w->s3 || !w->s2 || !w->s1[e] || !w->s3[e] || !w->s2[e])) return -3;
  wmat W1 = mk_wmat(w->w1[e], c->exp_fmt, sc ? w->s1[e] : NULL, c->f, c->d);
  wmat W3 = mk_wmat(w->w3[e], c->exp_fmt, sc ? w->s3[e] : NULL, c->f, c->d);
  wmat W2 = mk_wmat(w->w2[e], c->exp_fmt, sc ? w->s2[e] : NULL, c->d, c->f);
  matvec(&W1, x, a);
  matvec(&W3, x, b);
  for (int j = 0; j < c->f; ++j) a[j] = silu(a[j]) * b[j];
  matvec(&W2, a, y);
  return 0;
}

int orc_moe_block(const orc_cfg* c, const orc_weights* w, const float* Hp, int T,
                  const int32_t* force_sel, float* out, const orc_moe_taps* taps) {
  if (check_cfg(c, T) || !w || !Hp || !out || !w->wr) return -1;
  lut_init();
  const int d = c->d, E = c->E, k = c->top_k;
  float* xp = malloc(sizeof(float) * d);
  float* lg = malloc(sizeof(float) * E);
  float* pr = malloc(sizeof(float) * E);
  int32_t* sel = malloc(sizeof(int32_t) * k);
  float* g = malloc(sizeof(float) * k);
  float* y = malloc(sizeof(float) * d * (k + 1));
  float* ysh = y + (long)d * k;
  float* ys = malloc(sizeof(float) * d);
  float* a = malloc(sizeof(float) * c->f);
  float* b = malloc(sizeof(float) * c->f);
  int rc = 0;
  for (int i = 0; i < T && rc == 0; ++i) {
    router_token(c, w, Hp + (long)i * d, xp, lg, pr);
    if (force_sel) memcpy(sel, force_sel + (long)i * k, sizeof(int32_t) * k);
    else topk_desc(lg, E, k, sel);
    for (int t = 0; t < k; ++t) if (sel[t] < 0 || sel[t] >= E) rc = -1;
    if (rc) break;
    gates_of(pr, sel, k, g);
    for (int t = 0; t < k && rc == 0; ++t) rc = expert_fwd(c, w, sel[t], xp, y + (long)t * d, a, b);
    for (int r = 0; r < d; ++r) ysh[r] = 0.0f;
    for (int s = 0; s < c->n_shared && rc == 0; ++s) {
      rc = expert_fwd(c, w, E + s, xp, ys, a, b);
      for (int r = 0; r < d; ++r) ysh[r] += ys[r];
    }
    if (rc) break;
    float* oi = out + (long)i * d;
    for (int r = 0; r < d; ++r) {
      float acc = Hp[(long)i * d + r];
      for (int t = 0; t < k; ++t) acc += g[t] * y[(long)t * d + r];
      oi[r] = acc + ysh[r];
    }
    if (taps) {
      if (taps->xp) memcpy(taps->xp + (long)i * d, xp, sizeof(float) * d);
      if (taps->logits) memcpy(taps->logits + (long)i * E, lg, sizeof(float) * E);
      if (taps->sel) memcpy(taps->sel + (long)i * k, sel, sizeof(int32_t) * k);
      if (taps->gate) memcpy(taps->gate + (long)i * k, g, sizeof(float) * k);
      if (taps->y_sel) memcpy(taps->y_sel + (long)i * k * d, y, sizeof(float) * k * d);
      if (taps->y_shared) memcpy(taps->y_shared + (long)i * d, ysh, sizeof(float) * d);
    }
  }
  free(xp); free(lg); free(pr); free(sel); free(g); free(y); free(ys); free(a); free(b);
  return rc;
}

int orc_layer_step(const orc_cfg* c, const orc_weights* w, const float* H, int T,
                   void* kv, int L, float* out, const orc_attn_taps* at, const orc_moe_taps* mt) {
  if (check_cfg(c, T) || !out) return -1;
  float* hp = malloc(sizeof(float) * (size_t)c->d * (T > 0 ? T : 1));
  int rc = orc_attn_block(c, w, H, T, kv, L, hp, at);
  if (rc == 0) rc = orc_moe_block(c, w, hp, T, NULL, out, mt);
  free(hp);
  return rc;
}

/* ------------------------------------------------------------------ fp64 brute force */
int orc_layer_step_f64(const orc_cfg* c, const orc_weights* w, const float* H, int T,
                       const void* kv, int L, const int32_t* force_sel,
                       double* out, double* hp_out, double* kv_new_f64, double* logits_out,
                       int32_t* sel_out) {
  if (check_cfg(c, T) || !w || !H || !kv || !out || L < 0 || check_lowrank(c, w)) return -1;
  lut_init();
  const int d = c->d, nh = c->n_h, dh = c->d_h, dc = c->d_c, dr = c->d_r, E = c->E, k = c->top_k;
  const int qw = dh + dr, kvw = dc + dr, ql = c->q_lora;
  const long npos = (long)L + T;
  wmat WQ = mk_wmat(w->wq, c->attn_fmt, NULL, (long)nh * qw, d);
  wmat WDQ = mk_wmat(w->wdq, c->attn_fmt, NULL, ql, d);
  wmat WUQ = mk_wmat(w->wuq, c->attn_fmt, NULL, (long)nh * qw, ql);
  wmat WD = mk_wmat(w->wdkv, c->attn_fmt, NULL, kvw, d);
  wmat WO = mk_wmat(w->wo, c->attn_fmt, NULL, d, (long)nh * dh);
  wmat WUK = mk_wmat(w->wuk, c->attn_fmt, NULL, (long)nh * dh, dc);
  wmat WUV = mk_wmat(w->wuv, c->attn_fmt, NULL, (long)nh * dh, dc);
  wmat WR = mk_wmat(w->wr, c->attn_fmt, NULL, E, d);

  /* sparse attention: the indexer, and cache rows that carry their index key */
  const int sparse = c->idx_topk > 0, HI = c->idx_heads, dI = c->idx_dim, KI = c->idx_topk;
  const int rw = kvw + (sparse ? dI : 0);
  wmat WIQ = mk_wmat(sparse ? w->widx : NULL, c->attn_fmt, NULL, (long)HI * dI, d);
  wmat WIW = mk_wmat(sparse ? mat_row(w->widx, c->attn_fmt, (long)HI * dI, d) : NULL, c->attn_fmt, NULL, HI, d);
  wmat WIK = mk_wmat(sparse ? mat_row(w->widx, c->attn_fmt, (long)HI * dI + HI, d) : NULL, c->attn_fmt, NULL, dI, d);
  double* qi = malloc(sizeof(double) * (sparse ? (long)T * HI * dI : 1));
  double* wi = malloc(sizeof(double) * (sparse ? (long)T * HI : 1));
  double* isc = malloc(sizeof(double) * npos);
  long* selr = malloc(sizeof(long) * npos);
  /* all rows of the cache as double: prefill rows as stored, new rows rounded to storage */
  double* rows = malloc(sizeof(double) * npos * rw);
  for (long j = 0; j < L; ++j)
    for (int m = 0; m < rw; ++m) rows[j * rw + m] = (double)kv_get(kv, c->kv_fmt, rw, j, m);
  double* x = malloc(sizeof(double) * d);
  double* q = malloc(sizeof(double) * (long)T * nh * qw);
  double* ckv = malloc(sizeof(double) * rw);
  float* rowf = malloc(sizeof(float) * rw);
  float* rowr = malloc(sizeof(float) * rw);
  double* cq = malloc(sizeof(double) * (ql > 0 ? ql : 1));
  double* cqn = malloc(sizeof(double) * (ql > 0 ? ql : 1));
  double* cn = malloc(sizeof(double) * dc);
  for (int i = 0; i < T; ++i) {
    const long pos = (long)L + i;
    rmsnorm64(H + (long)i * d, w->gamma1, d, (double)c->eps, x);
    if (ql > 0) {
      matvec64(&WDQ, x, cq);
      rmsnorm64d(cq, w->gamma_q, ql, (double)c->eps, cqn);
      matvec64(&WUQ, cqn, q + (long)i * nh * qw);
    } else {
      matvec64(&WQ, x, q + (long)i * nh * qw);
    }
    matvec64(&WD, x, ckv);
    if (c->kv_norm) {
      rmsnorm64d(ckv, w->gamma_kv, dc, (double)c->eps, cn);
      memcpy(ckv, cn, sizeof(double) * dc);
    }
    for (int h = 0; h < nh; ++h) rope64(q + (long)i * nh * qw + (long)h * qw + dh, dr, pos, c->rope_base);
    rope64(ckv + dc, dr, pos, c->rope_base);
    if (sparse) {
      matvec64(&WIK, x, ckv + kvw);
      matvec64(&WIQ, x, qi + (long)i * HI * dI);
      matvec64(&WIW, x, wi + (long)i * HI);
    }
    for (int m = 0; m < rw; ++m) rowf[m] = (float)ckv[m];
    kv_round_row(c->kv_fmt, rw, rowf, rowr);
    for (int m = 0; m < rw; ++m) {
      rows[pos * rw + m] = (double)rowr[m];
      if (kv_new_f64 && m < kvw) kv_new_f64[(long)i * kvw + m] = (double)rowr[m];
    }
  }
  /* un-absorbed keys/values per head: kc[h][j][e] = W_UK[h] c_j, v[h][j][e] = W_UV[h] c_j */
  double* kc = malloc(sizeof(double) * (long)nh * npos * dh);
  double* vv = malloc(sizeof(double) * (long)nh * npos * dh);
#pragma omp parallel for schedule(static)
  for (long hj = 0; hj < (long)nh * npos; ++hj) {
    long h = hj / npos, j = hj % npos;
    for (int e = 0; e < dh; ++e) {
      double ak = 0.0, av = 0.0;
      for (int m = 0; m < dc; ++m) {
        ak += wat64(&WUK, h * dh + e, m) * rows[j * rw + m];
        av += wat64(&WUV, h * dh + e, m) * rows[j * rw + m];
      }
      kc[hj * dh + e] = ak;
      vv[hj * dh + e] = av;
    }
  }
  const double scale = 1.0 / sqrt((double)(dh + dr));
  double* o = malloc(sizeof(double) * nh * dh);
  double* att = malloc(sizeof(double) * d);
  double* hp = malloc(sizeof(double) * (long)T * d);
  for (int i = 0; i < T; ++i) {
    const long pos = (long)L + i;
    long nsel = pos + 1;
    if (sparse) {
#pragma omp parallel for schedule(static)
      for (long j = 0; j <= pos; ++j) {
        double sc = 0.0;
        for (int hh = 0; hh < HI; ++hh) {
          double dot = 0.0;
          for (int m = 0; m < dI; ++m) dot += qi[((long)i * HI + hh) * dI + m] * rows[j * rw + kvw + m];
          if (dot > 0.0) sc += wi[(long)i * HI + hh] * dot;
        }
        isc[j] = sc;
      }
      nsel = select_rows(isc, pos, KI, selr);
      if (w->force_isel)
        for (long u = 0; u < nsel; ++u) selr[u] = w->force_isel[(long)i * KI + u];
    } else {
      for (long j = 0; j <= pos; ++j) selr[j] = j;
    }
    for (int h = 0; h < nh; ++h) {
      const double* qh = q + (long)i * nh * qw + (long)h * qw;
      double* sc = malloc(sizeof(double) * nsel);
      double mx = -INFINITY;
      for (long u = 0; u < nsel; ++u) {
        const long j = selr[u];
        double a = 0.0;
        for (int e = 0; e < dh; ++e) a += qh[e] * kc[((long)h * npos + j) * dh + e];
        for (int r = 0; r < dr; ++r) a += qh[dh + r] * rows[j * rw + dc + r];
        sc[u] = a * scale;
        if (sc[u] > mx) mx = sc[u];
      }
      double sum = 0.0;
      for (long u = 0; u < nsel; ++u) { sc[u] = exp(sc[u] - mx); sum += sc[u]; }
      for (int e = 0; e < dh; ++e) {
        double a = 0.0;
        for (long u = 0; u < nsel; ++u) a += (sc[u] / sum) * vv[((long)h * npos + selr[u]) * dh + e];
        o[(long)h * dh + e] = a;
      }
      free(sc);
    }
    matvec64(&WO, o, att);
    for (int r = 0; r < d; ++r) hp[(long)i * d + r] = (double)H[(long)i * d + r] + att[r];
  }
  if (hp_out) memcpy(hp_out, hp, sizeof(double) * (long)T * d);

  /* MoE in double */
  double* xp = malloc(sizeof(double) * d);
  double* lg = malloc(sizeof(double) * E);
  double* a = malloc(sizeof(double) * c->f);
  double* b = malloc(sizeof(double) * c->f);
  double* y = malloc(sizeof(double) * d);
  int32_t* sel = malloc(sizeof(int32_t) * k);
  int rc = 0;
  for (int i = 0; i < T && rc == 0; ++i) {
    rmsnorm64d(hp + (long)i * d, w->gamma2, d, (double)c->eps, xp);
    matvec64(&WR, xp, lg);
    if (w->router_bias) for (int e = 0; e < E; ++e) lg[e] += (double)w->router_bias[e];
    if (logits_out) memcpy(logits_out + (long)i * E, lg, sizeof(double) * E);
    if (force_sel) {
      memcpy(sel, force_sel + (long)i * k, sizeof(int32_t) * k);
    } else {
      char* used = calloc((size_t)E, 1);
      for (int t = 0; t < k; ++t) {
        int best = -1;
        for (int e = 0; e < E; ++e) if (!used[e] && (best < 0 || lg[e] > lg[best])) best = e;
        used[best] = 1; sel[t] = best;
      }
      free(used);
    }
    if (sel_out) memcpy(sel_out + (long)i * k, sel, sizeof(int32_t) * k);
    double mx = -INFINITY;
    for (int e = 0; e < E; ++e) if (lg[e] > mx) mx = lg[e];
    double z = 0.0, zs = 0.0;
    for (int e = 0; e < E; ++e) z += exp(lg[e] - mx);
    for (int t = 0; t < k; ++t) zs += exp(lg[sel[t]] - mx) / z;
    double* oi = out + (long)i * d;
    for (int r = 0; r < d; ++r) oi[r] = hp[(long)i * d + r];
    for (int t = 0; t <= k + c->n_shared - 1 && rc == 0; ++t) {
      int e; double g;
      if (t < k) { e = sel[t]; g = (exp(lg[e] - mx) / z) / zs; }
      else { e = E + (t - k); g = 1.0; }
      if (!w->w1 || !w->w1[e] || !w->w3[e] || !w->w2[e]) { rc = -3; break; }
      int sc = c->exp_fmt == ORC_FP8B128 || c->exp_fmt == ORC_MXFP4;
      wmat W1 = mk_wmat(w->w1[e], c->exp_fmt, sc ? w->s1[e] : NULL, c->f, d);
      wmat W3 = mk_wmat(w->w3[e], c->exp_fmt, sc ? w->s3[e] : NULL, c->f, d);
      wmat W2 = mk_wmat(w->w2[e], c->exp_fmt, sc ? w->s2[e] : NULL, d, c->f);
      matvec64(&W1, xp, a);
      matvec64(&W3, xp, b);
      for (int j = 0; j < c->f; ++j) a[j] = silu64(a[j]) * b[j];
      matvec64(&W2, a, y);
      for (int r = 0; r < d; ++r) oi[r] += g * y[r];
    }
  }
  free(rows); free(x); free(q); free(ckv); free(rowf); free(rowr); free(kc); free(vv); free(o); free(att); free(hp);
  free(cq); free(cqn); free(cn); free(qi); free(wi); free(isc); free(selr);
  free(xp); free(lg); free(a); free(b); free(y); free(sel);
  return rc;
}

/* ------------------------------------------------------------------ stack pieces */
int orc_embed(const uint16_t* emb, int V, int d, const int32_t* tokens, int T, float* h) {
  if (!emb || !tokens || !h || V <= 0 || d <= 0) return -1;
  for (int i = 0; i < T; ++i) {
    if (tokens[i] < 0 || tokens[i] >= V) return -1;
    for (int k = 0; k < d; ++k) h[(long)i * d + k] = orc_bf16_to_f32(emb[(long)tokens[i] * d + k]);
  }
  return 0;
}

int orc_head(const uint16_t* head, int V, int d, const float* gamma_f, float eps,
             const float* h, int T, float* logits, int32_t* argmax) {
  return orc_head_fmt(head, ORC_BF16, NULL, V, d, gamma_f, eps, h, T, logits, argmax);
}

int orc_head_fmt(const void* head, int fmt, const float* scales, int V, int d, const float* gamma_f, float eps,
                 const float* h, int T, float* logits, int32_t* argmax) {
  if (!head || !gamma_f || !h || V <= 0 || d <= 0) return -1;
  if (fmt != ORC_BF16 && !(fmt == ORC_FP8B128 && scales)) return -1;
  lut_init();
  float* x = malloc(sizeof(float) * d);
  float* lg = logits ? NULL : malloc(sizeof(float) * V);
  wmat W = mk_wmat(head, fmt, scales, V, d);
  for (int i = 0; i < T; ++i) {
    float* li = logits ? logits + (long)i * V : lg;
    rmsnorm(h + (long)i * d, gamma_f, d, eps, x);
    matvec(&W, x, li);
    int best = 0;
    for (int v = 1; v < V; ++v) if (li[v] > li[best]) best = v;
    if (argmax) argmax[i] = best;
  }
  free(x); free(lg);
  return 0;
}

/* ------------------------------------------------------------------ sampled verification */
/* SplitMix64's output function (Steele, Lea and Flood, OOPSLA 2014; the
 * constants of the reference implementation splitmix64.c). */
uint64_t orc_splitmix64_mix(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
#define ORC_GOLDEN_GAMMA 0x9E3779B97F4A7C15ull

uint64_t orc_sample_key(uint64_t seed, uint32_t step) {
  return orc_splitmix64_mix(seed + ((uint64_t)step + 1) * ORC_GOLDEN_GAMMA);
}

/* Draw i of a step: the top 23 bits of SplitMix64's i-th output from the
 * step's key, as the midpoint (k + 1/2) 2^-23 -- in (0, 1), exact in fp32. */
float orc_sample_uniform(uint64_t key, uint64_t i) {
  const uint64_t r = orc_splitmix64_mix(key + (i + 1) * ORC_GOLDEN_GAMMA);
  return (float)(((double)(r >> 41) + 0.5) * 0x1p-23);
}

/* Speculative sampling with the drafts taken as point proposals (a draft
 * distribution that puts all its mass on the drafted token): row i's target
 * distribution is p_i = softmax(logits_i / tau).  Draft i+1 is accepted when
 * the row's acceptance draw is below p_i(draft); at the first rejection the
 * step commits a token drawn from p_i with the draft removed (renormalised),
 * and after T-1 acceptances a token drawn from p_{T-1}.  Token draws are
 * Gumbel-max: argmax_v logits_iv / tau - ln(-ln u_iv), ties to the lower id.
 * Draws: u_iv = uniform(key, i (V+1) + v) for v < V, the acceptance draw
 * uniform(key, i (V+1) + V).  All arithmetic in fp64 on the fp32 logits. */
int orc_verify_sampled(const float* logits, int V, int T, const int32_t* tokens, float tau, uint64_t key,
                       int32_t* sample, int32_t* committed) {
  if (!logits || !tokens || V <= 0 || T <= 0 || !(tau > 0.f)) return -1;
  const double it = 1.0 / (double)tau;
  int32_t* smp = malloc(sizeof(int32_t) * T);
  int32_t* res = malloc(sizeof(int32_t) * T);        /* row i's draw without draft i+1 */
  double* pd = malloc(sizeof(double) * T);           /* p_i(draft i+1) */
  for (int i = 0; i < T; ++i) {
    const float* l = logits + (long)i * V;
    const int dn = i + 1 < T ? tokens[i + 1] : -1;
    double M = -INFINITY;
    for (int v = 0; v < V; ++v) M = fmax(M, (double)l[v] * it);
    double S = 0.0;
    for (int v = 0; v < V; ++v) S += exp((double)l[v] * it - M);
    pd[i] = (dn >= 0 && dn < V) ? exp((double)l[dn] * it - M) / S : 0.0;
    double b = -INFINITY, bx = -INFINITY;
    int bi = -1, bxi = -1;
    for (int v = 0; v < V; ++v) {
      const double u = (double)orc_sample_uniform(key, (uint64_t)i * (uint64_t)(V + 1) + (uint64_t)v);
      const double y = (double)l[v] * it - log(-log(u));
      if (y > b) { b = y; bi = v; }
      if (v != dn && y > bx) { bx = y; bxi = v; }
    }
    smp[i] = bi;
    res[i] = bxi;
  }
  int n = 0, last = -1;
  for (int i = 0; i + 1 < T; ++i) {
    const double ua = (double)orc_sample_uniform(key, (uint64_t)i * (uint64_t)(V + 1) + (uint64_t)V);
    if (ua < pd[i]) {
      ++n;
      continue;
    }
    last = res[i];
    break;
  }
  if (n == T - 1) last = smp[T - 1];
  if (sample) memcpy(sample, smp, sizeof(int32_t) * T);
  if (committed) {
    committed[0] = n + 1;
    for (int j = 1; j <= n; ++j) committed[j] = tokens[j];
    committed[n + 1] = last;
  }
  free(smp); free(res); free(pd);
  return n + 1;
}

int orc_greedy_accept(const int32_t* tokens, const int32_t* a, int T, int32_t* committed) {
  if (!tokens || !a || T <= 0) return -1;
  int n = 0;
  while (n + 1 <= T - 1 && tokens[n + 1] == a[n]) ++n;
  if (committed) {
    for (int j = 1; j <= n; ++j) committed[j - 1] = tokens[j];
    committed[n] = a[n];
  }
  return n + 1;
}
