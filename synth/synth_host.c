/* Host build of the seeded synthetic-input generator; definitions in synth.h. */
#include "synth.h"
#include <math.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27; z *= 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static inline uint64_t key_of(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed ^ 0x6A09E667F3BCC909ull) + stream * GAMMA);
}
static inline int32_t ih4(uint64_t r) {
  int32_t s = (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
              (int32_t)((r >> 32) & 0xFFFF) + (int32_t)(r >> 48);
  return s - 131070;
}
/* volatile stores keep gcc from contracting the multiply and add into an FMA */
static inline float normal_at(uint64_t key, uint64_t i, float c, float mean) {
  volatile float p = (float)ih4(mix64(key + (i + 1) * GAMMA)) * c;
  if (mean != 0.0f) { volatile float q = p + mean; return q; }
  return p;
}

uint64_t mks_host_raw(uint64_t seed, uint64_t stream, uint64_t i) {
  return mix64(key_of(seed, stream) + (i + 1) * GAMMA);
}

void mks_host_raw_fill(uint64_t* dst, uint64_t n, uint64_t seed, uint64_t stream, uint64_t offset) {
  uint64_t k = key_of(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) dst[i] = mix64(k + (offset + (uint64_t)i + 1) * GAMMA);
}

uint16_t mks_host_bf16_encode(float x) {
  uint32_t u; memcpy(&u, &x, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint8_t mks_host_e4m3_encode(float x) {
  uint32_t u; memcpy(&u, &x, 4);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80);
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7E;          /* |x| >= 448: saturate */
  if (a < 0x3C800000u) {                              /* |x| < 2^-6: step 2^-9 */
    float af; memcpy(&af, &a, 4);
    float v = rintf(af * 512.0f);                     /* exact scaling, then RNE */
    return sign | (uint8_t)v;                         /* 8 carries into code 0x08 */
  }
  int e = (int)(a >> 23) - 127;                       /* -6 .. 8 */
  uint32_t mant = a & 0x7FFFFFu, q = mant >> 20, rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1;
  uint32_t code = ((uint32_t)(e + 7) << 3) + q;
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

void mks_host_normal_f32(float* dst, uint64_t n, uint64_t seed, uint64_t stream,
                         uint64_t offset, float c, float mean) {
  uint64_t k = key_of(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) dst[i] = normal_at(k, offset + (uint64_t)i, c, mean);
}

void mks_host_normal_bf16(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t stream,
                          uint64_t offset, float c, float mean) {
  uint64_t k = key_of(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i)
    dst[i] = mks_host_bf16_encode(normal_at(k, offset + (uint64_t)i, c, mean));
}

void mks_host_fp8_blocks(uint8_t* codes, float* scales, int64_t R, int64_t K,
                         uint64_t seed, uint64_t stream, float c) {
  uint64_t k = key_of(seed, stream);
  int64_t nbr = (R + 127) / 128, nbk = (K + 127) / 128;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < nbr * nbk; ++b) {
    int64_t br = b / nbk, bk = b % nbk;
    int64_t r0 = br * 128, r1 = r0 + 128 < R ? r0 + 128 : R;
    int64_t k0 = bk * 128, k1 = k0 + 128 < K ? k0 + 128 : K;
    float amax = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t j = k0; j < k1; ++j) {
        float w = fabsf(normal_at(k, (uint64_t)(r * K + j), c, 0.0f));
        if (w > amax) amax = w;
      }
    volatile float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    scales[b] = s;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t j = k0; j < k1; ++j) {
        volatile float v = normal_at(k, (uint64_t)(r * K + j), c, 0.0f) / s;
        codes[r * K + j] = mks_host_e4m3_encode(v);
      }
  }
}

void mks_host_fp8row_kv(uint8_t* dst, int64_t rows, int64_t kvw, int64_t row_bytes,
                        uint64_t seed, uint64_t stream, uint64_t scale_stream, float c) {
  uint64_t k = key_of(seed, stream), ks = key_of(seed, scale_stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t* row = dst + r * row_bytes;
    const int e = -6 + (int)(mix64(ks + ((uint64_t)r + 1) * GAMMA) % 3u);
    for (int64_t m = 0; m < kvw; ++m)
      row[m] = mks_host_e4m3_encode(ldexpf(normal_at(k, (uint64_t)(r * kvw + m), c, 0.0f), -e));
    const float sc = ldexpf(1.0f, e);
    memcpy(row + kvw, &sc, 4);
    memset(row + kvw + 4, 0, (size_t)(row_bytes - kvw - 4));
  }
}

uint8_t mks_host_e2m1_encode(float x) {
  static const float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t u; memcpy(&u, &x, 4);
  uint8_t sign = (uint8_t)((u >> 28) & 8u);
  float a = fabsf(x);
  int i = 0;
  while (i < 7 && a > mid[i]) ++i;
  if (i < 7 && a == mid[i] && (i & 1)) ++i;        /* a tie between codes i, i+1: the even one */
  return sign | (uint8_t)i;
}

/* floor(log2 a) for a finite a > 0, from the exponent bits (exact) */
static int floor_log2(float a) {
  uint32_t u; memcpy(&u, &a, 4);
  int e = (int)((u >> 23) & 0xFF);
  if (e) return e - 127;
  uint32_t m = u & 0x7FFFFFu;
  int k = -127;
  while (!(m & 0x400000u)) { m <<= 1; --k; }
  return k;
}

void mks_host_mxfp4_blocks(uint8_t* codes, uint8_t* scales, int64_t R, int64_t K,
                           uint64_t seed, uint64_t stream, float c) {
  uint64_t k = key_of(seed, stream);
  int64_t ng = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t gi = 0; gi < R * ng; ++gi) {
    int64_t r = gi / ng, g = gi % ng;
    float w[32];
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
      w[j] = normal_at(k, (uint64_t)(r * K + g * 32 + j), c, 0.0f);
      float a = fabsf(w[j]);
      if (a > amax) amax = a;
    }
    int code = 0;
    if (amax > 0.0f) {
      code = floor_log2(amax) - 2 + 127;
      if (code < 0) code = 0;
      if (code > 254) code = 254;
    }
    scales[gi] = (uint8_t)code;
    for (int j = 0; j < 32; j += 2) {
      uint8_t lo = mks_host_e2m1_encode(ldexpf(w[j], 127 - code));
      uint8_t hi = mks_host_e2m1_encode(ldexpf(w[j + 1], 127 - code));
      codes[r * (K / 2) + g * 16 + j / 2] = (uint8_t)(lo | (hi << 4));
    }
  }
}
