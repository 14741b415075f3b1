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
