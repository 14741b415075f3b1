/*
 * Seeded synthetic-input generator shared by the CPU oracle side and the GPU
 * side.  It holds none of the decoder layer's arithmetic: it only draws
 * numbers and encodes them into the storage formats the layer consumes.
 *
 * Definitions (both the host build, synth_host.c, and the device build,
 * synth_dev.hip, implement exactly these; a GPU test checks them bitwise):
 *
 *   mix64(z)     SplitMix64 output function (Steele, Lea and Flood, "Fast
 *                splittable pseudorandom number generators", OOPSLA 2014):
 *                z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31.
 *   key(s, t)    mix64(mix64(s ^ 0x6A09E667F3BCC909) + t * GAMMA),
 *                GAMMA = 0x9E3779B97F4A7C15 (SplitMix64's increment).
 *   raw(s, t, i) mix64(key(s, t) + (i + 1) * GAMMA)   -- counter based.
 *   ih4(r)       sum of the four 16-bit fields of r, minus 131070: an
 *                Irwin-Hall(4) integer in [-131070, 131070], mean 0,
 *                standard deviation 65536/sqrt(3) (to 1e-10 relative).
 *   normal(i)    (float)ih4(raw(s,t,i)) * c   [one fp32 rounding]
 *                then + mean in fp32 when mean != 0 [a second rounding];
 *                c = fp32(sigma * sqrt(3) / 65536) is passed in by the
 *                caller so both sides use the same constant.
 *   bf16(x)      round-to-nearest-even of the fp32 value to bfloat16.
 *   e4m3(x)      OCP 8-bit floating point E4M3 ("FN" variant: bias 7, no
 *                infinities, NaN = S.1111.111, max normal 448), round to
 *                nearest even, saturating at +-448.
 *   fp8 blocks   a [R][K] tensor of normal() values, element (r,k) drawn at
 *                counter r*K+k, cut into 128x128 blocks (ragged at the
 *                edges); per block s = amax/448 (s = 1 when amax == 0),
 *                codes q = e4m3(w / s) with IEEE division.  Scales are
 *                stored row-major [ceil(R/128)][ceil(K/128)].
 *   e2m1(x)      OCP Microscaling (MX) E2M1: magnitudes 0, 0.5, 1, 1.5, 2,
 *                3, 4, 6 with codes 0..7 and the sign in bit 3; round to
 *                nearest, a tie going to the even code; saturating at +-6.
 *   mxfp4 blocks a [R][K] tensor of normal() values (element (r,k) drawn at
 *                counter r*K+k, as for fp8 blocks), K a multiple of 32, cut
 *                into groups of 32 consecutive elements of a row; per group
 *                with amax = max |w|: e = floor(log2 amax) - 2 (exact, from
 *                amax's exponent bits; 2 is E2M1's largest exponent), scale
 *                code = e + 127 clamped to [0, 254] (code 0 when amax == 0),
 *                X = 2^(code - 127), elements q = e2m1(w / X) (an exact
 *                division by a power of two).  Codes are packed two per byte,
 *                element 2j in the low nibble of byte j: [R][K/2]; scale codes
 *                (E8M0) [R][K/32].
 *   fp8 KV rows  `rows` rows of `row_bytes` bytes (row_bytes >= kvw + 4);
 *                row r holds kvw E4M3 codes, then its fp32 scale, then zero
 *                bytes.  The scale is 2^e_r with e_r = -6 + (raw(s, u, r) mod 3)
 *                (u the scale stream), and code m is e4m3(normal(r*kvw+m) *
 *                2^-e_r) (an exact scaling by a power of two), so the decoded
 *                row approximates the same N(0, sigma) draws as the f32 / bf16
 *                caches.  With sigma = 1 no code saturates (|normal| < 3.47).
 */
#ifndef MK_SYNTH_H
#define MK_SYNTH_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* host (synth_host.c, OpenMP) */
uint64_t mks_host_raw(uint64_t seed, uint64_t stream, uint64_t i);
void mks_host_raw_fill(uint64_t* dst, uint64_t n, uint64_t seed, uint64_t stream, uint64_t offset);
void mks_host_normal_f32(float* dst, uint64_t n, uint64_t seed, uint64_t stream,
                         uint64_t offset, float c, float mean);
void mks_host_normal_bf16(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t stream,
                          uint64_t offset, float c, float mean);
void mks_host_fp8_blocks(uint8_t* codes, float* scales, int64_t R, int64_t K,
                         uint64_t seed, uint64_t stream, float c);
void mks_host_fp8row_kv(uint8_t* dst, int64_t rows, int64_t kvw, int64_t row_bytes,
                        uint64_t seed, uint64_t stream, uint64_t scale_stream, float c);
void mks_host_mxfp4_blocks(uint8_t* codes, uint8_t* scales, int64_t R, int64_t K,
                           uint64_t seed, uint64_t stream, float c);
uint8_t mks_host_e4m3_encode(float x);
uint8_t mks_host_e2m1_encode(float x);
uint16_t mks_host_bf16_encode(float x);

/* device (synth_dev.hip); every call is asynchronous on `stream_handle`
   (a hipStream_t, NULL = default stream) and returns 0 or a HIP error code. */
int mks_dev_normal_f32(float* dst, uint64_t n, uint64_t seed, uint64_t stream,
                       uint64_t offset, float c, float mean, void* stream_handle);
int mks_dev_normal_bf16(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t stream,
                        uint64_t offset, float c, float mean, void* stream_handle);
int mks_dev_fp8_blocks(uint8_t* codes, float* scales, int64_t R, int64_t K,
                       uint64_t seed, uint64_t stream, float c, void* stream_handle);
int mks_dev_raw_fill(uint64_t* dst, uint64_t n, uint64_t seed, uint64_t stream,
                     uint64_t offset, void* stream_handle);
int mks_dev_fp8row_kv(uint8_t* dst, int64_t rows, int64_t kvw, int64_t row_bytes,
                      uint64_t seed, uint64_t stream, uint64_t scale_stream, float c, void* hip_stream);
int mks_dev_mxfp4_blocks(uint8_t* codes, uint8_t* scales, int64_t R, int64_t K,
                         uint64_t seed, uint64_t stream, float c, void* stream_handle);

#ifdef __cplusplus
}
#endif
#endif
