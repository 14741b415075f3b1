// Device build of the seeded synthetic-input generator; definitions in synth.h.
// Built with -ffp-contract=off and correctly rounded fp32 division so that each
// value is bit-identical to the host build (synth_host.c).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "synth.h"

#pragma clang fp contract(off)

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27; z *= 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__host__ __device__ inline uint64_t key_of(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed ^ 0x6A09E667F3BCC909ull) + stream * GAMMA);
}
__device__ inline int32_t ih4(uint64_t r) {
  int32_t s = (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
              (int32_t)((r >> 32) & 0xFFFF) + (int32_t)(r >> 48);
  return s - 131070;
}
__device__ inline float normal_at(uint64_t key, uint64_t i, float c, float mean) {
  float p = (float)ih4(mix64(key + (i + 1) * GAMMA)) * c;
  return mean != 0.0f ? p + mean : p;
}
__device__ inline uint16_t bf16_encode(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline uint8_t e4m3_encode(float x) {
  uint32_t u = __float_as_uint(x);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80);
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7E;
  if (a < 0x3C800000u) {
    float v = rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint8_t)v;
  }
  int e = (int)(a >> 23) - 127;
  uint32_t mant = a & 0x7FFFFFu, q = mant >> 20, rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1;
  uint32_t code = ((uint32_t)(e + 7) << 3) + q;
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

__device__ inline uint8_t e2m1_encode(float x) {
  const float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  const uint8_t sign = (uint8_t)((__float_as_uint(x) >> 28) & 8u);
  const float a = fabsf(x);
  int i = 0;
  while (i < 7 && a > mid[i]) ++i;
  if (i < 7 && a == mid[i] && (i & 1)) ++i;
  return sign | (uint8_t)i;
}
__device__ inline int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)((u >> 23) & 0xFF);
  if (e) return e - 127;
  uint32_t m = u & 0x7FFFFFu;
  int k = -127;
  while (!(m & 0x400000u)) { m <<= 1; --k; }
  return k;
}

__global__ void k_raw(uint64_t* dst, uint64_t n, uint64_t key, uint64_t offset) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    dst[i] = mix64(key + (offset + i + 1) * GAMMA);
}
__global__ void k_normal_f32(float* dst, uint64_t n, uint64_t key, uint64_t offset, float c, float mean) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    dst[i] = normal_at(key, offset + i, c, mean);
}
__global__ void k_normal_bf16(uint16_t* dst, uint64_t n, uint64_t key, uint64_t offset, float c, float mean) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    dst[i] = bf16_encode(normal_at(key, offset + i, c, mean));
}
// One workgroup of 256 threads per 128x128 block.
__global__ __launch_bounds__(256) void k_fp8_blocks(uint8_t* codes, float* scales, int64_t R, int64_t K,
                                                    int64_t nbk, uint64_t key, float c) {
  __shared__ float red[256];
  int64_t b = blockIdx.x, br = b / nbk, bk = b % nbk;
  int64_t r0 = br * 128, r1 = min(r0 + 128, R);
  int64_t k0 = bk * 128, k1 = min(k0 + 128, K);
  int64_t rows = r1 - r0, cols = k1 - k0;
  float amax = 0.0f;
  for (int64_t e = threadIdx.x; e < rows * cols; e += 256) {
    int64_t r = r0 + e / cols, j = k0 + e % cols;
    amax = fmaxf(amax, fabsf(normal_at(key, (uint64_t)(r * K + j), c, 0.0f)));
  }
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  amax = red[0];
  float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) scales[b] = sc;
  for (int64_t e = threadIdx.x; e < rows * cols; e += 256) {
    int64_t r = r0 + e / cols, j = k0 + e % cols;
    codes[r * K + j] = e4m3_encode(normal_at(key, (uint64_t)(r * K + j), c, 0.0f) / sc);
  }
}

// One workgroup per KV row (grid-stride over rows).
__global__ __launch_bounds__(256) void k_fp8row_kv(uint8_t* dst, int64_t rows, int64_t kvw, int64_t row_bytes,
                                                   uint64_t key, uint64_t skey, float c) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    uint8_t* row = dst + r * row_bytes;
    const int e = -6 + (int)(mix64(skey + ((uint64_t)r + 1) * GAMMA) % 3u);
    for (int64_t m = threadIdx.x; m < row_bytes; m += blockDim.x) {
      uint8_t b = 0;
      if (m < kvw) {
        b = e4m3_encode(ldexpf(normal_at(key, (uint64_t)(r * kvw + m), c, 0.0f), -e));
      } else if (m < kvw + 4) {
        const uint32_t sb = __float_as_uint(ldexpf(1.0f, e));
        b = (uint8_t)(sb >> (8 * (m - kvw)));
      }
      row[m] = b;
    }
  }
}

// One thread per group of 32 consecutive elements of a row.
__global__ __launch_bounds__(256) void k_mxfp4_blocks(uint8_t* codes, uint8_t* scales, int64_t R, int64_t K,
                                                      uint64_t key, float c) {
  const int64_t ng = K / 32;
  for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < R * ng; gi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = gi / ng, g = gi % ng;
    float w[32];
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
      w[j] = normal_at(key, (uint64_t)(r * K + g * 32 + j), c, 0.0f);
      amax = fmaxf(amax, fabsf(w[j]));
    }
    int code = 0;
    if (amax > 0.0f) {
      code = floor_log2(amax) - 2 + 127;
      code = code < 0 ? 0 : (code > 254 ? 254 : code);
    }
    scales[gi] = (uint8_t)code;
    for (int j = 0; j < 32; j += 2) {
      const uint8_t lo = e2m1_encode(ldexpf(w[j], 127 - code));
      const uint8_t hi = e2m1_encode(ldexpf(w[j + 1], 127 - code));
      codes[r * (K / 2) + g * 16 + j / 2] = (uint8_t)(lo | (hi << 4));
    }
  }
}

inline unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  return (unsigned)(g > 65536 ? 65536 : (g == 0 ? 1 : g));
}

}  // namespace

extern "C" int mks_dev_raw_fill(uint64_t* dst, uint64_t n, uint64_t seed, uint64_t stream,
                                uint64_t offset, void* sh) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_raw, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)sh, dst, n,
                     key_of(seed, stream), offset);
  return (int)hipGetLastError();
}
extern "C" int mks_dev_normal_f32(float* dst, uint64_t n, uint64_t seed, uint64_t stream,
                                  uint64_t offset, float c, float mean, void* sh) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_normal_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)sh, dst, n,
                     key_of(seed, stream), offset, c, mean);
  return (int)hipGetLastError();
}
extern "C" int mks_dev_normal_bf16(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t stream,
                                   uint64_t offset, float c, float mean, void* sh) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_normal_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)sh, dst, n,
                     key_of(seed, stream), offset, c, mean);
  return (int)hipGetLastError();
}
extern "C" int mks_dev_fp8_blocks(uint8_t* codes, float* scales, int64_t R, int64_t K,
                                  uint64_t seed, uint64_t stream, float c, void* sh) {
  if (R <= 0 || K <= 0) return 0;
  int64_t nbr = (R + 127) / 128, nbk = (K + 127) / 128;
  hipLaunchKernelGGL(k_fp8_blocks, dim3((unsigned)(nbr * nbk)), dim3(256), 0, (hipStream_t)sh,
                     codes, scales, R, K, nbk, key_of(seed, stream), c);
  return (int)hipGetLastError();
}
extern "C" int mks_dev_fp8row_kv(uint8_t* dst, int64_t rows, int64_t kvw, int64_t row_bytes,
                                 uint64_t seed, uint64_t stream, uint64_t scale_stream, float c, void* sh) {
  if (rows <= 0) return 0;
  if (kvw <= 0 || row_bytes < kvw + 4) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fp8row_kv, dim3((unsigned)(rows < 65536 ? rows : 65536)), dim3(256), 0, (hipStream_t)sh,
                     dst, rows, kvw, row_bytes, key_of(seed, stream), key_of(seed, scale_stream), c);
  return (int)hipGetLastError();
}
extern "C" int mks_dev_mxfp4_blocks(uint8_t* codes, uint8_t* scales, int64_t R, int64_t K,
                                    uint64_t seed, uint64_t stream, float c, void* sh) {
  if (R <= 0 || K <= 0 || K % 32) return R <= 0 || K <= 0 ? 0 : (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mxfp4_blocks, dim3(grid_for((uint64_t)(R * (K / 32)))), dim3(256), 0, (hipStream_t)sh,
                     codes, scales, R, K, key_of(seed, stream), c);
  return (int)hipGetLastError();
}
