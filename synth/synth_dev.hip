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
