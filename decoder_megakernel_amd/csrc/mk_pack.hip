// Weight packing: canonical row-major tensors -> 1 KiB MFMA operand tiles.
// Tile (b, rt, kt), lane l (16 bytes): row rt*16 + l%16, columns
// kt*TK + (l/16)*TK/4 ... of matrix b; zeros outside the matrix.
#include "mk_common.h"

namespace mk {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_p;

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src, int es, int nb, int R, int K,
                                                   long long sb, long long sr, long long sk, int TK,
                                                   uint8_t* __restrict__ dst, long long dst_stride,
                                                   long long dst_off, int RT, int KT) {
  const long long total = (long long)nb * RT * KT * 64;
  const int epl = TK / 4;
  for (long long c = blockIdx.x * 256ll + threadIdx.x; c < total; c += (long long)gridDim.x * 256) {
    const int l = (int)(c & 63);
    long long tix = c >> 6;
    const int kt = (int)(tix % KT);
    tix /= KT;
    const int rt = (int)(tix % RT);
    const int b = (int)(tix / RT);
    const int r = rt * 16 + (l & 15);
    const int k0 = kt * TK + (l >> 4) * epl;
    uint8_t* o = dst + dst_off + (((long long)b * RT + rt) * KT + kt) * dst_stride + l * 16;
    if (sk == 1 && r < R && k0 + epl <= K) {
      const long long e0 = (long long)b * sb + (long long)r * sr + k0;
      *reinterpret_cast<u32x4_p*>(o) = *reinterpret_cast<const u32x4_p*>(src + e0 * es);
    } else {
      uint8_t tmp[16];
      for (int i = 0; i < epl; ++i) {
        const int k = k0 + i;
        const bool in = r < R && k < K;
        const long long e = (long long)b * sb + (long long)r * sr + (long long)k * sk;
        for (int q = 0; q < es; ++q) tmp[i * es + q] = in ? src[e * es + q] : 0;
      }
      for (int q = 0; q < 16; ++q) o[q] = tmp[q];
    }
  }
}

// MXFP4 codes are packed as a byte matrix [R][K/2] (two codes per byte, the
// strides in bytes, sk = 1): a tile's 64 byte columns are its 128 elements.
int launch_pack(const void* src, int fmt, int nb, int R, int K, long long sb, long long sr, long long sk,
                void* dst, long long dst_stride, long long dst_off, hipStream_t stream) {
  int TK = tile_k(fmt);
  const int es = elem_bytes(fmt);
  if (fmt == MK_FMT_MXFP4) {
    if (K % 2 || sk != 1) return (int)hipErrorInvalidValue;
    K /= 2;
    TK /= 2;
  }
  const int RT = (R + 15) / 16, KT = (K + TK - 1) / TK;
  const long long total = (long long)nb * RT * KT * 64;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint8_t*)src, es, nb, R,
                     K, sb, sr, sk, TK, (uint8_t*)dst, dst_stride, dst_off, RT, KT);
  return (int)hipGetLastError();
}

// MXFP4 scales: canonical E8M0 bytes [R][K/32] -> per tile (rt, kt) 64 bytes,
// byte l = the scale of row rt*16 + l%16 over columns kt*128 + (l/16)*32 ...,
// at dst + dst_off + (rt * KT + kt) * tile_stride.  R % 16 == 0, K % 128 == 0.
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ src, int R, int K,
                                                             uint8_t* __restrict__ dst, long long tile_stride,
                                                             long long dst_off) {
  const int KT = K / 128, G = K / 32;
  const long long total = (long long)(R / 16) * KT * 64;
  for (long long c = blockIdx.x * 256ll + threadIdx.x; c < total; c += (long long)gridDim.x * 256) {
    const int l = (int)(c & 63);
    const long long tix = c >> 6;
    const int kt = (int)(tix % KT), rt = (int)(tix / KT);
    const int r = rt * 16 + (l & 15), g = kt * 4 + (l >> 4);
    dst[dst_off + tix * tile_stride + l] = src[(long long)r * G + g];
  }
}

int launch_pack_mx_scales(const void* src, int R, int K, void* dst, long long tile_stride, long long dst_off,
                          hipStream_t stream) {
  if (R % 16 || K % 128) return (int)hipErrorInvalidValue;
  const long long total = (long long)(R / 16) * (K / 128) * 64;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_mx_scales_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint8_t*)src, R, K,
                     (uint8_t*)dst, tile_stride, dst_off);
  return (int)hipGetLastError();
}

}  // namespace mk
