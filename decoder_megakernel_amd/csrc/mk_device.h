// Device building blocks for the layer kernel: vector types, MFMA tile
// products, the grid barrier, and the workgroup "unit engine" that streams
// pre-tiled weights through the matrix cores.
#pragma once
#include "mk_common.h"

namespace mk {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ------------------------------------------------------------------ memory helpers
__device__ __forceinline__ u32x4 ld_stream16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Wait until this wave's outstanding vector memory operations completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Makes this workgroup's global writes visible device-wide: every wave drains
// its own stores, then one agent-scope release (L2 write-back) by thread 0.
// Must be called by all threads of the workgroup.
__device__ __forceinline__ void wg_release_begin() {
  wait_vmem();
  __syncthreads();
}

__device__ __forceinline__ uint64_t clock100() { return __builtin_amdgcn_s_memrealtime(); }

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x4& a, const f32x4& b) {
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}
// four OCP E4M3 codes (one dword) -> four floats (exact)
__device__ __forceinline__ f32x4 fp8x4_to_f32(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}
// eight codes -> eight bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return to_bf16x8(fp8x4_to_f32(w0), fp8x4_to_f32(w1));
}

// ------------------------------------------------------------------ MFMA
__device__ __forceinline__ f32x4 mma_bf16_k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16_k16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32_k4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Activation element type of the B operand for a weight format.
template <int FMT> struct Act { typedef __bf16 T; };
template <> struct Act<MK_FMT_F32> { typedef float T; };

// One 1 KiB weight tile times the activation slice this lane owns.
// `b` points at the lane's first activation element of the tile's k range:
// row (lane % 16) of the operand, column offset (lane / 16) * tile_k / 4.
template <int FMT>
__device__ __forceinline__ f32x4 tile_mma(const u32x4& a, const typename Act<FMT>::T* b, f32x4 acc);

template <>
__device__ __forceinline__ f32x4 tile_mma<MK_FMT_F32>(const u32x4& a, const float* b, f32x4 acc) {
  f32x4 av = __builtin_bit_cast(f32x4, a);
  f32x4 bv = *reinterpret_cast<const f32x4*>(b);
  acc = mma_f32_k4(av[0], bv[0], acc);
  acc = mma_f32_k4(av[1], bv[1], acc);
  acc = mma_f32_k4(av[2], bv[2], acc);
  acc = mma_f32_k4(av[3], bv[3], acc);
  return acc;
}
template <>
__device__ __forceinline__ f32x4 tile_mma<MK_FMT_BF16>(const u32x4& a, const __bf16* b, f32x4 acc) {
  return mma_bf16_k32(__builtin_bit_cast(bf16x8, a), *reinterpret_cast<const bf16x8*>(b), acc);
}
template <>
__device__ __forceinline__ f32x4 tile_mma<MK_FMT_FP8_B128>(const u32x4& a, const __bf16* b, f32x4 acc) {
  acc = mma_bf16_k32(fp8x8_to_bf16(a[0], a[1]), *reinterpret_cast<const bf16x8*>(b), acc);
  acc = mma_bf16_k32(fp8x8_to_bf16(a[2], a[3]), *reinterpret_cast<const bf16x8*>(b + 8), acc);
  return acc;
}

// ------------------------------------------------------------------ grid barrier
// Sense-reversing barrier over the whole persistent grid.  The wait is bounded:
// past `timeout_ticks` (100 MHz clock) the fault word is set and every later
// barrier returns false at once, so all workgroups leave the kernel.
__device__ __forceinline__ bool grid_barrier(const LayerParams& p, int idx, int* lds_flag) {
  wg_release_begin();
  if (threadIdx.x == 0) {
    int ok = 1;
    uint64_t t0 = clock100();
    if (p.trace) p.trace[(long long)blockIdx.x * (2 + 2 * kBarriers) + 1 + 2 * idx] = (long long)t0;
    BarrierState* b = p.bar;
    if (__hip_atomic_load(&b->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
      ok = 0;
    } else {
      uint32_t g = __hip_atomic_load(&b->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      uint32_t old = __hip_atomic_fetch_add(&b->count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == (uint32_t)gridDim.x - 1) {
        __hip_atomic_store(&b->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(&b->gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        while (__hip_atomic_load(&b->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
          __builtin_amdgcn_s_sleep(1);
          if ((long long)(clock100() - t0) > p.timeout_ticks) {
            __hip_atomic_store(&b->fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = 0;
            break;
          }
          if (__hip_atomic_load(&b->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
            ok = 0;
            break;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    if (p.trace) p.trace[(long long)blockIdx.x * (2 + 2 * kBarriers) + 2 + 2 * idx] = (long long)clock100();
    *lds_flag = ok;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// ------------------------------------------------------------------ unit engine
// A "unit" is 16 output rows times a range of NT weight tiles.  The 8 waves of
// the workgroup split the unit's tiles (wave w takes tiles w, w+8, ...), each
// accumulates a 16x16 MFMA block, and the partial blocks are summed in LDS in
// wave order (deterministic).  Loads run D tiles ahead across unit boundaries.
// Src provides: tile(u, t) -> const uint8_t*, bptr(u, t) -> B-operand pointer
// for this lane, scale(u, t) (fp8 only), and for DUAL units a second tile
// stream (W3 beside W1) at tile(u, t) + 1024 with scale2(u, t).
// Epi(u, row, col, v[, v2]) is called for every row < 16 and col < T.
template <int FMT, bool DUAL>
struct UnitRed {
  static constexpr int kFloats = kWaves * 64 * 4 * (DUAL ? 2 : 1);
};

// HILO: the activation operand is split into bf16 hi + lo parts (lo at
// bptr + src.lo_off); both are multiplied into the same accumulator, which
// keeps ~16 mantissa bits of an fp32 activation (used for the router logits).
template <int FMT, bool DUAL, bool HILO, class Src, class Epi>
__device__ __forceinline__ void run_units(int u0, int u1, int NT, int T, const Src& src, const Epi& epi, float* red) {
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c = (NT + kWaves - 1) / kWaves;  // tile slots per wave per unit
  const int total = (u1 - u0) * c;
  if (total <= 0) return;
  constexpr int D = 8;
  u32x4 buf[D];
  u32x4 buf2[D];
  auto issue = [&](int q, int r) {
    int uu = q / c, j = q - uu * c, t = w + kWaves * j;
    if (t < NT) {
      const uint8_t* tp = src.tile(u0 + uu, t) + lane * 16;
      buf[r] = ld_stream16(tp);
      if constexpr (DUAL) buf2[r] = ld_stream16(tp + 1024);
    }
  };
#pragma unroll
  for (int r = 0; r < D; ++r)
    if (r < total) issue(r, r);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < total; q0 += D) {
#pragma unroll
    for (int r = 0; r < D; ++r) {
      const int q = q0 + r;
      if (q < total) {
        const int uu = q / c, j = q - uu * c, t = w + kWaves * j;
        if (t < NT) {
          const auto* bp = src.bptr(u0 + uu, t);
          if constexpr (FMT == MK_FMT_FP8_B128) {
            f32x4 tmp = tile_mma<FMT>(buf[r], bp, zero);
            const float s = src.scale(u0 + uu, t);
            acc += tmp * s;
            if constexpr (DUAL) {
              f32x4 tmp2 = tile_mma<FMT>(buf2[r], bp, zero);
              acc2 += tmp2 * src.scale2(u0 + uu, t);
            }
          } else {
            acc = tile_mma<FMT>(buf[r], bp, acc);
            if constexpr (HILO) acc = tile_mma<FMT>(buf[r], bp + src.lo_off, acc);
            if constexpr (DUAL) acc2 = tile_mma<FMT>(buf2[r], bp, acc2);
          }
        }
        if (q + D < total) issue(q + D, r);
        if (j == c - 1) {
          // unit boundary: deterministic reduction over the 8 waves
          float* rb = red + ((uu & 1) ? UnitRed<FMT, DUAL>::kFloats : 0);
          *reinterpret_cast<f32x4*>(rb + (w * 64 + lane) * 4) = acc;
          if constexpr (DUAL) *reinterpret_cast<f32x4*>(rb + kWaves * 64 * 4 + (w * 64 + lane) * 4) = acc2;
          __syncthreads();
          if (threadIdx.x < 256) {
            const int col = threadIdx.x & 15, row = threadIdx.x >> 4;
            const int l = (row >> 2) * 16 + col, e = row & 3;
            if (col < T) {
              float v = 0.f, v2 = 0.f;
#pragma unroll
              for (int ww = 0; ww < kWaves; ++ww) {
                v += rb[(ww * 64 + l) * 4 + e];
                if constexpr (DUAL) v2 += rb[kWaves * 64 * 4 + (ww * 64 + l) * 4 + e];
              }
              epi(u0 + uu, row, col, v, v2);
            }
          }
          acc = zero;
          acc2 = zero;
        }
      }
    }
  }
  __syncthreads();
}

}  // namespace mk
