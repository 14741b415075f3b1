// Device building blocks for the layer kernel: vector types, MFMA tile
// products, the grid barrier, and the workgroup "unit engine" that streams
// pre-tiled weights through the matrix cores.
#pragma once
#include <type_traits>

#include "mk_common.h"

namespace mk {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// ------------------------------------------------------------------ memory helpers
// Loads from device (global) memory through global-address-space pointers.
// A load through a generic pointer becomes a FLAT instruction, which also
// counts in the LDS counter: every wait for an LDS read would then wait for
// all weight loads in flight as well.
template <class T>
using gptr = const __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ T ldg(const T* p) {
  return *(gptr<T>)(p);
}
__device__ __forceinline__ u32x4 ld_stream16(const uint8_t* p) {
  return __builtin_nontemporal_load((gptr<u32x4>)(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(gptr<u32x4>)(p); }
// A zero in a vector register that the compiler cannot see through.  An
// address offset by it counts as divergent, so its load is issued on the
// vector memory path (and counted with the weight loads around it) even when
// the address is the same for the whole wave.
__device__ __forceinline__ int vzero() {
  int z;
  asm("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}
// A register copy the compiler keeps: the copy gets a register of its own, so
// that the source register is free for the next value loaded into it (left to
// itself the compiler may merge the two, and a load into a register still in
// use then lands elsewhere and has to be moved back, after a wait for it).
__device__ __forceinline__ float keep_copy(float x) {
  float y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}
// Waits until the memory operation that produced x has returned (an
// instruction that reads x, so the compiler's counter wait covers exactly that
// operation and everything issued before it; an empty asm statement does not
// count as a read).
__device__ __forceinline__ void wait_for(uint32_t x) {
  uint32_t y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, let D[i][k] be the k-th 16-bit element of the 8 bytes at lane i's
// address; lane l of the group receives D[4e + l/4][l%4] as its element e.
// Hence, for a row-major bf16 matrix M in LDS, lane i = 4e + q pointing at
// M[r0 + e][c0 + 4q] hands every lane l the column slice M[r0 .. r0+3][c0 + l].
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Wait until this wave's outstanding vector memory operations completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Drains this workgroup's outstanding memory operations: every wave waits for
// its own loads and stores, then the workgroup synchronises.  Must be called by
// all threads of the workgroup.
__device__ __forceinline__ void wg_release_begin() {
  wait_vmem();
  __syncthreads();
}

// Agent-scope release (L2 write-back of this compute unit's XCD, so other XCDs
// can read what this workgroup wrote).  The write-back is complete when the
// wave's memory counter drains; the fence alone may leave that wait out when
// no load or store of the wave is pending (the write-back itself is not
// counted as pending), so it is spelled out.
__device__ __forceinline__ void release_agent() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  wait_vmem();
}
// Orders the compiler only: no load after it is moved above it.
__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

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
// eight codes -> eight bf16 (exact: every E4M3 value is a bf16 value, and the
// scale is 1), two codes per instruction
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// eight E4M3 codes (two dwords) times a scale -> eight bf16, two codes per
// instruction, assembled as dwords.  Exact while code * scale is a bf16 value
// (always, for a power-of-two scale inside bf16's range).
__device__ __forceinline__ u32x4 fp8x8_scaled_bf16(uint32_t w0, uint32_t w1, float s) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true))};
}
// fp32 -> OCP E4M3 code (bias 7, largest finite 448), round to nearest even,
// for |x| <= 448.  Below 2^-6 the codes are subnormal with a step of 2^-9
// (x * 512 is exact, rintf rounds half to even, and 8 is the smallest normal
// code); above, the fp32 mantissa is cut to 3 bits with the round-half-even
// increment and the exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t b = __builtin_bit_cast(uint32_t, a);
    code = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
    code = code < 0x7Eu ? code : 0x7Eu;
  }
  return sign | code;
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

// The B operand of one fp8 tile (its two k32 halves), read from LDS ahead of
// the product, and the product itself from registers.
struct BPair {
  bf16x8 lo, hi;
};
__device__ __forceinline__ BPair b_pair(const __bf16* b) {
  return BPair{*reinterpret_cast<const bf16x8*>(b), *reinterpret_cast<const bf16x8*>(b + 8)};
}
__device__ __forceinline__ f32x4 tile_mma_fp8(const u32x4& a, const BPair& b, f32x4 acc) {
  acc = mma_bf16_k32(fp8x8_to_bf16(a[0], a[1]), b.lo, acc);
  acc = mma_bf16_k32(fp8x8_to_bf16(a[2], a[3]), b.hi, acc);
  return acc;
}

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times
// the scale s -> eight bf16, one byte per instruction.  Exact: an E2M1 value
// times a power of two is a bf16 value while it stays in bf16's range.  The
// packed results are assembled as dwords (no element extraction).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float s) {
  const u32x4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3))};
  return __builtin_bit_cast(bf16x8, r);
}
// One MXFP4 tile (16 rows x 128 columns; the lane's 32 codes form one MX scale
// group of its row) times the lane's 32 activations at b: four k32 products,
// the group's scale s applied while the codes are widened.
__device__ __forceinline__ f32x4 tile_mma_mx(const u32x4& a, const __bf16* b, float s, f32x4 acc) {
#pragma unroll
  for (int d = 0; d < 4; ++d) acc = mma_bf16_k32(fp4x8_to_bf16(a[d], s), *reinterpret_cast<const bf16x8*>(b + 8 * d), acc);
  return acc;
}
// E8M0 scale byte -> the fp32 whose exponent field it is: 2^(e - 127) for
// 1 <= e <= 254; e = 0 (2^-127) as the subnormal with that value; e = 255 NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __builtin_bit_cast(float, (e << 23) | ((e == 0u || e == 255u) ? 0x00400000u : 0u));
}

// The scale of tile t of a unit whose scales start at sp.
//  fp8: one fp32 per 128x128 block; the unit's 16 rows lie in one block row,
//       so tile t (columns t * 64 ...) takes entry (t * 64) / 128.
//  MXFP4: 64 scale bytes per tile, byte l for lane l (its row's scale group);
//       the W1 and W3 scales of a dual stream alternate per tile (stride 128).
// vz (a vector zero, see vzero) keeps an fp8 scale load on the vector path.
template <int FMT, bool DUAL>
__device__ __forceinline__ float tile_scale(const float* sp, int t, int lane, int vz = 0) {
  if constexpr (FMT == MK_FMT_MXFP4) {
    const uint8_t* b = reinterpret_cast<const uint8_t*>(sp);
    return e8m0_to_f32(ldg(b + t * (DUAL ? 128 : 64) + lane + vz));
  } else {
    return ldg(sp + ((t * tile_k(FMT)) >> 7) + vz);
  }
}

// ------------------------------------------------------------------ tracing
// Timestamps of a traced launch are kept in LDS (the last KiB of the dynamic
// allocation, which no phase uses) and written out once at the end, so that no
// trace store is outstanding when a phase waits on its memory counter.
constexpr int kTraceLdsOff = kLdsBytes - 1024;
static_assert(kTraceStride * 8 <= 1024 - 16, "trace stamps and the barrier flag share the last KiB of LDS");
__device__ __forceinline__ long long* trace_lds() {
  extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
  return reinterpret_cast<long long*>(dyn_lds + kTraceLdsOff);
}

// ------------------------------------------------------------------ grid barrier
// Two-level barrier over the whole persistent grid (see BarrierState).  Each
// workgroup drains its stores into its XCD's L2 before it arrives.  With
// xcd_release (a grid that is a multiple of 8), the groups are the XCDs --
// MI355X runs workgroup b of a launch on XCD b % 8 -- and the last arrival of a
// group writes that XCD's L2 back once (agent-scope release) for all of its
// workgroups: a write-back per workgroup put the slowest workgroups' write-
// backs on every phase's critical path (measured: 15 us per layer launch).
// Every workgroup checks its XCD (hardware register XCC_ID) at each arrival; one
// on another XCD than its group's writes its own stores back and sets the
// fault word, so such a launch is reported, never silently wrong.  Otherwise
// the groups are kBarGroup consecutive workgroups and each workgroup writes its
// own stores back.  There is no acquire (L1/L2 invalidate) after the release:
// every buffer one workgroup writes and another reads after a barrier is
// written once per launch and read by no compute unit before it is written,
// and the caches are invalidated when a launch starts, so no cache can hold a
// stale copy of it; a per-workgroup invalidate would only make the first loads
// of the next phase miss (measured on MI355X: about 2 us for the first load
// after an agent-scope acquire, 0.3 us without).  The wait is bounded: past
// `timeout_ticks` (100 MHz clock) the fault word is set and every later barrier
// returns false at once, so all workgroups leave the kernel.
__device__ __forceinline__ bool grid_barrier(const LayerParams& p, int idx, int* lds_flag) {
  wg_release_begin();
  if (threadIdx.x == 0) {
    int ok = 1;
    uint64_t t0 = clock100();
    if (p.trace) trace_lds()[1 + 2 * idx] = (long long)t0;
    BarrierState* b = p.bar;
    if (__hip_atomic_load(&b->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
      ok = 0;
    } else {
      // the generation is read (and waited for) before this workgroup arrives
      const uint32_t g = __hip_atomic_load(&b->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t nwg = gridDim.x;
      bool last = false;
      if (p.xcd_release) {
        // groups = XCDs (workgroup b on XCD b % 8): every workgroup's stores are
        // in its XCD's L2 when it arrives, so the group's last arrival writes
        // that L2 back once for all of them.  A workgroup on another XCD than
        // its group's writes its own stores back and flags the launch.
        const uint32_t grp = blockIdx.x & 7, gsz = nwg / 8;
        const uint32_t gpow = gsz > 1 ? 1u << (32 - __builtin_clz(gsz - 1)) : 1u;
        const uint32_t add = blockIdx.x < 8 ? gpow - gsz + 1 : 1u;
        if ((__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7u) != grp) {
          __hip_atomic_store(&b->fault, kFaultXcd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          release_agent();
        }
        if (((__hip_atomic_fetch_add(&b->grp[grp].n, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add) &
             (gpow - 1)) == 0) {
          release_agent();
          last = ((__hip_atomic_fetch_add(&b->top.n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u) & 7u) == 0;
        }
      } else {
        release_agent();
        const uint32_t grp = blockIdx.x / kBarGroup;
        const uint32_t ngrp = (nwg + kBarGroup - 1) / kBarGroup;
        const uint32_t gsz = min((uint32_t)kBarGroup, nwg - grp * kBarGroup);
        const uint32_t add = blockIdx.x % kBarGroup == 0 ? kBarGroup - gsz + 1 : 1u;
        const uint32_t tpow = ngrp > 1 ? 1u << (32 - __builtin_clz(ngrp - 1)) : 1u;
        const uint32_t tadd = grp == 0 ? tpow - ngrp + 1 : 1u;
        if (((__hip_atomic_fetch_add(&b->grp[grp].n, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add) &
             (kBarGroup - 1)) == 0)
          last = ((__hip_atomic_fetch_add(&b->top.n, tadd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + tadd) &
                  (tpow - 1)) == 0;
      }
      if (last) {
        __hip_atomic_fetch_add(&b->gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        // the generation and the fault word are requested together, so one
        // poll costs one memory round trip
        while (true) {
          const uint32_t gc = __hip_atomic_load(&b->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t fc = __hip_atomic_load(&b->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (fc != 0) {
            ok = 0;
            break;
          }
          if (gc != g) break;
          if ((long long)(clock100() - t0) > p.timeout_ticks) {
            __hip_atomic_store(&b->fault, kFaultTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      compiler_fence();
    }
    if (p.trace) trace_lds()[2 + 2 * idx] = (long long)clock100();
    *lds_flag = ok;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// ------------------------------------------------------------------ unit engine
// A "unit" is 16 output rows times a range of NT weight tiles.  The 8 waves of
// the workgroup split the unit's tiles (wave w takes tiles w, w+8, ...), each
// accumulates a 16x16 MFMA block, and the partial blocks are summed in LDS in
// wave order (deterministic).  Every wave keeps D tile loads in flight (16 KiB
// per wave, the depth this GPU needs to approach its streaming bandwidth) and
// the stream runs on across unit boundaries.
// Src provides: base(u) -> first byte of unit u's tile 0 (tiles are `stride`
// bytes apart; for DUAL units the second matrix's tile sits 1024 bytes after
// the first), bbase(u) -> this lane's B-operand pointer for tile 0 of unit u,
// and for fp8 sbase(u) / sbase2(u) -> the unit's row of 128x128 block scales.
// Epi(u, row, col, v, v2) is called for every row < 16 and col < T.
template <int FMT, bool DUAL>
struct UnitRed {
  static constexpr int kFloats = kWaves * 64 * 4 * (DUAL ? 2 : 1);
};

// HILO: the activation operand is split into bf16 hi + lo parts (lo at
// bptr + src.lo_off); both are multiplied into the same accumulator, which
// keeps ~16 mantissa bits of an fp32 activation (used for the router logits).
template <int FMT, bool DUAL, bool HILO, class Src, class Epi>
__device__ __forceinline__ void run_units(int u0, int u1, int NT, int T, const Src& src, const Epi& epi, float* red) {
  constexpr int D = DUAL ? 8 : 16;
  constexpr int TK = tile_k(FMT);
  constexpr long long STRIDE = DUAL ? 2048 : 1024;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c = (NT + kWaves - 1) / kWaves;  // tile slots per wave per unit
  const int nu = u1 - u0;
  const int total = nu * c;
  if (total <= 0) return;
  u32x4 buf[D];
  u32x4 buf2[D];
  float sc[D], sc2[D];
  // issue cursor (block scales travel with their tiles)
  int iu = 0, ij = 0;
  const uint8_t* ib = src.base(u0) + lane * 16;
  const float* isp = nullptr;
  const float* isp2 = nullptr;
  if constexpr (scaled_fmt(FMT)) {
    isp = src.sbase(u0);
    if constexpr (DUAL) isp2 = src.sbase2(u0);
  }
  auto issue = [&](int r) {
    const int t = w + kWaves * ij;
    if (t < NT) {
      const uint8_t* tp = ib + (long long)t * STRIDE;
      buf[r] = ld_stream16(tp);
      if constexpr (DUAL) buf2[r] = ld_stream16(tp + 1024);
      if constexpr (scaled_fmt(FMT)) {
        sc[r] = tile_scale<FMT, DUAL>(isp, t, lane);
        if constexpr (DUAL) sc2[r] = tile_scale<FMT, DUAL>(isp2, t, lane);
      }
    }
    if (++ij == c) {
      ij = 0;
      if (++iu < nu) {
        ib = src.base(u0 + iu) + lane * 16;
        if constexpr (scaled_fmt(FMT)) {
          isp = src.sbase(u0 + iu);
          if constexpr (DUAL) isp2 = src.sbase2(u0 + iu);
        }
      }
    }
  };
#pragma unroll
  for (int r = 0; r < D; ++r)
    if (r < total) issue(r);
  // consume cursor
  int cu = 0, cj = 0;
  const typename Act<FMT>::T* bp0 = src.bbase(u0);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < total; q0 += D) {
#pragma unroll
    for (int r = 0; r < D; ++r) {
      const int q = q0 + r;
      if (q < total) {
        const int t = w + kWaves * cj;
        if (t < NT) {
          const auto* bp = bp0 + t * TK;
          if constexpr (FMT == MK_FMT_FP8_B128) {
            const f32x4 tmp = tile_mma<FMT>(buf[r], bp, zero);
            acc += tmp * sc[r];
            if constexpr (DUAL) {
              const f32x4 tmp2 = tile_mma<FMT>(buf2[r], bp, zero);
              acc2 += tmp2 * sc2[r];
            }
          } else if constexpr (FMT == MK_FMT_MXFP4) {
            acc = tile_mma_mx(buf[r], bp, sc[r], acc);
            if constexpr (DUAL) acc2 = tile_mma_mx(buf2[r], bp, sc2[r], acc2);
          } else {
            acc = tile_mma<FMT>(buf[r], bp, acc);
            if constexpr (HILO) acc = tile_mma<FMT>(buf[r], bp + src.lo_off, acc);
            if constexpr (DUAL) acc2 = tile_mma<FMT>(buf2[r], bp, acc2);
          }
        }
        if (q + D < total) issue(r);
        if (++cj == c) {
          // unit boundary: deterministic reduction over the 8 waves
          cj = 0;
          float* rb = red + ((cu & 1) ? UnitRed<FMT, DUAL>::kFloats : 0);
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
              epi(u0 + cu, row, col, v, v2);
            }
          }
          acc = zero;
          acc2 = zero;
          if (++cu < nu) bp0 = src.bbase(u0 + cu);
        }
      }
    }
  }
  __syncthreads();
}


// Wave-level units: each wave of the workgroup owns whole units (16 rows, all
// NT tiles) -- units u0 + w, u0 + w + 8, ... of the workgroup's range -- so no
// cross-wave reduction or workgroup barrier is needed; the D-deep load ring runs
// across the wave's units.  Epi(u, row, col, v, v2) is called per lane for the
// four rows it holds (row = 4*(lane/16) + e, col = lane % 16 < T).
template <int FMT, bool DUAL, class Src, class Epi>
__device__ __forceinline__ void run_wave_units(int u0, int u1, int NT, int T, const Src& src, const Epi& epi) {
  constexpr int D = DUAL ? 8 : 16;
  constexpr int TK = tile_k(FMT);
  constexpr long long STRIDE = DUAL ? 2048 : 1024;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nu = u1 - u0 > w ? (u1 - u0 - w + kWaves - 1) / kWaves : 0;   // units of this wave
  const int total = nu * NT;
  if (total <= 0) return;
  u32x4 buf[D];
  u32x4 buf2[D];
  float sc[D], sc2[D];
  int iu = 0, it = 0;
  const uint8_t* ib = src.base(u0 + w) + lane * 16;
  const float* isp = nullptr;
  const float* isp2 = nullptr;
  if constexpr (scaled_fmt(FMT)) {
    isp = src.sbase(u0 + w);
    if constexpr (DUAL) isp2 = src.sbase2(u0 + w);
  }
  auto issue = [&](int r) {
    const uint8_t* tp = ib + (long long)it * STRIDE;
    buf[r] = ld_stream16(tp);
    if constexpr (DUAL) buf2[r] = ld_stream16(tp + 1024);
    if constexpr (scaled_fmt(FMT)) {
      sc[r] = tile_scale<FMT, DUAL>(isp, it, lane);
      if constexpr (DUAL) sc2[r] = tile_scale<FMT, DUAL>(isp2, it, lane);
    }
    if (++it == NT) {
      it = 0;
      if (++iu < nu) {
        const int u = u0 + w + kWaves * iu;
        ib = src.base(u) + lane * 16;
        if constexpr (scaled_fmt(FMT)) {
          isp = src.sbase(u);
          if constexpr (DUAL) isp2 = src.sbase2(u);
        }
      }
    }
  };
#pragma unroll
  for (int r = 0; r < D; ++r)
    if (r < total) issue(r);
  int cu = 0, ct = 0;
  const typename Act<FMT>::T* bp0 = src.bbase(u0 + w);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < total; q0 += D) {
#pragma unroll
    for (int r = 0; r < D; ++r) {
      const int q = q0 + r;
      if (q < total) {
        const auto* bp = bp0 + ct * TK;
        if constexpr (FMT == MK_FMT_FP8_B128) {
          const f32x4 tmp = tile_mma<FMT>(buf[r], bp, zero);
          acc += tmp * sc[r];
          if constexpr (DUAL) {
            const f32x4 tmp2 = tile_mma<FMT>(buf2[r], bp, zero);
            acc2 += tmp2 * sc2[r];
          }
        } else if constexpr (FMT == MK_FMT_MXFP4) {
          acc = tile_mma_mx(buf[r], bp, sc[r], acc);
          if constexpr (DUAL) acc2 = tile_mma_mx(buf2[r], bp, sc2[r], acc2);
        } else {
          acc = tile_mma<FMT>(buf[r], bp, acc);
          if constexpr (DUAL) acc2 = tile_mma<FMT>(buf2[r], bp, acc2);
        }
        if (q + D < total) issue(r);
        if (++ct == NT) {
          ct = 0;
          const int u = u0 + w + kWaves * cu;
          const int col = lane & 15, g = lane >> 4;
          if (col < T) {
#pragma unroll
            for (int e = 0; e < 4; ++e) epi(u, 4 * g + e, col, acc[e], acc2[e]);
          }
          acc = zero;
          acc2 = zero;
          if (++cu < nu) bp0 = src.bbase(u0 + w + kWaves * cu);
        }
      }
    }
  }
}


// Branch-free streaming engine.  A wave's work is a sequence of chunks of D
// contiguous tiles; a chunk lies inside one unit.  WG mode: every unit's NT
// tiles are cut into 8 contiguous slices, wave w takes slice w of each unit of
// the workgroup's range, and unit results are reduced across waves in LDS.
// Wave mode: wave w owns units u0+w, u0+w+8, ... whole.  The loop body is
// straight-line (the next chunk's loads are issued unconditionally, the very
// last prefetch reads `dummy`, an L2-resident scratch block), so the compiler
// can keep exact s_waitcnt counts and D loads stay in flight.
// Requires: slice (NT/8 in WG mode, NT in wave mode) a multiple of D.
// Registers of one chunk of D tiles (and, for fp8, their block scales).
template <int FMT, bool DUAL, int D>
struct Chunk {
  u32x4 buf[D];
  u32x4 buf2[D];
  float sc[D], sc2[D];
};

// Issues the loads of a stream's first chunk (the same one run_stream would
// load first), so that they can be in flight while the activation operand is
// staged; run_stream<..., PRIMED = true> then starts from these registers.
// The D loads are issued whether or not this workgroup has work (without work,
// or with `enable` false, they read `dummy`), so the number of loads in flight
// after the call does not depend on a branch and later waits for older loads
// can count past them.
//
// Only the first PD tiles of the chunk are requested here (the rest when the
// stream starts): a whole chunk from every wave of the grid would fill the
// memory queues, and the activation loads that follow would wait behind it.
template <int FMT, bool DUAL, bool WG, int D, int PD = D, class Src>
__device__ __forceinline__ void stream_prime(Chunk<FMT, DUAL, D>& c, int u0, int u1, int NT, const Src& src,
                                             const uint8_t* dummy, bool enable = true) {
  constexpr long long STRIDE = DUAL ? 2048 : 1024;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int slice = WG ? NT / kWaves : NT;
  const int nu = WG ? (u1 - u0) : (u1 - u0 > w ? (u1 - u0 - w + kWaves - 1) / kWaves : 0);
  const bool any = enable && nu > 0 && slice / D > 0;
  const int toff = WG ? w * slice : 0;
  const uint8_t* cbase = dummy + lane * 16;
  const float* sp = reinterpret_cast<const float*>(dummy);
  const float* sp2 = sp;
  int soff = 0;
  if (any) {
    const int u = WG ? u0 : u0 + w;
    cbase = src.base(u) + lane * 16 + (long long)toff * STRIDE;
    if constexpr (scaled_fmt(FMT)) {
      sp = src.sbase(u);
      if constexpr (DUAL) sp2 = src.sbase2(u);
    }
    soff = toff;
  }
#pragma unroll
  for (int r = 0; r < PD; ++r) {
    c.buf[r] = ld_stream16(cbase + r * STRIDE);
    if constexpr (DUAL) c.buf2[r] = ld_stream16(cbase + r * STRIDE + 1024);
    if constexpr (scaled_fmt(FMT)) {
      const int st = any ? soff + r : 0;
      c.sc[r] = tile_scale<FMT, DUAL>(sp, st, lane);
      if constexpr (DUAL) c.sc2[r] = tile_scale<FMT, DUAL>(sp2, st, lane);
    }
  }
}

template <int FMT, bool DUAL, bool HILO, bool WG, int D, bool PRIMED = false, int PD = D, class Src, class Epi>
__device__ __forceinline__ void run_stream(int u0, int u1, int NT, int T, const Src& src, const Epi& epi, float* red,
                                           const uint8_t* dummy, Chunk<FMT, DUAL, D>* pre = nullptr) {
  constexpr int TK = tile_k(FMT);
  constexpr long long STRIDE = DUAL ? 2048 : 1024;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int slice = WG ? NT / kWaves : NT;
  const int cps = slice / D;
  const int ustep = WG ? 1 : kWaves;
  const int ufirst = WG ? u0 : u0 + w;
  const int nu = WG ? (u1 - u0) : (u1 - u0 > w ? (u1 - u0 - w + kWaves - 1) / kWaves : 0);
  const int nchunks = nu * cps;
  if (nchunks <= 0) return;
  const int toff = WG ? w * slice : 0;
  const float* dsc = reinterpret_cast<const float*>(dummy);
  Chunk<FMT, DUAL, D> local;
  Chunk<FMT, DUAL, D>& ck = PRIMED ? *pre : local;
  u32x4 (&buf)[D] = ck.buf;
  u32x4 (&buf2)[D] = ck.buf2;
  float (&sc)[D] = ck.sc;
  float (&sc2)[D] = ck.sc2;
  auto load_chunk = [&](const uint8_t* cbase, const float* sp, const float* sp2, int tfirst) {
#pragma unroll
    for (int r = 0; r < D; ++r) {
      buf[r] = ld_stream16(cbase + r * STRIDE);
      if constexpr (DUAL) buf2[r] = ld_stream16(cbase + r * STRIDE + 1024);
      if constexpr (scaled_fmt(FMT)) {
        sc[r] = tile_scale<FMT, DUAL>(sp, tfirst + r, lane);
        if constexpr (DUAL) sc2[r] = tile_scale<FMT, DUAL>(sp2, tfirst + r, lane);
      }
    }
  };
  if constexpr (!PRIMED) {
    const int u = ufirst;
    const float* sp = nullptr;
    const float* sp2 = nullptr;
    if constexpr (scaled_fmt(FMT)) {
      sp = src.sbase(u);
      if constexpr (DUAL) sp2 = src.sbase2(u);
    }
    load_chunk(src.base(u) + lane * 16 + (long long)toff * STRIDE, sp, sp2, toff);
  } else if constexpr (PD < D) {
    // the tiles of the first chunk that stream_prime left out
    const int u = ufirst;
    const uint8_t* cbase = src.base(u) + lane * 16 + (long long)toff * STRIDE;
#pragma unroll
    for (int r = PD; r < D; ++r) {
      buf[r] = ld_stream16(cbase + r * STRIDE);
      if constexpr (DUAL) buf2[r] = ld_stream16(cbase + r * STRIDE + 1024);
      if constexpr (scaled_fmt(FMT)) {
        sc[r] = tile_scale<FMT, DUAL>(src.sbase(u), toff + r, lane);
        if constexpr (DUAL) sc2[r] = tile_scale<FMT, DUAL>(src.sbase2(u), toff + r, lane);
      }
    }
  }
  int cu = 0, cc = 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < nchunks; ++k) {
    int ncc = cc + 1, ncu = cu;
    if (ncc == cps) {
      ncc = 0;
      ++ncu;
    }
    const bool has_next = k + 1 < nchunks;
    const int un = ufirst + ncu * ustep;
    const int tn = toff + ncc * D;
    const uint8_t* nb = has_next ? src.base(un) + lane * 16 + (long long)tn * STRIDE : dummy + lane * 16;
    const float* nsp = dsc;
    const float* nsp2 = dsc;
    if constexpr (scaled_fmt(FMT)) {
      if (has_next) {
        nsp = src.sbase(un);
        if constexpr (DUAL) nsp2 = src.sbase2(un);
      }
    }
    const int tc = toff + cc * D;
    const auto* bp = src.bbase(ufirst + cu * ustep) + tc * TK;
#pragma unroll
    for (int r = 0; r < D; ++r) {
      if constexpr (FMT == MK_FMT_FP8_B128) {
        const f32x4 tmp = tile_mma<FMT>(buf[r], bp + r * TK, zero);
        acc += tmp * sc[r];
        if constexpr (DUAL) {
          const f32x4 tmp2 = tile_mma<FMT>(buf2[r], bp + r * TK, zero);
          acc2 += tmp2 * sc2[r];
        }
      } else if constexpr (FMT == MK_FMT_MXFP4) {
        acc = tile_mma_mx(buf[r], bp + r * TK, sc[r], acc);
        if constexpr (DUAL) acc2 = tile_mma_mx(buf2[r], bp + r * TK, sc2[r], acc2);
      } else {
        acc = tile_mma<FMT>(buf[r], bp + r * TK, acc);
        if constexpr (HILO) acc = tile_mma<FMT>(buf[r], bp + r * TK + src.lo_off, acc);
        if constexpr (DUAL) acc2 = tile_mma<FMT>(buf2[r], bp + r * TK, acc2);
      }
      buf[r] = ld_stream16(nb + r * STRIDE);
      if constexpr (DUAL) buf2[r] = ld_stream16(nb + r * STRIDE + 1024);
      if constexpr (scaled_fmt(FMT)) {
        const int st = has_next ? tn + r : 0;
        sc[r] = tile_scale<FMT, DUAL>(nsp, st, lane);
        if constexpr (DUAL) sc2[r] = tile_scale<FMT, DUAL>(nsp2, st, lane);
      }
    }
    if (ncc == 0) {
      const int u = ufirst + cu * ustep;
      if constexpr (WG) {
        float* rb = red + ((cu & 1) ? UnitRed<FMT, DUAL>::kFloats : 0);
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
            epi(u, row, col, v, v2);
          }
        }
      } else {
        const int col = lane & 15, g = lane >> 4;
        if (col < T) {
#pragma unroll
          for (int e = 0; e < 4; ++e) epi(u, 4 * g + e, col, acc[e], acc2[e]);
        }
      }
      acc = zero;
      acc2 = zero;
    }
    cc = ncc;
    cu = ncu;
  }
  if constexpr (WG) __syncthreads();
}

// Workgroup-mode streaming over a unit sequence handed out at run time, so
// that workgroups on faster XCDs take more units.  Workgroup b first takes
// units b and b + nwg; the others (2 nwg + i) are handed out by eight ticket
// counters, counter c owning the units with i % 8 == c: a workgroup draws
// from the counter of its XCD (b % 8) and moves on to the next counter when
// that one is exhausted, which spreads the atomics over eight addresses.
// Wave 0 asks for the ticket of unit j+2 when unit j starts and publishes the
// answer through LDS (`seq`, two slots) at unit j's reduction, so the ticket's
// round trip overlaps a whole unit of streaming and the next unit's first
// chunk is always requested one chunk ahead, as in run_stream.  The counters
// `ctr[kCntStride * c]` must be zero before the first workgroup gets here.  Requires slice = NT/8
// to be a multiple of D.
//
// SPLIT = 2: the workgroup works on two units at a time (a group of units
// 2g, 2g + 1 is what a ticket hands out), waves 0-3 on the first and 4-7 on the
// second, each unit's NT tiles cut into 4 slices -- twice the bytes per wave
// of a unit, for formats whose rows hold few tiles.  A group's second unit
// beyond U (odd U) is streamed again as unit U - 1 and discarded.
//
// With a Done callback (not NoDone), the epilogue works on row pairs instead:
// epi(u, row0, col, v0, v2_0, v1, v2_1) for rows row0 and row0 + 1 (threads
// < 128) writes them with value-returning atomics and returns the reply.  A
// unit is published one unit later: at the end of the next unit every thread
// uses the replies it holds (so it waits for those writes alone, not for the
// chunk requested since, which a wait for all its memory operations would
// drain), and after a workgroup barrier thread 0 calls done(u).  The last
// unit is published when the stream ends.
//
// `pre` runs after the first chunk has been requested and before it is used
// (the activation operand can be staged there while that chunk is on its way).
struct NoDone {
  __device__ void operator()(int) const {}
};
struct NoPre {
  __device__ void operator()() const {}
};
template <int FMT, bool DUAL, int D, int SPLIT = 1, class Src, class Epi, class Done = NoDone, class Pre = NoPre>
__device__ __forceinline__ void run_stream_dyn(int U, int NT, int T, const Src& src, const Epi& epi, float* red,
                                               const uint8_t* dummy, uint32_t* ctr, int* seq,
                                               const Done& done = Done(), const Pre& pre = Pre()) {
  constexpr bool kPairs = !std::is_same<Done, NoDone>::value;
  constexpr int TK = tile_k(FMT);
  constexpr long long STRIDE = DUAL ? 2048 : 1024;
  constexpr int WPU = kWaves / SPLIT;              // waves per unit
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nwg = (int)gridDim.x;
  const int half = w / WPU;                        // which unit of the group this wave streams
  const int slice = NT / WPU;
  const int cps = slice / D;
  const int toff = (w % WPU) * slice;
  const int UG = (U + SPLIT - 1) / SPLIT;          // unit groups
  auto sub = [&](int g) { return min(g * SPLIT + half, U - 1); };
  int cur = (int)blockIdx.x < UG ? (int)blockIdx.x : -1;
  int nxt = (int)blockIdx.x + nwg < UG ? (int)blockIdx.x + nwg : -1;
  if (cur < 0 || cps <= 0) {
    pre();
    return;
  }
  const float* dsc = reinterpret_cast<const float*>(dummy);
  u32x4 buf[D], buf2[D];
  float sc[D], sc2[D];
  {
    // issued exactly as the loop issues a chunk (same order, scales on the
    // vector path too), so that the loop's waits count the same loads whether
    // it is entered from here or from its own end
    const int u = sub(cur);
    const uint8_t* cbase = src.base(u) + lane * 16 + (long long)toff * STRIDE;
    const int vz = vzero();
#pragma unroll
    for (int r = 0; r < D; ++r) {
      buf[r] = ld_stream16(cbase + r * STRIDE);
      if constexpr (DUAL) buf2[r] = ld_stream16(cbase + r * STRIDE + 1024);
      if constexpr (scaled_fmt(FMT)) {
        sc[r] = tile_scale<FMT, DUAL>(src.sbase(u), toff + r, lane, vz);
        if constexpr (DUAL) sc2[r] = tile_scale<FMT, DUAL>(src.sbase2(u), toff + r, lane, vz);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  pre();
  uint32_t tk = 0;
  int cq = (int)blockIdx.x & 7;     // counter drawn from (thread 0)
  int cc = 0, par = 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // fp8: each tile's B operand is read one tile ahead (bn) and its scaled
  // product is added one tile later (tp * sp), so neither the LDS latency nor
  // the MFMA latency lies between a tile's arrival and the request of its
  // successor; the sums are formed in the same order as without the delay
  BPair bn;
  f32x4 tp = zero, tp2 = zero;
  float sp = 0.f, sp2 = 0.f;
  if constexpr (FMT == MK_FMT_FP8_B128) bn = b_pair(src.bbase(sub(cur)) + toff * TK);
  uint32_t reply = 0;               // row-pair epilogue: the reply of this thread's last write
  int prev = -1;                    // row-pair epilogue: the unit written but not yet published
  while (true) {
    if (cc == 0 && threadIdx.x == 0)
      tk = __hip_atomic_fetch_add(ctr + kCntStride * cq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ncc = cc + 1, un = cur;
    if (ncc == cps) {
      ncc = 0;
      un = nxt;
    }
    const bool has_next = un >= 0;
    const int tn = toff + ncc * D;
    const int unu = has_next ? sub(un) : 0;
    const uint8_t* nb = has_next ? src.base(unu) + lane * 16 + (long long)tn * STRIDE : dummy + lane * 16;
    const float* nsp = dsc;
    const float* nsp2 = dsc;
    if constexpr (scaled_fmt(FMT)) {
      if (has_next) {
        nsp = src.sbase(unu);
        if constexpr (DUAL) nsp2 = src.sbase2(unu);
      }
    }
    const auto* bp = src.bbase(sub(cur)) + (toff + cc * D) * TK;
#pragma unroll
    for (int r = 0; r < D; ++r) {
      if constexpr (FMT == MK_FMT_FP8_B128) {
        const BPair b = bn;
        bn = b_pair(r + 1 < D ? bp + (r + 1) * TK : (has_next ? src.bbase(unu) + tn * TK : bp));
        const f32x4 tmp = tile_mma_fp8(buf[r], b, zero);
        acc += tp * sp;
        tp = tmp;
        sp = keep_copy(sc[r]);
        if constexpr (DUAL) {
          const f32x4 tmp2 = tile_mma_fp8(buf2[r], b, zero);
          acc2 += tp2 * sp2;
          tp2 = tmp2;
          sp2 = keep_copy(sc2[r]);
        }
      } else if constexpr (FMT == MK_FMT_MXFP4) {
        acc = tile_mma_mx(buf[r], bp + r * TK, sc[r], acc);
        if constexpr (DUAL) acc2 = tile_mma_mx(buf2[r], bp + r * TK, sc2[r], acc2);
      } else {
        acc = tile_mma<FMT>(buf[r], bp + r * TK, acc);
        if constexpr (DUAL) acc2 = tile_mma<FMT>(buf2[r], bp + r * TK, acc2);
      }
      buf[r] = ld_stream16(nb + r * STRIDE);
      if constexpr (DUAL) buf2[r] = ld_stream16(nb + r * STRIDE + 1024);
      if constexpr (scaled_fmt(FMT)) {
        const int st = has_next ? tn + r : 0;
        sc[r] = tile_scale<FMT, DUAL>(nsp, st, lane);
        if constexpr (DUAL) sc2[r] = tile_scale<FMT, DUAL>(nsp2, st, lane);
      }
      // tile r's next load leaves before tile r + 1 is used: the loads stay in
      // the order they are consumed, so each wait is for one tile and D tiles
      // stay in flight (left to itself the scheduler bunches the loads late
      // and an early tile then waits for nearly the whole chunk)
      __builtin_amdgcn_sched_barrier(0);
    }
    cc = ncc;
    if (ncc != 0) continue;
    // unit `cur` complete: reduce across the waves, publish the unit after nxt
    if constexpr (FMT == MK_FMT_FP8_B128) {
      acc += tp * sp;
      tp = zero;
      sp = 0.f;
      if constexpr (DUAL) {
        acc2 += tp2 * sp2;
        tp2 = zero;
        sp2 = 0.f;
      }
    }
    float* rb = red + (par ? UnitRed<FMT, DUAL>::kFloats : 0);
    *reinterpret_cast<f32x4*>(rb + (w * 64 + lane) * 4) = acc;
    if constexpr (DUAL) *reinterpret_cast<f32x4*>(rb + kWaves * 64 * 4 + (w * 64 + lane) * 4) = acc2;
    if (threadIdx.x == 0) {
      long long un2 = 2LL * nwg + 8LL * tk + cq;
      for (int tries = 1; un2 >= UG && tries < 8; ++tries) {
        cq = (cq + 1) & 7;
        tk = __hip_atomic_fetch_add(ctr + kCntStride * cq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        un2 = 2LL * nwg + 8LL * tk + cq;
      }
      seq[par] = un2 < UG ? (int)un2 : -1;
    }
    __syncthreads();
    if constexpr (!kPairs) {
      if (threadIdx.x < 256 * SPLIT) {
        const int h = threadIdx.x >> 8, t = threadIdx.x & 255;
        const int col = t & 15, row = t >> 4;
        const int l = (row >> 2) * 16 + col, e = row & 3;
        const int u = cur * SPLIT + h;
        if (col < T && u < U) {
          float v = 0.f, v2 = 0.f;
#pragma unroll
          for (int ww = h * WPU; ww < (h + 1) * WPU; ++ww) {
            v += rb[(ww * 64 + l) * 4 + e];
            if constexpr (DUAL) v2 += rb[kWaves * 64 * 4 + (ww * 64 + l) * 4 + e];
          }
          epi(u, row, col, v, v2);
        }
      }
    } else {
      // the previous unit's writes have completed once their replies are here
      // (used before this unit's writes reuse the register)
      wait_for(reply);
      if (threadIdx.x < 128 * SPLIT) {
        const int h = threadIdx.x >> 7, t = threadIdx.x & 127;
        const int col = t & 15, row = (t >> 4) * 2;
        const int l = (row >> 2) * 16 + col, e = row & 3;
        const int u = cur * SPLIT + h;
        if (col < T && u < U) {
          float v0 = 0.f, v1 = 0.f, w0 = 0.f, w1 = 0.f;
#pragma unroll
          for (int ww = h * WPU; ww < (h + 1) * WPU; ++ww) {
            v0 += rb[(ww * 64 + l) * 4 + e];
            v1 += rb[(ww * 64 + l) * 4 + e + 1];
            if constexpr (DUAL) {
              w0 += rb[kWaves * 64 * 4 + (ww * 64 + l) * 4 + e];
              w1 += rb[kWaves * 64 * 4 + (ww * 64 + l) * 4 + e + 1];
            }
          }
          reply = epi(u, row, col, v0, w0, v1, w1);
        }
      }
      __syncthreads();
      if (threadIdx.x == 0 && prev >= 0)
        for (int h = 0; h < SPLIT; ++h)
          if (prev * SPLIT + h < U) done(prev * SPLIT + h);
      prev = cur;
    }
    acc = zero;
    acc2 = zero;
    cur = nxt;
    nxt = nxt >= 0 ? seq[par] : -1;
    par ^= 1;
    if (cur < 0) break;
  }
  if constexpr (kPairs) {
    wait_for(reply);
    __syncthreads();
    if (threadIdx.x == 0 && prev >= 0)
      for (int h = 0; h < SPLIT; ++h)
        if (prev * SPLIT + h < U) done(prev * SPLIT + h);
  }
  __syncthreads();
}

// Dispatch: the branch-free engine when the slice length allows, else the
// general engines (ragged shapes).
template <int FMT, bool DUAL, bool HILO, class Src, class Epi>
__device__ __forceinline__ void stream_units_wg(int u0, int u1, int NT, int T, const Src& src, const Epi& epi,
                                                float* red, const uint8_t* dummy) {
  const int slice = NT % kWaves == 0 ? NT / kWaves : 0;
  constexpr int DMAX = DUAL ? 8 : 16;
  if (slice > 0 && slice % DMAX == 0) run_stream<FMT, DUAL, HILO, true, DMAX>(u0, u1, NT, T, src, epi, red, dummy);
  else if (slice > 0 && slice % 4 == 0) run_stream<FMT, DUAL, HILO, true, 4>(u0, u1, NT, T, src, epi, red, dummy);
  else if (slice > 0 && slice % 2 == 0) run_stream<FMT, DUAL, HILO, true, 2>(u0, u1, NT, T, src, epi, red, dummy);
  else run_units<FMT, DUAL, HILO>(u0, u1, NT, T, src, epi, red);
}
// Workgroup-mode streaming whose first chunk may have been primed: when the
// slice allows the full-depth engine (`primed` tells whether stream_prime ran
// with the same arguments), else the general engines.
template <int FMT, bool DUAL, bool HILO, int PD = (DUAL ? 8 : 16), class Src, class Epi>
__device__ __forceinline__ void stream_units_wg_primed(int u0, int u1, int NT, int T, const Src& src, const Epi& epi,
                                                       float* red, const uint8_t* dummy,
                                                       Chunk<FMT, DUAL, DUAL ? 8 : 16>& pre, bool primed) {
  constexpr int DMAX = DUAL ? 8 : 16;
  if (primed) run_stream<FMT, DUAL, HILO, true, DMAX, true, PD>(u0, u1, NT, T, src, epi, red, dummy, &pre);
  else stream_units_wg<FMT, DUAL, HILO>(u0, u1, NT, T, src, epi, red, dummy);
}
// Whether stream_units_wg_primed can use a primed first chunk for this slice.
__host__ __device__ constexpr bool wg_primable(int NT, bool dual) {
  return NT % kWaves == 0 && (NT / kWaves) % (dual ? 8 : 16) == 0;
}

template <int FMT, bool DUAL, class Src, class Epi>
__device__ __forceinline__ void stream_units_wave(int u0, int u1, int NT, int T, const Src& src, const Epi& epi,
                                                  const uint8_t* dummy) {
  constexpr int DMAX = DUAL ? 8 : 16;
  if (NT % DMAX == 0) run_stream<FMT, DUAL, false, false, DMAX>(u0, u1, NT, T, src, epi, nullptr, dummy);
  else run_wave_units<FMT, DUAL>(u0, u1, NT, T, src, epi);
}

}  // namespace mk
