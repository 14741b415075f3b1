// The layer megakernel: one persistent launch computes a whole verify step of a
// latent-attention mixture-of-experts decoder layer (the step listed, kernel by
// kernel, in "Why one GB300 doesn't beat 4x RTX PRO 6000 at single-stream
// decode", section "Where the 11.2 ms goes"; the attention algebra is the
// multi-head latent attention of the DeepSeek-V2 paper, section 2.1).
//
// Phases, separated by grid barriers (all workgroups are co-resident):
//   P0  RMSNorm-1 (every workgroup, into LDS) ; [W_Q; W_DKV] x, split-K partials
//   P1  RoPE on q^R and the shared key, KV insert ; absorbed query q~ = W_UK^T q^C
//   P2  latent attention, split over (query tile, KV range): partial (Z, max, sum)
//   P3  merge of the KV splits (log-sum-exp) into z and o = W_UV z, per
//       (head, pair of verify rows)
//   P4  H' = H + W_O o
//   P5  RMSNorm-2 (every workgroup, into LDS) ; router logits on E/16
//       workgroups, each keeping the top k of its 16 experts per token as
//       candidates; the shared experts' gate+up on the other workgroups
//   P6  every workgroup: top-k / gates / the distinct-expert work list from the
//       candidates; gate+up projections of every routed expert: silu(W1 x) * W3 x
//   P7  down projections W2 h of every listed expert
//   P8  out = H' + sum_k gate_k y_k + y_shared
#pragma once
#include <type_traits>

#include "mk_device.h"

namespace mk {

// Tiles of a phase's first chunk requested ahead of its activation rows (of 16).
constexpr int kPrimeTiles = 8;

// ------------------------------------------------------------------ LDS plan
struct LdsPlan {
  int xb;        // bytes of one activation operand [kMaxT][dmax + pad]
  __device__ LdsPlan(const LayerParams& p, int esize) {
    int dmax = p.d;
    if (p.nh * p.dh > dmax) dmax = p.nh * p.dh;
    if (p.f > dmax) dmax = p.f;
    xb = kMaxT * (dmax + kXPad) * esize;
    xb = (xb + 255) & ~255;
  }
};
constexpr int kFlagOff = kLdsBytes - 16;        // the barrier flag, after the trace stamps
constexpr int kSeqOff = kLdsBytes - 32;         // two ints: unit sequence of the ticket-fed streams
__device__ __forceinline__ int* seq_lds() {
  extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
  return reinterpret_cast<int*>(dyn_lds + kSeqOff);
}

// sub-phase timestamp (thread 0, only when tracing)
__device__ __forceinline__ void trace_x(const LayerParams& p, int slot) {
  if (p.trace && threadIdx.x == 0) trace_lds()[2 + 2 * kBarriers + slot] = (long long)clock100();
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sums of N values over the wave, all reduced together so that each step's
// cross-lane moves are issued back to back: DPP moves (VALU, no LDS round
// trip) combine the lanes of each row of 16, then two swizzles combine the
// four rows.  The association differs from lane to lane, so the N results are
// to be read from one lane (lane 0 here).
template <int N>
__device__ __forceinline__ void wave_sums(float (&v)[N]) {
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  typedef std::integral_constant<int, 0xB1> qp1032;    // quad_perm [1,0,3,2]
  typedef std::integral_constant<int, 0x4E> qp2301;    // quad_perm [2,3,0,1]
  typedef std::integral_constant<int, 0x124> ror4;     // row_ror:4
  typedef std::integral_constant<int, 0x128> ror8;     // row_ror:8
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp(v[i], qp1032());
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp(v[i], qp2301());
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp(v[i], ror4());
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp(v[i], ror8());
  float u[N];
#pragma unroll
  for (int i = 0; i < N; ++i) u[i] = __shfl_xor(v[i], 16);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += u[i];
#pragma unroll
  for (int i = 0; i < N; ++i) u[i] = __shfl_xor(v[i], 32);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += u[i];
}

// [a, b) = the i-th of `parts` near-equal slices of [0, total) (total * parts < 2^32)
__device__ __forceinline__ void split_range(int total, int parts, int i, int& a, int& b) {
  a = (int)((unsigned)total * (unsigned)i / (unsigned)parts);
  b = (int)((unsigned)total * (unsigned)(i + 1) / (unsigned)parts);
}

template <class A> __device__ inline A to_act(float v);
template <> __device__ inline float to_act<float>(float v) { return v; }
template <> __device__ inline __bf16 to_act<__bf16>(float v) { return (__bf16)v; }

template <class A> __device__ __forceinline__ void store4(A* dst, const f32x4& v);
template <> __device__ __forceinline__ void store4<float>(float* dst, const f32x4& v) {
  *reinterpret_cast<f32x4*>(dst) = v;
}
template <> __device__ __forceinline__ void store4<__bf16>(__bf16* dst, const f32x4& v) {
  bf16x4 b;
  b[0] = (__bf16)v[0]; b[1] = (__bf16)v[1]; b[2] = (__bf16)v[2]; b[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4*>(dst) = b;
}
template <class A> __device__ __forceinline__ f32x4 round4(const f32x4& v);
template <> __device__ __forceinline__ f32x4 round4<float>(const f32x4& v) { return v; }
template <> __device__ __forceinline__ f32x4 round4<__bf16>(const f32x4& v) {
  return f32x4{(float)(__bf16)v[0], (float)(__bf16)v[1], (float)(__bf16)v[2], (float)(__bf16)v[3]};
}

// Stages T <= kMaxT fp32 rows of length K (K % 4 == 0, K <= kMaxModel) into
// LDS as the MFMA operand type, row stride XS.  Wave w holds the float4
// columns w*64 + lane + 512 c of every row, so a lane keeps at most
// kMaxT x kRowCh float4s and the gain slice they share.  With NORM the rows
// are RMS-normalised, but not on the way: what is stored is h * gamma, and
// 1/rms = rsqrt(mean(h^2) + eps) of each row (the VALU's reciprocal square
// root instruction, about 1 ulp; the waves' partial sums of squares meet in
// LDS and are added in wave order) goes to LDS (rsc_lds) for the consumers'
// epilogues to scale their products by -- W (h gamma / rms) = (W (h gamma)) /
// rms -- so no cross-wave reduction lies between the row loads and the stores
// the first matrix product waits for.  `lo` (optional) receives the remainder
// x - round(x) for the router's split operand.
//
// issue() only requests the row (and gain) loads; finish() stores them.  A
// phase that also streams weights calls issue(), then requests its first
// weight chunk, then finish(): each wave's loads complete in order, so the
// activation rows arrive ahead of the weights instead of behind them.  Every
// lane issues the same number of loads (indices past a row are clamped to its
// last float4, rows past T-1 to row T-1; neither is stored), so the compiler
// can wait for exactly the older loads.
constexpr int kRowCh = kMaxModel / (kWaves * 64 * 4);     // float4s per lane per row
constexpr int kNormLdsOff = kLdsBytes - 640;              // [kWaves][kMaxT] partial sums
constexpr int kRscLdsOff = kLdsBytes - 384;               // [kMaxT] 1/rms of the staged rows
static_assert(kTraceStride * 8 <= 384, "the normalisation partials follow the trace stamps");
__device__ __forceinline__ const float* rsc_lds() {
  extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
  return reinterpret_cast<const float*>(dyn_lds + kRscLdsOff);
}
template <class A, bool NORM>
struct RowStager {
  f32x4 v[kMaxT][kRowCh];
  f32x4 gm[kRowCh];
  __device__ __forceinline__ void issue(const float* src, int T, int K, const float* gamma) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n4 = K / 4;
#pragma unroll
    for (int c = 0; c < kRowCh; ++c) {
      const int i = min(w * 64 + lane + c * kWaves * 64, n4 - 1);
      if constexpr (NORM) gm[c] = ldg(reinterpret_cast<const f32x4*>(gamma + 4 * i));
#pragma unroll
      for (int t = 0; t < kMaxT; ++t)
        v[t][c] = ldg(reinterpret_cast<const f32x4*>(src + (long long)min(t, T - 1) * K + 4 * i));
    }
  }
  // The rows as sums of S split-K partials: row t element k = sum_s
  // part[(s T + t) stride + k] (the S loads of an element are issued together).
  __device__ __forceinline__ void issue_sum(const float* part, int S, int T, long long stride, int K,
                                            const float* gamma) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n4 = K / 4;
#pragma unroll
    for (int c = 0; c < kRowCh; ++c) {
      const int i = min(w * 64 + lane + c * kWaves * 64, n4 - 1);
      if constexpr (NORM) gm[c] = ldg(reinterpret_cast<const f32x4*>(gamma + 4 * i));
#pragma unroll
      for (int t = 0; t < kMaxT; ++t) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < S; ++s)
          a += ldg(reinterpret_cast<const f32x4*>(part + ((long long)s * T + min(t, T - 1)) * stride + 4 * i));
        v[t][c] = a;
      }
    }
  }
  __device__ __forceinline__ void finish(int T, int K, A* xs, A* lo, int XS, float eps, bool tr = false) {
    extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
    float* part = reinterpret_cast<float*>(dyn_lds + kNormLdsOff);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n4 = K / 4;
    if constexpr (NORM) {
      float ss[kMaxT];
#pragma unroll
      for (int t = 0; t < kMaxT; ++t) {
        ss[t] = 0.f;
#pragma unroll
        for (int c = 0; c < kRowCh; ++c)
          if (w * 64 + lane + c * kWaves * 64 < n4)
            ss[t] += v[t][c][0] * v[t][c][0] + v[t][c][1] * v[t][c][1] + v[t][c][2] * v[t][c][2] +
                     v[t][c][3] * v[t][c][3];
      }
      if (tr && threadIdx.x == 0) trace_lds()[2 + 2 * kBarriers + 11] = (long long)clock100();
      wave_sums(ss);
      if (lane == 0) {
#pragma unroll
        for (int t = 0; t < kMaxT; ++t) part[w * kMaxT + t] = ss[t];
      }
    }
#pragma unroll
    for (int c = 0; c < kRowCh; ++c) {
      const int i = w * 64 + lane + c * kWaves * 64;
      if (i < n4) {
#pragma unroll
        for (int t = 0; t < kMaxT; ++t) {
          if (t < T) {
            f32x4 x = v[t][c];
            if constexpr (NORM) x = x * gm[c];
            store4<A>(xs + (long long)t * XS + 4 * i, x);
            if (lo) store4<A>(lo + (long long)t * XS + 4 * i, x - round4<A>(x));
          }
        }
      }
    }
    __syncthreads();
    if constexpr (NORM) {
      // read by the epilogues after a later workgroup barrier
      if ((int)threadIdx.x < kMaxT) {
        float ss = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) ss += part[ww * kMaxT + threadIdx.x];
        reinterpret_cast<float*>(dyn_lds + kRscLdsOff)[threadIdx.x] = __builtin_amdgcn_rsqf(ss * (1.0f / (float)K) + eps);
      }
    }
  }
};

// Copies T <= kMaxT rows of length K already in the operand type A from global
// memory into LDS (row stride XS): wave w copies row w in 16-byte pieces.
// issue() / finish() split as in RowStager.
template <class A>
struct RowCopier {
  static constexpr int EPV = 16 / sizeof(A);                  // elements per 16 bytes
  static constexpr int CH = kMaxStageK / EPV / 64;
  u32x4 v[CH];
  __device__ __forceinline__ void issue(const A* src, int T, int K) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nv = K / EPV;
    const A* row = src + (long long)min(w, T - 1) * K;
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = ld16(row + min(lane + 64 * c, nv - 1) * EPV);
  }
  __device__ __forceinline__ void finish(int T, int K, A* xs, int XS) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nv = K / EPV;
    if (w < T) {
      A* xr = xs + (long long)w * XS;
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (lane + 64 * c < nv) {
          const uint2 lo = {v[c][0], v[c][1]}, hi = {v[c][2], v[c][3]};
          *reinterpret_cast<uint2*>(xr + (lane + 64 * c) * EPV) = lo;
          *reinterpret_cast<uint2*>(xr + (lane + 64 * c) * EPV + EPV / 2) = hi;
        }
    }
    __syncthreads();
  }
};

template <class A>
__device__ __forceinline__ void rows_copy_lds(const A* src, int T, int K, A* xs, int XS) {
  RowCopier<A> c;
  c.issue(src, T, K);
  c.finish(T, K, xs, XS);
}

template <class A>
__device__ __forceinline__ const A* b_lane(const A* xs, int XS, int T, int TK) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int jj = j < T ? j : T - 1;
  return xs + jj * XS + g * (TK / 4);
}

// ------------------------------------------------------------------ P0
// LR (low-rank query): the query rows are W_DQ's ql rows (c^Q) instead of W_Q's.
template <int AF, bool LR = false, bool SP = false>
__device__ __forceinline__ void phase_qkv(const LayerParams& p, char* smem) {
  typedef typename Act<AF>::T A;
  constexpr int TK = tile_k(AF);
  const int T = p.T, XS = p.d + kXPad;
  LdsPlan lp(p, sizeof(A));
  A* xs = reinterpret_cast<A*>(smem);
  float* red = reinterpret_cast<float*>(smem + lp.xb);
  const int nqp = LR ? p.ql : p.nq;
  const int nidx = SP ? p.ihead * p.idim + p.ihead + p.idim : 0;     // the indexer's rows (sparse attention)
  const int RTq = nqp / 16, RTkv = (p.kvw + 15) / 16, RTi = nidx / 16, KT = p.d / TK, S = p.sch.s_q, NT = KT / S;
  const int U = (RTq + RTkv + RTi) * S;
  int u0, u1;
  split_range(U, gridDim.x, blockIdx.x, u0, u1);
  const A* bl = b_lane<A>(xs, XS, T, TK);
  const int nrow = nqp + p.kvw + nidx;
  struct Src {
    const uint8_t* wq; const uint8_t* wd; const uint8_t* wi; int RTq, RTkv, KT, S, NT; const A* bl;
    __device__ const uint8_t* base(int u) const {
      const int rt = u / S, s = u - rt * S;
      const uint8_t* b = rt < RTq ? wq + (long long)rt * KT * 1024
                       : (!SP || rt < RTq + RTkv) ? wd + (long long)(rt - RTq) * KT * 1024
                       : wi + (long long)(rt - RTq - RTkv) * KT * 1024;
      return b + (long long)s * NT * 1024;
    }
    __device__ const A* bbase(int u) const { return bl + (u % S) * NT * TK; }
    __device__ const float* sbase(int) const { return nullptr; }
    __device__ const float* sbase2(int) const { return nullptr; }
  } src{LR ? p.wdq : p.wq, p.wdkv, p.widx, RTq, RTkv, KT, S, NT, bl};
  float* part = p.qkv_part;
  const int nq = nqp, kvw = p.kvw;
  const float* rsc = rsc_lds();       // the staged rows are h * gamma: scale by 1/rms
  auto epi = [=](int u, int row, int col, float v, float) {
    v *= rsc[col];
    int rt = u / S, s = u - rt * S;
    int idx;
    if (rt < RTq) idx = rt * 16 + row;
    else if (!SP || rt < RTq + RTkv) {
      int r = (rt - RTq) * 16 + row;
      if (r >= kvw) return;
      idx = nq + r;
    } else {
      idx = nq + kvw + (rt - RTq - RTkv) * 16 + row;
    }
    part[((long long)s * T + col) * nrow + idx] = v;
  };
  // the input rows are requested first, then the first weight chunk, so the
  // rows are normalised while the weights are on their way
  RowStager<A, true> rs;
  rs.issue(p.H, T, p.d, p.g1);
  trace_x(p, 10);
  Chunk<AF, false, 16> ck;
  const bool pr = wg_primable(NT, false);
  stream_prime<AF, false, true, 16, kPrimeTiles>(ck, u0, u1, NT, src, p.dummy, pr);
  trace_x(p, 3);
  rs.finish(T, p.d, xs, (A*)nullptr, XS, p.eps, p.trace != nullptr);
  trace_x(p, 5);
  stream_units_wg_primed<AF, false, false, kPrimeTiles>(u0, u1, NT, T, src, epi, red, p.dummy, ck, pr);
}

// ------------------------------------------------------------------ P0b (low-rank query)
// q = W_UQ (q-norm(c^Q)): every workgroup sums the split-K partials of c^Q for
// the T rows, stages c^Q * gamma_q into LDS with 1/rms per row (as RMSNorm-1
// is staged), then the row tiles of W_UQ are streamed over the grid and each
// product is scaled by its row's 1/rms into qbuf [T][nq].
template <int AF, bool SP = false>
__device__ __forceinline__ void phase_uq(const LayerParams& p, char* smem) {
  typedef typename Act<AF>::T A;
  constexpr int TK = tile_k(AF);
  const int T = p.T, K = p.ql, XS = K + kXPad;
  LdsPlan lp(p, sizeof(A));
  A* xs = reinterpret_cast<A*>(smem);
  float* red = reinterpret_cast<float*>(smem + lp.xb);
  const int RT = p.nq / 16, KT = K / TK;
  int u0, u1;
  split_range(RT, gridDim.x, blockIdx.x, u0, u1);
  const A* bl = b_lane<A>(xs, XS, T, TK);
  struct Src {
    const uint8_t* w; int KT; const A* bl;
    __device__ const uint8_t* base(int u) const { return w + (long long)u * KT * 1024; }
    __device__ const A* bbase(int) const { return bl; }
    __device__ const float* sbase(int) const { return nullptr; }
    __device__ const float* sbase2(int) const { return nullptr; }
  } src{p.wuq, KT, bl};
  float* q = p.qbuf;
  const int nq = p.nq;
  const float* rsc = rsc_lds();
  auto epi = [=](int u, int row, int col, float v, float) { q[(long long)col * nq + u * 16 + row] = v * rsc[col]; };
  RowStager<A, true> rs;
  rs.issue_sum(p.qkv_part, p.sch.s_q, T, p.ql + p.kvw + (SP ? p.ihead * p.idim + p.ihead + p.idim : 0), K, p.gq);
  rs.finish(T, K, xs, (A*)nullptr, XS, p.eps);
  stream_units_wg<AF, false, false>(u0, u1, KT, T, src, epi, red, p.dummy);
}

// ------------------------------------------------------------------ P1
// sin and cos of 2 pi x for |x| <= 1/2 (x in turns), in fp64: x is split into
// the nearest quarter turn n/4 and g = x - n/4 in [-1/8, 1/8], the Taylor
// series of sin and cos at t = 2 pi g (|t| <= pi/4) are summed to t^17 and t^16
// (remainders below 1e-17), and the quarter turn swaps and negates the pair.
__device__ __forceinline__ void sincos_turns(double x, double& sn, double& cs) {
  const double n = rint(4.0 * x);
  const double t = (x - 0.25 * n) * 6.283185307179586476925286766559;
  const double t2 = t * t;
  double ps = 0.0, pc = 0.0;
  double fs = 1.0 / 355687428096000.0;        // 1/17!
  double fc = 1.0 / 20922789888000.0;         // 1/16!
#pragma unroll
  for (int k = 8; k >= 0; --k) {
    ps = ps * t2 + ((k & 1) ? -fs : fs);
    pc = pc * t2 + ((k & 1) ? -fc : fc);
    fs *= (double)((2 * k + 1) * (2 * k));    // 1/(2k+1)! -> 1/(2k-1)!
    fc *= (double)((2 * k) * (2 * k - 1));    // 1/(2k)!   -> 1/(2k-2)!
  }
  const double s0 = ps * t, c0 = pc;
  const int q = (int)n & 3;
  sn = q == 0 ? s0 : q == 1 ? c0 : q == 2 ? -s0 : -c0;
  cs = q == 0 ? c0 : q == 1 ? -s0 : q == 2 ? -c0 : s0;
}

// Rotation of pair i at position pos by the angle pos * rope_base^(-2i/d_rope):
// the frequency is rope_step^i (square-and-multiply in fp64), the angle is
// taken in turns and reduced to [-1/2, 1/2] in fp64 before sin and cos.
__device__ __forceinline__ void rope_cs(long long pos, int pidx, double step, float& c, float& s) {
  double th = 1.0, b = step;
  for (int e = pidx; e > 0; e >>= 1) {
    if (e & 1) th *= b;
    b *= b;
  }
  const double x = (double)pos * (th * 0.15915494309189533576888376337251);   // / (2 pi)
  double sn, cs;
  sincos_turns(x - rint(x), sn, cs);
  c = (float)cs;
  s = (float)sn;
}

// Work items are spread over the threads [tid0, tid0 + nthreads) of the grid
// given by the caller (`tid` is this thread's index in that range).  LR: the
// layer has a low-rank query, which P0b left whole in qbuf; the first
// projection's partials then hold [c^Q | c | k_R] rows of ql + kvw values.
// SP (sparse attention): the partial rows end with the indexer's rows [q^I | w^I | k^I], and
// each new cache row also receives its index key k^I after the RoPE key.
template <int KF, bool LR = false, bool SP = false>
__device__ __forceinline__ void phase_rope_kv(const LayerParams& p, int L, int tid, int nthreads) {
  const int T = p.T, S = p.sch.s_q, dr2 = p.dr / 2;
  const int kvoff = LR ? p.ql : p.nq;                              // where c starts in a partial row
  const int kioff = kvoff + p.kvw + (SP ? p.ihead * p.idim + p.ihead : 0);   // where k^I starts
  const int nrow = kvoff + p.kvw + (SP ? p.ihead * p.idim + p.ihead + p.idim : 0);
  const int per_t = p.dc + dr2 + p.nh * dr2 + (SP ? p.idim : 0);
  const float* part = p.qkv_part;
  auto psum = [&](int t, int idx) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += ldg(part + ((long long)s * T + t) * nrow + idx);
    return v;
  };
  // element idx of row t's query [n_h][d_h + d_r]
  auto qval = [&](int t, int idx) { return LR ? ldg(p.qbuf + (long long)t * p.nq + idx) : psum(t, idx); };
  if constexpr (KF == MK_FMT_FP8_ROW || LR) {
    // One wave per new cache row (the thread range is whole waves): each lane
    // forms runs of 8 consecutive values (latent, 4 rotated key pairs, or with
    // sparse attention the index key, whose runs follow the RoPE key's).
    // With the latent norm the wave first takes the latent's mean square and
    // scales it by 1/rms and the gain.  fp8 rows: the wave takes the row
    // maximum, the row's scale is the smallest power of two 2^e with
    // max <= 448 * 2^e, and each value is stored as E4M3(v / 2^e); fp32 / bf16
    // rows store the values.
    const int lane = tid & 63, wv = tid >> 6, nwv = nthreads >> 6;
    const int rb = kv_row_bytes(KF, p.kv_row), nrun = p.kvw / 8, nall = p.kv_row / 8;
    for (int t = wv; t < T; t += nwv) {
      const long long pos = (long long)L + t;
      // the key's RoPE pairs: lane j < d_r / 2 forms pair j's cos and sin, and the
      // lanes holding rotated runs fetch theirs (shuffles in uniform control flow)
      float rc = 1.f, rsn = 0.f;
      if (lane < dr2) rope_cs(pos, lane, p.rope_step, rc, rsn);
      float pcs[2][4], psn[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = lane + 64 * i;
        const int pb = (8 * c >= p.dc && c < nrun) ? (8 * c - p.dc) / 2 : 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          pcs[i][k] = __shfl(rc, pb + k);
          psn[i][k] = __shfl(rsn, pb + k);
        }
      }
      float v[2][8];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = lane + 64 * i, m0 = 8 * c;
#pragma unroll
        for (int k = 0; k < 8; ++k) v[i][k] = 0.f;
        if (c < nall) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
          const int off = c < nrun ? kvoff + m0 : kioff + (m0 - p.kvw);
          for (int s = 0; s < S; ++s) {
            const float* src = part + ((long long)s * T + t) * nrow + off;
            a += ldg(reinterpret_cast<const f32x4*>(src));
            b += ldg(reinterpret_cast<const f32x4*>(src + 4));
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[i][k] = a[k];
            v[i][k + 4] = b[k];
          }
          if (m0 >= p.dc && c < nrun) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float cs = pcs[i][k], sn = psn[i][k];
              const float x0 = v[i][2 * k], x1 = v[i][2 * k + 1];
              v[i][2 * k] = x0 * cs - x1 * sn;
              v[i][2 * k + 1] = x0 * sn + x1 * cs;
            }
          }
        }
      }
      if (LR && p.kv_norm) {
        // RMSNorm of the latent (runs below d_c), as 1 / sqrt(mean square + eps) times the gain
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (8 * (lane + 64 * i) < p.dc)
#pragma unroll
            for (int k = 0; k < 8; ++k) ss += v[i][k] * v[i][k];
        ss = wave_sum(ss);
        const float r = 1.0f / sqrtf(ss / (float)p.dc + p.eps);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int m0 = 8 * (lane + 64 * i);
          if (m0 < p.dc) {
            const f32x4 g0 = ldg(reinterpret_cast<const f32x4*>(p.gkv + m0));
            const f32x4 g1 = ldg(reinterpret_cast<const f32x4*>(p.gkv + m0 + 4));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              v[i][k] = (v[i][k] * r) * g0[k];
              v[i][k + 4] = (v[i][k + 4] * r) * g1[k];
            }
          }
        }
      }
      if constexpr (KF != MK_FMT_FP8_ROW) {
        // fp32 / bf16 rows: the values themselves
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int c = lane + 64 * i;
          if (c < nall) {
            if constexpr (KF == MK_FMT_F32) {
              float* dst = reinterpret_cast<float*>(p.kv) + pos * p.kv_row + 8 * c;
              *reinterpret_cast<f32x4*>(dst) = f32x4{v[i][0], v[i][1], v[i][2], v[i][3]};
              *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[i][4], v[i][5], v[i][6], v[i][7]};
            } else {
              bf16x8 o;
#pragma unroll
              for (int k = 0; k < 8; ++k) o[k] = (__bf16)v[i][k];
              *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(p.kv) + pos * p.kv_row + 8 * c) = o;
            }
          }
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[i][k]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      int e = 0;
      if (amax > 0.f) {
        const uint32_t ab = __builtin_bit_cast(uint32_t, amax);
        e = (int)(ab >> 23) - 135 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0);   // mantissa above 1.75
        e = e < -100 ? -100 : e;
      }
      const float inv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);
      uint8_t* row = reinterpret_cast<uint8_t*>(p.kv) + pos * rb;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = lane + 64 * i;
        if (c < nall) {
          uint32_t w0 = 0, w1 = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            w0 |= e4m3_rne(v[i][k] * inv) << (8 * k);
            w1 |= e4m3_rne(v[i][k + 4] * inv) << (8 * k);
          }
          *reinterpret_cast<u32x2*>(row + 8 * c) = u32x2{w0, w1};
        }
      }
      // the scale and the zero padding: the 16 bytes after the codes (kv_row is a multiple of 16)
      if (lane == 0)
        *reinterpret_cast<u32x4*>(row + p.kv_row) = u32x4{(uint32_t)(127 + e) << 23, 0u, 0u, 0u};
    }
    // the queries' RoPE pairs, one per thread
    const int per_q = p.nh * dr2;
    for (int it = tid; it < T * per_q; it += nthreads) {
      const int t = it / per_q, q = it - t * per_q, h = q / dr2, pi = q - h * dr2;
      const long long pos = (long long)L + t;
      const int src = h * p.qw + p.dh + 2 * pi;
      const float x0 = qval(t, src), x1 = qval(t, src + 1);
      float c, sn;
      rope_cs(pos, pi, p.rope_step, c, sn);
      p.qrope[((long long)t * p.nh + h) * p.dr + 2 * pi] = x0 * c - x1 * sn;
      p.qrope[((long long)t * p.nh + h) * p.dr + 2 * pi + 1] = x0 * sn + x1 * c;
    }
    return;
  }
  for (int it = tid; it < T * per_t; it += nthreads) {
    const int t = it / per_t, r = it - t * per_t;
    const long long pos = (long long)L + t;
    if (SP && r >= p.dc + dr2 + p.nh * dr2) {
      // the row's index key, after the RoPE key
      const int m = r - (p.dc + dr2 + p.nh * dr2);
      const float v = psum(t, kioff + m);
      if (KF == MK_FMT_F32) reinterpret_cast<float*>(p.kv)[pos * p.kv_row + p.kvw + m] = v;
      else reinterpret_cast<__bf16*>(p.kv)[pos * p.kv_row + p.kvw + m] = (__bf16)v;
      continue;
    }
    if (r < p.dc) {
      float v = psum(t, p.nq + r);
      if (KF == MK_FMT_F32) reinterpret_cast<float*>(p.kv)[pos * p.kv_row + r] = v;
      else reinterpret_cast<__bf16*>(p.kv)[pos * p.kv_row + r] = (__bf16)v;
      continue;
    }
    // a RoPE pair: of the key (k^R, into the cache) or of head h's query
    const bool key = r < p.dc + dr2;
    const int q = r - p.dc - dr2, h = key ? 0 : q / dr2, pi = key ? r - p.dc : q - h * dr2;
    const int src = key ? p.nq + p.dc + 2 * pi : h * p.qw + p.dh + 2 * pi;
    const float x0 = psum(t, src), x1 = psum(t, src + 1);
    float c, sn;
    rope_cs(pos, pi, p.rope_step, c, sn);
    const float v0 = x0 * c - x1 * sn, v1 = x0 * sn + x1 * c;
    if (key) {
      const long long o = pos * p.kv_row + p.dc + 2 * pi;
      if (KF == MK_FMT_F32) {
        reinterpret_cast<float*>(p.kv)[o] = v0;
        reinterpret_cast<float*>(p.kv)[o + 1] = v1;
      } else {
        reinterpret_cast<__bf16*>(p.kv)[o] = (__bf16)v0;
        reinterpret_cast<__bf16*>(p.kv)[o + 1] = (__bf16)v1;
      }
    } else {
      p.qrope[((long long)t * p.nh + h) * p.dr + 2 * pi] = v0;
      p.qrope[((long long)t * p.nh + h) * p.dr + 2 * pi + 1] = v1;
    }
  }
}

// B operand held in registers for wave-level units.
template <int FMT> struct BReg { typedef bf16x8 T; };
template <> struct BReg<MK_FMT_F32> { typedef f32x4 T; };

template <int FMT>
__device__ __forceinline__ f32x4 tile_mma_reg(const u32x4& a, const typename BReg<FMT>::T& b, f32x4 acc);
template <>
__device__ __forceinline__ f32x4 tile_mma_reg<MK_FMT_F32>(const u32x4& a, const f32x4& b, f32x4 acc) {
  f32x4 av = __builtin_bit_cast(f32x4, a);
  acc = mma_f32_k4(av[0], b[0], acc);
  acc = mma_f32_k4(av[1], b[1], acc);
  acc = mma_f32_k4(av[2], b[2], acc);
  acc = mma_f32_k4(av[3], b[3], acc);
  return acc;
}
template <>
__device__ __forceinline__ f32x4 tile_mma_reg<MK_FMT_BF16>(const u32x4& a, const bf16x8& b, f32x4 acc) {
  return mma_bf16_k32(__builtin_bit_cast(bf16x8, a), b, acc);
}
// 4 (f32) or 8 (bf16) consecutive floats from global memory as the B-operand type
template <int FMT>
__device__ __forceinline__ typename BReg<FMT>::T load_b(const float* src);
template <>
__device__ __forceinline__ f32x4 load_b<MK_FMT_F32>(const float* src) { return ldg(reinterpret_cast<const f32x4*>(src)); }
template <>
__device__ __forceinline__ bf16x8 load_b<MK_FMT_BF16>(const float* src) {
  return to_bf16x8(ldg(reinterpret_cast<const f32x4*>(src)), ldg(reinterpret_cast<const f32x4*>(src + 4)));
}

template <int FMT>
__device__ __forceinline__ typename BReg<FMT>::T make_b(const f32x4& a, const f32x4& b);
template <>
__device__ __forceinline__ f32x4 make_b<MK_FMT_F32>(const f32x4& a, const f32x4&) { return a; }
template <>
__device__ __forceinline__ bf16x8 make_b<MK_FMT_BF16>(const f32x4& a, const f32x4& b) { return to_bf16x8(a, b); }

// q~[t][h][m] = sum_e W_UK[h][e][m] q^C[t][h][e]  (wave-level units: one head, 16 m-rows, all of K).
// LR: q^C comes whole from qbuf (low-rank query) instead of the split-K partials.
template <int AF, bool LR = false, bool SP = false>
__device__ __forceinline__ void phase_absorb(const LayerParams& p) {
  constexpr int TK = tile_k(AF);
  constexpr int EPL = TK / 4;          // elements per lane per tile
  const int T = p.T, S = LR ? 1 : p.sch.s_q;
  const int nrow = LR ? p.nq : p.nq + p.kvw + (SP ? p.ihead * p.idim + p.ihead + p.idim : 0);
  const float* qsrc = LR ? p.qbuf : p.qkv_part;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int jj = j < T ? j : T - 1;
  const int RT = p.dc / 16, KT = p.dh / TK, U = p.nh * RT;
  for (int u = blockIdx.x + gridDim.x * w; u < U; u += gridDim.x * kWaves) {
    const int h = u / RT, rt = u - h * RT;
    const uint8_t* tiles = p.wuk + (long long)u * KT * 1024 + lane * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    u32x4 at[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
      if (kt < KT) at[kt] = ld_stream16(tiles + kt * 1024);
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      if (kt >= KT) break;
      const u32x4 a = at[kt];
      const int e0 = kt * TK + g * EPL;
      f32x4 q0 = {0.f, 0.f, 0.f, 0.f}, q1 = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < S; ++s) {
        const float* src = qsrc + ((long long)s * T + jj) * nrow + h * p.qw + e0;
        q0 += ldg(reinterpret_cast<const f32x4*>(src));
        if (EPL == 8) q1 += ldg(reinterpret_cast<const f32x4*>(src + 4));
      }
      acc = tile_mma_reg<AF>(a, make_b<AF>(q0, q1), acc);
    }
    if (j < T) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.qabs[((long long)j * p.nh + h) * p.dc + rt * 16 + 4 * g + e] = acc[e];
    }
  }
}

// ------------------------------------------------------------------ P1b, P1c sparse attention
// Index queries: during P1 the grid sums the split-K partials of the indexer's
// query rows q^I (T x idx_heads x idx_dim) into bf16 and of its head weights
// w^I into fp32, once, so that every workgroup of the index-score phase reads
// half the bytes of the fp32 partials.
template <bool LR>
__device__ __forceinline__ void stage_index_queries(const LayerParams& p, int gi, int gn) {
  const int T = p.T, HI = p.ihead, dI = p.idim, S = p.sch.s_q;
  const int qoff = (LR ? p.ql : p.nq) + p.kvw, woff = qoff + HI * dI, nrow = woff + HI + dI;
  const int n4 = HI * dI / 4, nq4 = T * n4;
  const float* part = p.qkv_part;
  for (int i = gi; i < nq4 + T * HI; i += gn) {
    if (i < nq4) {
      const int t = i / n4, e = (i - t * n4) * 4;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < S; ++s) a += ldg(reinterpret_cast<const f32x4*>(part + ((long long)s * T + t) * nrow + qoff + e));
      store4<__bf16>(reinterpret_cast<__bf16*>(p.iq) + (long long)t * HI * dI + e, a);
    } else {
      const int k = i - nq4, t = k / HI, h = k - t * HI;
      float a = 0.f;
      for (int s = 0; s < S; ++s) a += ldg(part + ((long long)s * T + t) * nrow + woff + h);
      p.iw[k] = a;
    }
  }
}

// Order-preserving 32-bit key of a score: a larger float has a larger key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Index scores: the cache rows [0, L + T) are cut into chunks of 16 spread over
// the grid; a workgroup stages up to kIdxBlk of its chunks' index keys in LDS
// (bf16, row stride idx_dim + 8; F8: fp8 rows, whose index-key codes are widened
// with the row's scale, exactly).  Wave w scores verify row t = w / (8 / T)
// against every (8 / T)-th staged chunk, with that row's index queries held in
// registers: S[head][key] = q^I_head . k^I_key on the matrix cores (16 heads x
// 16 keys per product, idim / 32 k-steps), then the sum over heads of
// w^I_head * max(0, S) -- four heads per lane, the four lane groups added by
// shuffles.  Scores go to iscore[t][key] (row stride idx_max_rows, a multiple of 4).
constexpr int kIdxBlk = 32;                       // chunks of 16 keys staged at a time
static_assert(kIdxBlk * 16 * (128 + 8) * 2 + kMaxT * 256 * 4 <= kLdsBytes - 1024,
              "index keys (idx_dim <= 128) and head weights (idx_heads <= 256) fit the LDS");
template <int NKB, bool F8>                       // idx_dim / 32, fp8 cache rows
__device__ __forceinline__ void iscore_rows(const LayerParams& p, int L, char* smem) {
  constexpr int kMaxHt = 16 / NKB;                // idx_heads * idx_dim <= 8192: 16 query fragments per lane
  const int T = p.T, HI = p.ihead, nht = HI / 16, dI = NKB * 32, KS = dI + 8;
  __bf16* ks = reinterpret_cast<__bf16*>(smem);                              // [kIdxBlk * 16][KS]
  float* wsm = reinterpret_cast<float*>(smem + kIdxBlk * 16 * KS * 2);       // [T][HI]
  for (int i = threadIdx.x; i < T * HI; i += kThreads) wsm[i] = ldg(p.iw + i);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int wpt = T < kWaves ? kWaves / T : 1;
  const bool act = w < T * wpt;
  const int t = act ? w / wpt : 0, sub = w - t * wpt;
  bf16x8 qf[kMaxHt][NKB];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.iq) + (long long)t * HI * dI + g * 8;
#pragma unroll
    for (int ht = 0; ht < kMaxHt; ++ht)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        qf[ht][kb] = ht < nht && act ? __builtin_bit_cast(bf16x8, ld16(qrow + (ht * 16 + j) * dI + kb * 32))
                                     : bf16x8{};
  }
  const int Lt = L + T, nch = (Lt + 15) / 16, np = dI / 8;
  int c0, c1;
  split_range(nch, gridDim.x, blockIdx.x, c0, c1);
  const __bf16* kvb = reinterpret_cast<const __bf16*>(p.kv) + p.kvw;
  const uint8_t* kv8 = reinterpret_cast<const uint8_t*>(p.kv);
  const long long rb8 = kv_row_bytes(MK_FMT_FP8_ROW, p.kv_row);
  for (int cb = c0; cb < c1; cb += kIdxBlk) {
    const int nb = min(kIdxBlk, c1 - cb), tot = nb * 16 * np;
    constexpr int kB = 8;                         // 16-byte loads in flight per thread
    __syncthreads();                              // the previous block's keys are no longer read
    if constexpr (F8) {
      // 16 codes (16 bytes) and the row's scale per piece -> 16 bf16
      const int np16 = np / 2, tot16 = tot / 2;
      for (int i0 = threadIdx.x; i0 < tot16; i0 += kB * kThreads) {
        u32x4 v[kB];
        float sc[kB];
#pragma unroll
        for (int q = 0; q < kB; ++q) {
          const int i = min(i0 + q * kThreads, tot16 - 1), k = i / np16;
          const uint8_t* row = kv8 + (long long)min(cb * 16 + k, Lt - 1) * rb8;
          v[q] = ldg(reinterpret_cast<const u32x4*>(row + p.kvw + (i - k * np16) * 16));
          sc[q] = ldg(reinterpret_cast<const float*>(row + p.kv_row));
        }
#pragma unroll
        for (int q = 0; q < kB; ++q) {
          const int i = i0 + q * kThreads, k = i / np16;
          if (i < tot16) {
            __bf16* dst = ks + k * KS + (i - k * np16) * 16;
            *reinterpret_cast<u32x4*>(dst) = fp8x8_scaled_bf16(v[q][0], v[q][1], sc[q]);
            *reinterpret_cast<u32x4*>(dst + 8) = fp8x8_scaled_bf16(v[q][2], v[q][3], sc[q]);
          }
        }
      }
    } else {
      // bf16 rows: 8 values (16 bytes) per piece
      for (int i0 = threadIdx.x; i0 < tot; i0 += kB * kThreads) {
        u32x4 v[kB];
#pragma unroll
        for (int q = 0; q < kB; ++q) {
          const int i = min(i0 + q * kThreads, tot - 1), k = i / np;
          v[q] = ld16(kvb + (long long)min(cb * 16 + k, Lt - 1) * p.kv_row + (i - k * np) * 8);
        }
#pragma unroll
        for (int q = 0; q < kB; ++q) {
          const int i = i0 + q * kThreads, k = i / np;
          if (i < tot) *reinterpret_cast<u32x4*>(ks + k * KS + (i - k * np) * 8) = v[q];
        }
      }
    }
    __syncthreads();
    if (!act) continue;
    for (int cl = sub; cl < nb; cl += wpt) {
      bf16x8 kf[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) kf[kb] = *reinterpret_cast<const bf16x8*>(ks + (cl * 16 + j) * KS + kb * 32 + g * 8);
      float sc = 0.f;
#pragma unroll
      for (int ht = 0; ht < kMaxHt; ++ht) {
        if (ht < nht) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) acc = mma_bf16_k32(qf[ht][kb], kf[kb], acc);
          const f32x4 wh = *reinterpret_cast<const f32x4*>(wsm + t * HI + ht * 16 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc += acc[e] > 0.f ? wh[e] * acc[e] : 0.f;
        }
      }
      sc += __shfl_xor(sc, 16);
      sc += __shfl_xor(sc, 32);
      const int key = (cb + cl) * 16 + j;
      if (g == 0 && key < Lt) {
        p.iscore[(long long)t * p.imax + key] = sc;
        p.ik16[(long long)t * p.imax + key] = (uint16_t)(order_key(sc) >> 16);
      }
    }
  }
}
template <bool F8>
__device__ __forceinline__ void phase_iscore(const LayerParams& p, int L, char* smem) {
  switch (p.idim / 32) {
    case 1: iscore_rows<1, F8>(p, L, smem); break;
    case 2: iscore_rows<2, F8>(p, L, smem); break;
    case 3: iscore_rows<3, F8>(p, L, smem); break;
    default: iscore_rows<4, F8>(p, L, smem); break;
  }
}

// Top-k per verify row: row t keeps its idx_topk highest scores among cache
// rows [0, L + t], by a radix select on the scores' order-preserving 32-bit
// keys, digit by digit from the top; each digit is the bin where the running
// count from the top of a histogram reaches the rows still to take (found by a
// scan over the threads).  Row t is shared by P = grid / T workgroups, each
// taking a part of at least 2048 consecutive rows; the index-score phase also
// stored every key's top 16 bits, and the parts work on those:
//  - each part counts the top 11 bits of its rows in LDS and adds the bins into
//    the row's histogram in memory (device-scope atomics), then waits until
//    every part of the row has (a bounded wait on a counter) and reads the sum:
//    every part finds the same first digit;
//  - each part writes its rows at or above that digit's bin -- the kept rows
//    above it and the candidates in it -- as (row, full 32-bit key) pairs (the
//    scores read for those rows only), in ascending order from its first row's
//    place, with their count, and counts itself done;
//  - the row's first part waits for the others, gathers the pairs into a list
//    in LDS (ascending rows), takes the last 21 bits from the list (11 + 10),
//    and writes the kept rows in ascending order (each lane's place found by
//    ballots); of the rows equal to the threshold key the lower ones are kept.
// Pairs, counts and histograms are written and read with device-scope
// accesses, so no cache on the way holds a stale copy.  When the list would
// not fit in LDS (many equal or nearly equal scores), the first part alone
// takes every digit and the output from the row's full keys.
// Inclusive scan of v over the workgroup's threads: wave scans by shuffles,
// then the wave totals through LDS (buf: kWaves ints).  Ends synced.
__device__ __forceinline__ int wg_scan_incl(int v, int* buf) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) buf[w] = v;
  __syncthreads();
  int base = 0;
  for (int u = 0; u < w; ++u) base += buf[u];
  __syncthreads();
  return v + base;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
constexpr int kTopkBatch = 8;                     // float4 tiles in flight per lane
constexpr int kTopkBins = 2048;
constexpr int kTopkList = 11264;                  // LDS list capacity (rows)
constexpr int kTopkPart = 2048;                   // least rows of one part of a row
// calls f(tile base, keys of the lane's 4 rows) for the wave's float tiles in
// [b0, b1); rows at or past n read a clamped address (the row's own stride holds them)
template <class F>
__device__ __forceinline__ void for_tiles(const float* sc, int b0, int b1, int n, F&& f) {
  const int lane = threadIdx.x & 63, cap = (n - 1) / 4 * 4;
  for (int b = b0; b < b1; b += 256 * kTopkBatch) {
    f32x4 v[kTopkBatch];
#pragma unroll
    for (int q = 0; q < kTopkBatch; ++q) v[q] = ldg(reinterpret_cast<const f32x4*>(sc + min(b + q * 256 + 4 * lane, cap)));
#pragma unroll
    for (int q = 0; q < kTopkBatch; ++q) {
      if (b + q * 256 < b1) {
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = order_key(v[q][e]);
        f(b + q * 256, u);
      }
    }
  }
}
// the 8 16-bit keys of rows [b, b + 8) (b a multiple of 8; rows at or past n
// read a clamped address inside the row's stride)
__device__ __forceinline__ void keys16(const uint16_t* k16, int b, int n, uint32_t (&u)[8]) {
  const u32x4 v = ld16(k16 + min(b, (n - 1) / 8 * 8));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u[2 * e] = v[e] & 0xFFFFu;
    u[2 * e + 1] = v[e] >> 16;
  }
}
// the digit of a 2048-bin histogram: thread x holds bins 2047 - 4x .. 2044 - 4x
// (h4[q] = bin 2047 - 4x - q); the thread whose running count from the top
// reaches `need` writes the bin, the rows in higher bins and the rows in it to
// res[0..2].  Ends synced.
__device__ __forceinline__ void digit_of(const int (&h4)[4], int need, int* sbuf, int* res) {
  const int s4 = h4[0] + h4[1] + h4[2] + h4[3];
  const int incl = wg_scan_incl(s4, sbuf);
  const int before = incl - s4;
  if (before < need && need <= incl) {
    int cum = before, dg = 0, hb = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (cum + h4[q] >= need) {
        dg = kTopkBins - 1 - 4 * (int)threadIdx.x - q;
        hb = h4[q];
        break;
      }
      cum += h4[q];
    }
    res[0] = dg;
    res[1] = cum;
    res[2] = hb;
  }
  __syncthreads();
}
// Thread 0 waits (bounded) until *ctr reaches `target`; false when the wait gave
// up or the launch already failed (the fault word is then set).
__device__ __forceinline__ bool wait_count(const LayerParams& p, const uint32_t* ctr, uint32_t target) {
  const uint64_t t0 = clock100();
  while (true) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    if (__hip_atomic_load(&p.bar->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
    if ((long long)(clock100() - t0) > p.timeout_ticks) {
      __hip_atomic_store(&p.bar->fault, kFaultTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}
struct TopkLds {
  int* hist;       // [kWaves][kTopkBins]
  int* sbuf;       // [kWaves]
  int* res;        // digit: bin, rows in higher bins, rows in it; flag
  int* wc;         // [kWaves][2]
  int* poff;       // [kThreads] parts' places in the list
  uint32_t* lkey;  // [kTopkList]
  int* lrow;       // [kTopkList]
  __device__ explicit TopkLds(char* smem) {
    hist = reinterpret_cast<int*>(smem);
    sbuf = hist + kWaves * kTopkBins;
    res = sbuf + kWaves;
    wc = res + 4;
    poff = wc + 2 * kWaves;
    lkey = reinterpret_cast<uint32_t*>(poff + kThreads);
    lrow = reinterpret_cast<int*>(lkey + kTopkList);
  }
};
static_assert((kWaves * kTopkBins + kWaves + 4 + 2 * kWaves + kThreads + 2 * kTopkList) * 4 <= kLdsBytes - 1024,
              "the top-k LDS plan fits");
// Writes the kept rows of one group of up to 64 x NE rows in ascending order:
// lane l holds rows[l * NE + e] (ok: the row takes part) with keys u; G / E
// count the rows above / at the threshold before the group (wave-uniform, updated).
template <int NE>
__device__ __forceinline__ void topk_write(int32_t* out, const int (&rows)[NE], const uint32_t (&u)[NE],
                                           const bool (&ok)[NE], uint32_t thr, int need, int& G, int& E) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (1ull << lane) - 1ull;
  bool gt[NE], eq[NE];
  int gb = 0, eb = 0, gs = 0, es = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    gt[e] = ok[e] && u[e] > thr;
    eq[e] = ok[e] && u[e] == thr;
    const uint64_t bg = __ballot(gt[e]), be = __ballot(eq[e]);
    gb += __popcll(bg & lt);
    eb += __popcll(be & lt);
    gs += __popcll(bg);
    es += __popcll(be);
  }
  int gi = G + gb, ei = E + eb;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    if (gt[e]) {
      out[gi + min(ei, need)] = rows[e];
      ++gi;
    } else if (eq[e]) {
      if (ei < need) out[gi + ei] = rows[e];
      ++ei;
    }
  }
  G += gs;
  E += es;
}
// the digit of the next pass from the per-wave histograms (thread x sums bins
// 2047 - 4x .. 2044 - 4x of all waves); updates the threshold's bits and the
// rows still to take at them, returns the digit
__device__ __forceinline__ int topk_next_digit(const TopkLds& s, int shift, uint32_t dmask, uint32_t& prefix,
                                               uint32_t& mask, int& need) {
  int g4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int bin = kTopkBins - 1 - 4 * (int)threadIdx.x - q;
    g4[q] = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) g4[q] += s.hist[v * kTopkBins + bin];
  }
  digit_of(g4, need, s.sbuf, s.res);
  const int dg = s.res[0];
  prefix |= (uint32_t)dg << shift;
  mask |= dmask << shift;
  need -= s.res[1];
  return dg;
}
__device__ __forceinline__ void topk_clear_hist(int* hw) {      // a wave clears its own histogram
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < kTopkBins / 256; ++c) *reinterpret_cast<int4*>(hw + 4 * (lane + 64 * c)) = int4{0, 0, 0, 0};
}
// One workgroup takes every digit and the output from row t's full keys: wave
// w reads a contiguous range of the row in tiles of 256 (a float4 per lane);
// its histograms also give how many of its rows lie above and at the
// threshold, so the waves' output places follow from eight counts.
__device__ __forceinline__ void topk_full_row(const float* sc, int n, int K, int32_t* out, const TopkLds& s) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int* hw = s.hist + w * kTopkBins;
  uint32_t prefix = 0u, mask = 0u;
  int need = K;
  const int segw = (n + kWaves * 256 - 1) / (kWaves * 256) * 256;
  const int wb = min(n, w * segw), we = min(n, wb + segw);
  int above = 0, at = 0;                          // this wave's rows above / at the threshold
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    __syncthreads();                              // every wave is done with the histograms
    topk_clear_hist(hw);
    const uint32_t pf = prefix, mk = mask;
    for_tiles(sc, wb, we, n, [&](int b, const uint32_t (&u)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (b + 4 * lane + e < we && (u[e] & mk) == pf) atomicAdd(&hw[(u[e] >> shift) & dmask], 1);
    });
    __syncthreads();
    const int dg = topk_next_digit(s, shift, dmask, prefix, mask, need);
    int a = 0;                                    // this wave's rows in its bins above the digit
#pragma unroll
    for (int c = 0; c < kTopkBins / 64; ++c) a += lane + 64 * c > dg ? hw[lane + 64 * c] : 0;
    above += wave_sum_int(a);
    if (pass == 2) at = hw[dg];
  }
  if (lane == 0) {
    s.wc[2 * w] = above;
    s.wc[2 * w + 1] = at;
  }
  __syncthreads();
  int G = 0, E = 0;                               // rows above / at the threshold before the wave's range
  for (int v = 0; v < w; ++v) {
    G += s.wc[2 * v];
    E += s.wc[2 * v + 1];
  }
  for_tiles(sc, wb, we, n, [&](int b, const uint32_t (&u)[4]) {
    int rows[4];
    bool ok[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rows[e] = b + 4 * lane + e;
      ok[e] = rows[e] < we;
    }
    topk_write<4>(out, rows, u, ok, prefix, need, G, E);
  });
}
// The parts' work; returns true when this workgroup (a row's first part) must
// take the row from its full keys instead.
__device__ __forceinline__ bool topk_parts(const LayerParams& p, int L, const TopkLds& s) {
  const int T = p.T, K = p.itopk, P = max(1, (int)gridDim.x / T);
  const int t = blockIdx.x / P, part = blockIdx.x - t * P;
  if (t >= T) return false;
  const int n = L + t + 1;
  int32_t* out = p.isel + (long long)t * K;
  if (n <= K) {
    if (part == 0)
      for (int i = threadIdx.x; i < n; i += kThreads) out[i] = i;
    return false;
  }
  const float* sc = p.iscore + (long long)t * p.imax;
  const int S = max(kTopkPart, ((n + P - 1) / P + 511) / 512 * 512), parts = (n + S - 1) / S;
  if (parts > kThreads || S / 512 > kThreads) return part == 0;   // (beyond the parts' LDS tables)
  if (part >= parts) return false;
  const uint16_t* k16 = p.ik16 + (long long)t * p.imax;
  uint32_t* ghist = p.ihist + (long long)t * kTopkBins;
  uint32_t* done1 = p.ictr + t * kIdxCtrStride;                // parts that added their bins
  uint32_t* done2 = done1 + kIdxCtrStride / 2;                  // parts that wrote their pairs
  uint64_t* pairs = reinterpret_cast<uint64_t*>(p.icand) + (long long)t * p.imax;
  uint32_t* pcnt = p.icnt + t * kThreads;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int kb = part * S, ke = min(n, kb + S), ntile = (ke - kb + 511) / 512;
  // ---- this part's first-digit histogram, added into the row's
  int* lh = s.hist;                               // one histogram for the workgroup
  for (int i = threadIdx.x; i < kTopkBins / 4; i += kThreads) reinterpret_cast<int4*>(lh)[i] = int4{0, 0, 0, 0};
  __syncthreads();
  uint32_t u0k[8];                                // the keys of the wave's first tile, kept for the later passes
  for (int tile = w; tile < ntile; tile += kWaves) {
    const int b = kb + tile * 512 + 8 * lane;
    uint32_t u[8];
    keys16(k16, b, n, u);
    if (tile == w)
#pragma unroll
      for (int e = 0; e < 8; ++e) u0k[e] = u[e];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (b + e < ke) atomicAdd(&lh[u[e] >> 5], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kTopkBins; i += kThreads) {
    const int v = lh[i];
    if (v) __hip_atomic_fetch_add(ghist + i, (uint32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wg_release_begin();                             // the additions are performed
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(done1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.res[3] = wait_count(p, done1, (uint32_t)parts);
  }
  __syncthreads();
  if (!s.res[3]) return false;
  // ---- the first digit (top 11 bits) from the row's histogram
  int h4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    h4[q] = (int)__hip_atomic_load(ghist + kTopkBins - 1 - 4 * threadIdx.x - q, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  digit_of(h4, K, s.sbuf, s.res);
  const int d0 = s.res[0], cum0 = s.res[1], nlist = s.res[1] + s.res[2];
  const uint32_t lo = (uint32_t)d0 << 5;
  // ---- this part's rows at or above the digit's bin, as (full key, row)
  // pairs in ascending row order from the part's first row's place
  int* tc = s.poff;                               // [ntile]: a tile's pairs, then its first place
  for (int tile = w; tile < ntile; tile += kWaves) {
    const int b = kb + tile * 512 + 8 * lane;
    uint32_t u[8];
    if (tile == w) {
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = u0k[e];
    } else {
      keys16(k16, b, n, u);
    }
    int c = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) c += __popcll(__ballot(b + e < ke && u[e] >= lo));
    if (lane == 0) tc[tile] = c;
  }
  __syncthreads();
  const int tcv = (int)threadIdx.x < ntile ? tc[threadIdx.x] : 0;
  const int tinc = wg_scan_incl(tcv, s.sbuf);
  if ((int)threadIdx.x < ntile) tc[threadIdx.x] = tinc - tcv;
  if (threadIdx.x == kThreads - 1) s.res[3] = tinc;             // the part's pairs
  __syncthreads();
  for (int tile = w; tile < ntile; tile += kWaves) {
    const int b = kb + tile * 512 + 8 * lane;
    uint32_t u[8];
    if (tile == w) {
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = u0k[e];
    } else {
      keys16(k16, b, n, u);
    }
    bool sel[8];
    int pb = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sel[e] = b + e < ke && u[e] >= lo;
      pb += __popcll(__ballot(sel[e]) & lt);
    }
    // the selected rows' full 32-bit keys (their scores, read only for them)
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = sel[e] ? ldg(sc + b + e) : 0.f;
    int pos = kb + tc[tile] + pb;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (sel[e]) {
        __hip_atomic_store(pairs + pos, ((uint64_t)order_key(f[e]) << 32) | (uint32_t)(b + e), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        ++pos;
      }
  }
  if (threadIdx.x == 0) __hip_atomic_store(pcnt + part, (uint32_t)s.res[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wg_release_begin();                             // the pairs are written
  if (threadIdx.x == 0) __hip_atomic_fetch_add(done2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (part != 0) return false;
  // ---- the row's first part: every part's pairs, in order, into the LDS list
  if (threadIdx.x == 0) s.res[3] = wait_count(p, done2, (uint32_t)parts);
  __syncthreads();
  if (!s.res[3]) return false;
  bool fits = nlist <= kTopkList;
  if (fits) {
    const int pc = (int)threadIdx.x < parts
                       ? (int)__hip_atomic_load(pcnt + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0;
    const int pinc = wg_scan_incl(pc, s.sbuf);
    s.poff[threadIdx.x] = pinc - pc;
    if (threadIdx.x == kThreads - 1) s.res[3] = pinc;
    __syncthreads();
    fits = s.res[3] == nlist;                     // (always: the same keys and digit)
  }
  if (!fits) return true;
  // list place m: part q with poff[q] <= m < poff[q + 1], its pair m - poff[q]
  constexpr int kU = 8;
  for (int m0 = threadIdx.x; m0 < nlist; m0 += kThreads * kU) {
    uint64_t e[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int m = min(m0 + u * kThreads, nlist - 1);
      int a = 0, z = parts - 1;                   // the last part whose first place <= m
      while (a < z) {
        const int mid = (a + z + 1) >> 1;
        if (s.poff[mid] <= m) a = mid;
        else z = mid - 1;
      }
      e[u] = __hip_atomic_load(pairs + a * S + (m - s.poff[a]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int m = m0 + u * kThreads;
      if (m < nlist) {
        s.lrow[m] = (int)(uint32_t)e[u];
        s.lkey[m] = (uint32_t)(e[u] >> 32);
      }
    }
  }
  __syncthreads();
  uint32_t prefix = (uint32_t)d0 << 21, mask = 2047u << 21;     // the threshold's bits found so far
  int need = K - cum0;                                          // rows at the prefix still to take
  int* hw = s.hist + w * kTopkBins;
  auto list_digit = [&](int shift, uint32_t dmask) {
    topk_clear_hist(hw);
    for (int m = threadIdx.x; m < nlist; m += kThreads) {
      const uint32_t u = s.lkey[m];
      if ((u & mask) == prefix) atomicAdd(&hw[(u >> shift) & dmask], 1);
    }
    __syncthreads();
    topk_next_digit(s, shift, dmask, prefix, mask, need);
  };
  list_digit(10, 2047u);                          // bits 10..20
  list_digit(0, 1023u);                           // bits 0..9
  // ---- output: wave w writes list entries [w * segl, (w + 1) * segl)
  const int segl = (nlist + kWaves * 64 - 1) / (kWaves * 64) * 64;
  const int lb = min(nlist, w * segl), le = min(nlist, lb + segl);
  int ga = 0, ea = 0;
  for (int m = lb + lane; m < le; m += 64) {
    const uint32_t u = s.lkey[m];
    ga += u > prefix;
    ea += u == prefix;
  }
  ga = wave_sum_int(ga);
  ea = wave_sum_int(ea);
  if (lane == 0) {
    s.wc[2 * w] = ga;
    s.wc[2 * w + 1] = ea;
  }
  __syncthreads();
  int G = 0, E = 0;
  for (int v = 0; v < w; ++v) {
    G += s.wc[2 * v];
    E += s.wc[2 * v + 1];
  }
  for (int m0 = lb; m0 < le; m0 += 64) {
    const int m = m0 + lane;
    const bool ok[1] = {m < le};
    const int rows[1] = {ok[0] ? s.lrow[m] : 0};
    const uint32_t u[1] = {ok[0] ? s.lkey[m] : 0u};
    topk_write<1>(out, rows, u, ok, prefix, need, G, E);
  }
  return false;
}

__device__ __forceinline__ void phase_topk(const LayerParams& p, int L, char* smem) {
  const TopkLds s(smem);
  if (topk_parts(p, L, s)) {
    const int t = blockIdx.x / max(1, (int)gridDim.x / p.T);
    topk_full_row(p.iscore + (long long)t * p.imax, L + t + 1, p.itopk, p.isel + (long long)t * p.itopk, s);
  }
}

// ------------------------------------------------------------------ P2 attention
// Units (query tile of 16 queries q = t*nh + h, KV range).  Per wave: chunks of
// 16 keys; S^T = K Q^T on the matrix cores (keys x queries), online softmax per
// query column, Z^T += C^T P^T with C staged in the wave's LDS slice.  The 8
// waves' states are merged in LDS and the split's partial (Z, running max,
// running sum) is written out; P3 merges the splits.
template <int KF>
struct AttnTypes;
template <> struct AttnTypes<MK_FMT_BF16> {
  typedef __bf16 E;
  static constexpr int KBW = 32;   // dims per QK block
};
template <> struct AttnTypes<MK_FMT_F32> {
  typedef float E;
  static constexpr int KBW = 16;
};
// fp8 rows: codes are loaded (8 bytes per lane and block) and widened to bf16
// with the key's row scale when used, so the attention arithmetic is the bf16 one
template <> struct AttnTypes<MK_FMT_FP8_ROW> {
  typedef __bf16 E;
  static constexpr int KBW = 32;
};

constexpr float kAttSlack = 8.f;                 // softmax reference moves when exceeded by this much

// Long contexts: a unit is four query tiles and one key split (see
// phase_attention_shared).  Used when the layer allows it (the dense bf16
// cache of the 512 + 64 latent shape, with room for the partials) and a split
// of the one-tile plan would hold at least kAttShareRows keys.
constexpr int kAttShareRows = 1024;
__device__ __forceinline__ bool attn_shared(const LayerParams& p, int NQT, int Lt) {
  const int s1 = max(1, (int)gridDim.x / NQT);
  return p.att_share && (Lt + s1 - 1) / s1 >= kAttShareRows;
}
// KV splits per query tile and keys per split (the same in P2 and P3).
__device__ __forceinline__ void attn_splits(int NQT, int Lt, int& s_kv, int& SK, bool shared = false) {
  s_kv = (int)gridDim.x / (shared ? (NQT + 3) / 4 : NQT);
  if (s_kv < 1) s_kv = 1;
  const int nchunk_all = (Lt + 15) / 16;
  if (s_kv > nchunk_all) s_kv = nchunk_all;
  SK = ((Lt + s_kv - 1) / s_kv + 15) / 16 * 16;
}

// EXACT: d_latent + d_rope == KBMAX * KBW and d_latent == 16 * DBMAX, so every
// per-block bound is a compile-time constant (no guards inside the loops).
//
// One unit = (query tile of 16 rows of [q~ | q^R], a split of the keys).  The
// waves form four pairs; pair c takes key chunks (16 keys) c, c + 4, ... of the
// split, and wave 2c + h of the pair takes half h of the key dims: latent
// blocks [0, la) or [la, n_lat) (la = ceil(n_lat / 2)) plus a share of the
// RoPE blocks.  Each wave computes its half of S = Q K^T for the chunk, the two
// halves are added through LDS (both waves then hold the same scores and run
// the same online softmax), and each wave multiplies P into its own half of
// the latent accumulator Z with the value rows it already loaded (its latent
// blocks, staged in its LDS slice and read transposed).  The next chunk's key
// rows are requested before the current chunk is used.  At the end the four
// pairs' (m, l, Z) are merged in LDS.
// SP (sparse attention): query tile qt holds 16 heads of one verify row t (n_heads
// is a multiple of 16), and its keys are that row's kept cache rows (isel), of
// which there are min(idx_topk, L + t + 1); the splits cut min(idx_topk, L + T)
// positions of the kept list.
template <int KF, int KBMAX, int DBMAX, bool EXACT, bool SP = false>
__device__ __forceinline__ void phase_attention(const LayerParams& p, int L, char* smem) {
  typedef typename AttnTypes<KF>::E E;
  constexpr int KBW = AttnTypes<KF>::KBW;
  constexpr bool F8 = KF == MK_FMT_FP8_ROW;
  constexpr int KM = F8 ? MK_FMT_BF16 : KF;             // format of the arithmetic
  typedef typename std::conditional<F8, u32x2, u32x4>::type KR;   // a lane's key bits per block
  constexpr int PB = KBW / 16;                         // 16-dim value blocks per key-dim block
  constexpr int NLMAX = DBMAX / PB;                    // latent key-dim blocks, at most
  constexpr int KHMAX = EXACT ? (NLMAX + 1) / 2 + (KBMAX - NLMAX + 1) / 2 : (KBMAX + 1) / 2;
  constexpr int DBH = (NLMAX + 1) / 2 * PB;            // value blocks per half, at most
  const int T = p.T, nh = p.nh;
  const int dc = EXACT ? 16 * DBMAX : p.dc, kvw = EXACT ? KBMAX * KBW : p.kvw;
  const int NQ = T * nh, NQT = (NQ + 15) / 16, Lt = SP ? min(p.itopk, L + T) : L + T;
  const int nlat = EXACT ? NLMAX : dc / KBW, KB = EXACT ? KBMAX : kvw / KBW, nrope = KB - nlat;
  const int la = (nlat + 1) / 2, ra = nrope / 2;
  int s_kv, SK;
  attn_splits(NQT, Lt, s_kv, SK);
  const int units = NQT * s_kv;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int hf = w & 1, cg = w >> 1;
  // this wave's key-dim blocks: nl latent ones from l0, then nr RoPE ones from r0
  const int l0 = hf ? la : 0, nl = hf ? nlat - la : la;
  const int r0 = nlat + (hf ? ra : 0), nr = hf ? nrope - ra : ra;
  const int nk = nl + nr;
  const int CSH = la * KBW + 8;                        // LDS row stride of a value slice
  E* vs = reinterpret_cast<E*>(smem) + (long long)w * 16 * CSH;
  const int QS = kvw + 8;                              // LDS row stride of the query tile
  E* qs = reinterpret_cast<E*>(smem) + (long long)kWaves * 16 * CSH;
  f32x4* sx = reinterpret_cast<f32x4*>(smem + (((long long)kWaves * 16 * CSH + 16LL * QS) * sizeof(E) + 15) / 16 * 16);
  const E* qlane = qs + j * QS + g * (KBW / 4);
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(p.kv);
  const long long rb = kv_row_bytes(KF, p.kv_row);
  auto kblk = [&](int i) { return (EXACT ? i < NLMAX / 2 : i < nl) ? l0 + i : r0 + i - nl; };
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int qt = u / s_kv, s = u - qt * s_kv;
    const int qi = qt * 16 + j, qc = qi < NQ ? qi : NQ - 1;
    const int tq = qc / nh;
    const int limit = L + tq;                          // keys 0..limit are visible
    const int tt = SP ? (qt * 16) / nh : 0;            // sparse: the tile's verify row
    const int cnt = SP ? min(p.itopk, L + tt + 1) : 0; // sparse: its kept rows
    const int32_t* kept = SP ? p.isel + (long long)tt * p.itopk : nullptr;
    const int k0 = s * SK, k1 = min(Lt, k0 + SK);
    const int nch = k1 > k0 ? (k1 - k0 + 15) / 16 : 0;
    const int nit = (nch + 3) / 4;                     // chunk rounds (the same for every wave)
    // key rows of chunk c of this split, this wave's dims; chunks past the
    // split read clamped rows (their scores are masked)
    KR ka[KHMAX], kn[KHMAX];
    float ksa = 1.f, ksn = 1.f;                        // fp8 rows: the key's row scale
    auto load_chunk = [&](int c, KR (&kr)[KHMAX], float& ks) {
      const int pk = min(k0 + c * 16 + j, (SP ? cnt : Lt) - 1);
      const int key = SP ? ldg(kept + pk) : pk;
      const uint8_t* row = kvb + key * rb;
      if constexpr (F8) {
#pragma unroll
        for (int i = 0; i < KHMAX; ++i)
          if (EXACT || i < nk) kr[i] = ldg(reinterpret_cast<const u32x2*>(row + kblk(i) * KBW + g * 8));
        ks = ldg(reinterpret_cast<const float*>(row + (SP ? p.kv_row : kvw)));   // after all codes
      } else {
        const E* er = reinterpret_cast<const E*>(row) + g * (KBW / 4);
#pragma unroll
        for (int i = 0; i < KHMAX; ++i)
          if (EXACT || i < nk) kr[i] = ld16(er + kblk(i) * KBW);
      }
    };
    // query tile -> LDS (shared by the 8 waves): qs[16][kvw + 8] = [q~ | rotated q^R];
    // its loads go out first, then this wave's first key rows, so that
    // storing the query waits for the query only
    __syncthreads();
    {
      const int n4 = kvw / 4;
      f32x4 qv[5];
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        const int i = min((int)threadIdx.x + c * kThreads, 16 * n4 - 1);
        const int jq = i / n4, dd = (i - jq * n4) * 4;
        const int qq = min(qt * 16 + jq, NQ - 1);
        const float* src = dd < dc ? p.qabs + (long long)qq * dc + dd : p.qrope + (long long)qq * p.dr + (dd - dc);
        qv[c] = ldg(reinterpret_cast<const f32x4*>(src));
      }
      __builtin_amdgcn_sched_barrier(0);     // keep every query load ahead of the key rows
      load_chunk(cg, ka, ksa);
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        const int i = threadIdx.x + c * kThreads;
        if (i < 16 * n4) {
          const int jq = i / n4, dd = (i - jq * n4) * 4;
          store4<E>(qs + jq * QS + dd, qv[c]);
        }
      }
    }
    __syncthreads();
    trace_x(p, 0);
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[DBH];
#pragma unroll
    for (int db = 0; db < DBH; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < nit; ++it) {
      const int c = cg + 4 * it;
      const int kbase = k0 + c * 16;
      load_chunk(c + 4, kn, ksn);
      // this wave's half of S^T = K Q^T; its latent blocks also go to its
      // value slice (row-major) for the value product
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KHMAX; ++i) {
        if (EXACT || i < nk) {
          u32x4 kb;
          if constexpr (F8) kb = fp8x8_scaled_bf16(ka[i][0], ka[i][1], ksa);
          else kb = ka[i];
          st = tile_mma_reg<KM>(kb, *reinterpret_cast<const typename BReg<KM>::T*>(qlane + kblk(i) * KBW), st);
          if (EXACT ? i < NLMAX / 2 : i < nl)
            *reinterpret_cast<u32x4*>(vs + j * CSH + i * KBW + g * (KBW / 4)) = kb;
        }
      }
      // the two halves added (the same order of addition in both waves)
      f32x4* sxb = sx + (it & 1) * (kWaves * 64);
      sxb[w * 64 + lane] = st;
      __syncthreads();
      {
        const f32x4 o = sxb[(w ^ 1) * 64 + lane];
        st = hf ? o + st : st + o;
      }
      // scores: lane (g, j) elem e = S[query j][key kbase + 4g + e]
      float sc[4];
      float cmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = kbase + 4 * g + e;
        sc[e] = ((SP ? kk < cnt : kk <= limit) && kk < k1) ? st[e] * p.scale : -INFINITY;
        cmax = fmaxf(cmax, sc[e]);
      }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      // The reference maximum m_run moves only when a chunk's maximum exceeds
      // it by more than kAttSlack: any reference gives the same softmax, and
      // exponentials up to e^kAttSlack are safe in fp32 sums, so the running
      // sum and the accumulator are rescaled on few chunks (the decision is the
      // same in every lane of the wave: both waves of a pair hold the same scores).
      const int DBh = EXACT ? DBH : nl * PB;
      const bool move = cmax > m_run + kAttSlack;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float m_new = move ? cmax : m_run;
        const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DBH; ++db)
          if (db < DBh) acc[db] *= alpha;
        m_run = m_new;
      }
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[e] = m_run == -INFINITY ? 0.f : __expf(sc[e] - m_run);
      float ps = pe[0] + pe[1] + pe[2] + pe[3];
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run += ps;
      if (KM == MK_FMT_BF16) {
        bf16x4 pb;
#pragma unroll
        for (int e = 0; e < 4; ++e) pb[e] = (__bf16)pe[e];
        // A operand (dims x keys) read transposed from the row-major slice:
        // lane (g, 4e + q) points at key 4g + e, dims 16 db + 4q .. + 3
        const __bf16* tb = reinterpret_cast<const __bf16*>(vs) + (4 * g + (j >> 2)) * CSH + 4 * (j & 3);
#pragma unroll
        for (int d0 = 0; d0 < DBH; d0 += 8) {
          bf16x4 av[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (d0 + i < DBh) av[i] = lds_read_tr16(tb + (d0 + i) * 16);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (d0 + i < DBh) acc[d0 + i] = mma_bf16_k16(av[i], pb, acc[d0 + i]);
        }
      } else {
#pragma unroll
        for (int db = 0; db < DBH; ++db) {
          if (db < DBh) {
            f32x4 a = acc[db];
#pragma unroll
            for (int e = 0; e < 4; ++e) a = mma_f32_k4((float)vs[(4 * g + e) * CSH + db * 16 + j], pe[e], a);
            acc[db] = a;
          }
        }
      }
      // the slice is rewritten by the next round of this wave only
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < KHMAX; ++i) ka[i] = kn[i];
      ksa = ksn;
    }
    // merge the four pairs' (m, l, Z): every wave rescales its half of Z to the
    // common maximum and stores it; wave w then adds latent blocks w, w + 8, ...
    // over the pairs in a fixed order and writes them out.
    __syncthreads();
    trace_x(p, 1);
    // Partial state layout in LDS: block b of the latent of pair c holds, per
    // lane, the 4 values of acc (MFMA result layout: lane (g, j) has dims
    // 16 b + 4 g + e of query j), so every access is one 16-byte vector.  In
    // global memory the partial is query-major ([16 queries][d_latent]), so
    // that the merge reads one query's latent as contiguous memory.
    const int DB = dc / 16;
    f32x4* mb = reinterpret_cast<f32x4*>(smem);                 // [4][DB][64]
    float* ml = reinterpret_cast<float*>(smem) + 4 * DB * 64 * 4;   // [8][64][2]
    ml[(w * 64 + lane) * 2] = m_run;
    ml[(w * 64 + lane) * 2 + 1] = l_run;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) M = fmaxf(M, ml[(2 * cc * 64 + lane) * 2]);
    const float sw = M == -INFINITY ? 0.f : __expf(m_run - M);
    {
      const int DBh = EXACT ? DBH : nl * PB;
      f32x4* zb = mb + ((long long)cg * DB + l0 * PB) * 64;
#pragma unroll
      for (int db = 0; db < DBH; ++db)
        if (db < DBh) zb[db * 64 + lane] = acc[db] * sw;
    }
    __syncthreads();
    {
      f32x4* zp = reinterpret_cast<f32x4*>(p.att_part + (long long)u * 16 * dc);
      constexpr int NBW = (DBMAX + kWaves - 1) / kWaves;
      f32x4 t[NBW][4];
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int db = w + kWaves * i;
        if (db < DB) {
#pragma unroll
          for (int b = 0; b < 4; ++b) t[i][b] = mb[((long long)b * DB + db) * 64 + lane];
        }
      }
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int db = w + kWaves * i;
        if (db < DB) zp[j * (dc / 4) + db * 4 + g] = (t[i][0] + t[i][1]) + (t[i][2] + t[i][3]);
      }
    }
    if (w == 0 && g == 0) {
      float Ls = 0.f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float mw = ml[(2 * cc * 64 + lane) * 2];
        Ls += mw == -INFINITY ? 0.f : ml[(2 * cc * 64 + lane) * 2 + 1] * __expf(mw - M);
      }
      p.att_ml[((long long)u * 16 + j) * 2] = M;
      p.att_ml[((long long)u * 16 + j) * 2 + 1] = Ls;
    }
    trace_x(p, 2);
  }
}

// P2 for long contexts (dense, bf16 cache, d_latent 512 + d_rope 64): one unit
// = (a group of four query tiles, one key split).  Pair c of the 8 waves takes
// tile 4 * group + c, and every pair works on the same key chunk, which the
// workgroup stages in LDS once: each chunk's 16 rows are loaded by all threads
// kStageAhead chunks ahead into registers and stored into a ring of three LDS
// buffers one round before use, so a key row is read from memory once per four
// query tiles instead of once per tile.  As in phase_attention, the two waves
// of a pair take half of the key dims each (their query fragments held in
// LDS for the whole unit), add their halves of S through LDS, run the
// same online softmax and multiply P into their half of Z, reading the value
// rows transposed from the staged chunk.  A pair's partial (Z, max, sum) is its
// tile's partial for this split; no merge across pairs is needed.
constexpr int kStageAhead = 2;
__device__ __forceinline__ void phase_attention_shared(const LayerParams& p, int L, char* smem) {
  constexpr int KBW = 32, NLAT = 16, DC = 512, KVW = 576, NKB = 9, DBH = 16;
  constexpr int KS = KVW + 8;                          // LDS row stride (bf16) of queries and keys
  constexpr int PIECES = 16 * KVW / 8;                 // 16-byte pieces of one chunk (1152)
  constexpr int PT = (PIECES + kThreads - 1) / kThreads;   // per thread (3)
  const int T = p.T, nh = p.nh;
  const int NQ = T * nh, NQT = (NQ + 15) / 16, NG = (NQT + 3) / 4, Lt = L + T;
  int s_kv, SK;
  attn_splits(NQT, Lt, s_kv, SK, true);
  const int units = NG * s_kv;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int hf = w & 1, cg = w >> 1;
  __bf16* qs = reinterpret_cast<__bf16*>(smem);                        // [4 tiles][16][KS]
  __bf16* ring = qs + 4 * 16 * KS;                                     // [3][16][KS]
  f32x4* sx = reinterpret_cast<f32x4*>(ring + 3 * 16 * KS);            // [2][8 waves][64]
  const __bf16* kvb = reinterpret_cast<const __bf16*>(p.kv);
  // this wave's key blocks: latent blocks 8 hf .. 8 hf + 7, then RoPE block 16 + hf
  auto kblk = [&](int i) { return i < 8 ? 8 * hf + i : NLAT + hf; };
#pragma unroll 1
  for (int v = blockIdx.x; v < units; v += gridDim.x) {
    const int grp = v / s_kv, s = v - grp * s_kv;
    const int qt = grp * 4 + cg;                       // this pair's tile (qt >= NQT: the pair only keeps step)
    const bool live = qt < NQT;
    const int qc = min(min(qt, NQT - 1) * 16 + j, NQ - 1);
    const int limit = L + qc / nh;                     // keys 0..limit are visible
    const int k0 = s * SK, k1 = min(Lt, k0 + SK);
    const int nch = k1 > k0 ? (k1 - k0 + 15) / 16 : 0;
    // the 16-byte pieces this thread loads of chunk c (rows past the split clamped)
    auto load_chunk = [&](int c, u32x4 (&r)[PT]) {
#pragma unroll
      for (int q = 0; q < PT; ++q) {
        const int pc = min((int)threadIdx.x + q * kThreads, PIECES - 1), row = pc / (KVW / 8);
        const int key = min(k0 + c * 16 + row, Lt - 1);
        r[q] = ld16(kvb + (long long)key * KVW + (pc - row * (KVW / 8)) * 8);
      }
    };
    auto store_chunk = [&](int slot, const u32x4 (&r)[PT]) {
#pragma unroll
      for (int q = 0; q < PT; ++q) {
        const int pc = (int)threadIdx.x + q * kThreads, row = pc / (KVW / 8);
        if (pc < PIECES)
          *reinterpret_cast<u32x4*>(ring + (slot * 16 + row) * KS + (pc - row * (KVW / 8)) * 8) = r[q];
      }
    };
    __syncthreads();                                   // the previous unit is done with the LDS
    // the four tiles' queries [q~ | rotated q^R] -> LDS (bf16), loads first,
    // then chunk 0 and the next kStageAhead chunks
    {
      // two rounds of 9 float4s per thread (4 tiles x 16 queries x 144 float4s)
      constexpr int N4 = KVW / 4, NV = 9, NQV = 4 * 16 * N4;
      u32x4 c0[PT];
      load_chunk(0, c0);
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        f32x4 qv[NV];
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          const int i = min((int)threadIdx.x + (half * NV + c) * kThreads, NQV - 1);
          const int jq = i / N4, dd = (i - jq * N4) * 4;
          const int qq = min(grp * 64 + jq, NQ - 1);
          const float* src = dd < DC ? p.qabs + (long long)qq * DC + dd : p.qrope + (long long)qq * p.dr + (dd - DC);
          qv[c] = ldg(reinterpret_cast<const f32x4*>(src));
        }
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          const int i = threadIdx.x + (half * NV + c) * kThreads;
          if (i < NQV) {
            const int jq = i / N4, dd = (i - jq * N4) * 4;
            store4<__bf16>(qs + jq * KS + dd, qv[c]);
          }
        }
      }
      store_chunk(0, c0);
    }
    u32x4 pre[kStageAhead][PT];                        // chunks c + 1 .. c + kStageAhead
#pragma unroll
    for (int a = 0; a < kStageAhead; ++a) load_chunk(1 + a, pre[a]);
    __syncthreads();
    // this wave's query fragments (B operand): query j, dims kblk(i) * 32 + 8 g .. + 7
    const __bf16* qlane = qs + (cg * 16 + j) * KS + g * 8;
    trace_x(p, 0);
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[DBH];
#pragma unroll
    for (int db = 0; db < DBH; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
      const int kbase = k0 + c * 16;
      const __bf16* kc = ring + (c % 3) * 16 * KS;
      // this wave's half of S^T = K Q^T (keys from the staged chunk)
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NKB; ++i)
        st = mma_bf16_k32(*reinterpret_cast<const bf16x8*>(kc + j * KS + kblk(i) * KBW + g * 8),
                          *reinterpret_cast<const bf16x8*>(qlane + kblk(i) * KBW), st);
      f32x4* sxb = sx + (c & 1) * (kWaves * 64);
      sxb[w * 64 + lane] = st;
      // the next chunk goes to its ring slot (its readers are two rounds back)
      // and the chunk kStageAhead past it is requested
      if (c + 1 < nch) store_chunk((c + 1) % 3, pre[0]);
#pragma unroll
      for (int a = 0; a + 1 < kStageAhead; ++a)
#pragma unroll
        for (int q = 0; q < PT; ++q) pre[a][q] = pre[a + 1][q];
      load_chunk(c + 1 + kStageAhead, pre[kStageAhead - 1]);
      __syncthreads();
      {
        const f32x4 o = sxb[(w ^ 1) * 64 + lane];
        st = hf ? o + st : st + o;
      }
      float sc[4];
      float cmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = kbase + 4 * g + e;
        sc[e] = (kk <= limit && kk < k1) ? st[e] * p.scale : -INFINITY;
        cmax = fmaxf(cmax, sc[e]);
      }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const bool move = cmax > m_run + kAttSlack;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        const float m_new = move ? cmax : m_run;
        const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DBH; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[e] = m_run == -INFINITY ? 0.f : __expf(sc[e] - m_run);
      float ps = pe[0] + pe[1] + pe[2] + pe[3];
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l_run += ps;
      bf16x4 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[e] = (__bf16)pe[e];
      // A operand (dims x keys) read transposed from the staged rows: lane
      // (g, 4e + q) points at key 4g + e, dims 256 hf + 16 db + 4q .. + 3
      const __bf16* tb = kc + (4 * g + (j >> 2)) * KS + 256 * hf + 4 * (j & 3);
#pragma unroll
      for (int d0 = 0; d0 < DBH; d0 += 8) {
        bf16x4 av[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) av[i] = lds_read_tr16(tb + (d0 + i) * 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[d0 + i] = mma_bf16_k16(av[i], pb, acc[d0 + i]);
      }
    }
    trace_x(p, 1);
    if (live) {
      // the pair's partial: wave hf writes latent dims 256 hf .. 256 hf + 255 of
      // its 16 queries (query-major), wave 0 of the pair the (max, sum)
      const int u = qt * s_kv + s;
      f32x4* zp = reinterpret_cast<f32x4*>(p.att_part + (long long)u * 16 * DC);
#pragma unroll
      for (int db = 0; db < DBH; ++db) zp[j * (DC / 4) + (16 * hf + db) * 4 + g] = acc[db];
      if (hf == 0 && g == 0) {
        p.att_ml[((long long)u * 16 + j) * 2] = m_run;
        p.att_ml[((long long)u * 16 + j) * 2 + 1] = l_run;
      }
    }
    trace_x(p, 2);
  }
}

// ------------------------------------------------------------------ P3  split merge and o = W_UV z
// One unit = (head h, a group of up to kMergeRows verify rows).  Wave w
// requests row tile w of W_UV^(h) first; then two threads per latent item
// (row ti, float4 r4 of the latent) each load the (max, sum) and the partial
// of half of the KV splits in one round trip and merge them with their own
// running maximum; the halves are combined through LDS into
// z = sum_s exp(m_s - M) Z_s / sum_s exp(m_s - M) l_s, kept in LDS as the
// matrix-core operand (and written to the z buffer); finally wave w multiplies
// its row tile.  Only the queries of its own unit are merged, so no partial is
// read twice and no grid barrier separates the merge from the up-projection.
constexpr int kMergeRows = 2;
constexpr int kMergeSB = 12;                      // splits per thread per batch
constexpr int kMergeXOff = 8192;                  // LDS: half-merge exchange after the z operand
template <int AF, bool SP = false>
__device__ __forceinline__ void phase_merge_uv(const LayerParams& p, int L, char* smem, bool shared = false) {
  typedef typename Act<AF>::T A;
  constexpr int TK = tile_k(AF);
  constexpr int KTMAX = 16;                       // d_latent / tile_k <= 16 for every supported shape
  const int T = p.T, nh = p.nh, dc = p.dc, dh = p.dh;
  const int NQ = T * nh, NQT = (NQ + 15) / 16;
  int s_kv, SK;
  attn_splits(NQT, SP ? min(p.itopk, L + T) : L + T, s_kv, SK, shared);
  const int TG = (T + kMergeRows - 1) / kMergeRows;
  const int U = nh * TG, XS = dc + kXPad, RT = dh / 16, KT = dc / TK, D4 = dc / 4;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  A* zs = reinterpret_cast<A*>(smem);                                  // [kMergeRows][XS]
  float* xch = reinterpret_cast<float*>(smem + kMergeXOff);            // [256 items][8]: M, L, Z
  const f32x4* part = reinterpret_cast<const f32x4*>(p.att_part);
  const f32x2* mlp = reinterpret_cast<const f32x2*>(p.att_ml);
  for (int u = blockIdx.x; u < U; u += gridDim.x) {
    const int h = u / TG, tg = u - h * TG;
    const int t0 = tg * kMergeRows, nt = min(kMergeRows, T - t0);
    // (1) this wave's W_UV row tile (waves past the last row tile load it again)
    u32x4 wt[KTMAX];
    {
      const uint8_t* tb = p.wuv + ((long long)(h * RT + min(w, RT - 1)) * KT) * 1024 + lane * 16;
#pragma unroll
      for (int kt = 0; kt < KTMAX; ++kt) wt[kt] = ld_stream16(tb + (long long)min(kt, KT - 1) * 1024);
    }
    // (2) half merges: item it = (ti, r4), half hf takes splits hf, hf + 2, ...
    const int it = min((int)threadIdx.x & 255, nt * D4 - 1), hf = threadIdx.x >> 8;
    const int ti = it / D4, r4 = it - ti * D4;
    const int q = (t0 + ti) * nh + h, qt = q >> 4, jq = q & 15;
    const f32x4* zp = part + (long long)qt * s_kv * 4 * dc + jq * D4 + r4;
    const f32x2* mp = mlp + (long long)qt * s_kv * 16 + jq;
    float Mh = -INFINITY, Lh = 0.f;
    f32x4 Zh = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = hf; s0 < s_kv; s0 += 2 * kMergeSB) {
      f32x2 ml[kMergeSB];
      f32x4 zz[kMergeSB];
#pragma unroll
      for (int b = 0; b < kMergeSB; ++b) {
        const int sp = min(s0 + 2 * b, s_kv - 1);
        ml[b] = ldg(mp + (long long)sp * 16);
        zz[b] = ldg(zp + (long long)sp * 4 * dc);
      }
      float Mb = Mh;
#pragma unroll
      for (int b = 0; b < kMergeSB; ++b)
        if (s0 + 2 * b < s_kv) Mb = fmaxf(Mb, ml[b][0]);
      if (Mb != -INFINITY) {
        const float sc = Mh == -INFINITY ? 0.f : __expf(Mh - Mb);
        Lh *= sc;
        Zh *= sc;
#pragma unroll
        for (int b = 0; b < kMergeSB; ++b) {
          if (s0 + 2 * b < s_kv && ml[b][0] != -INFINITY) {
            const float e = __expf(ml[b][0] - Mb);
            Lh += e * ml[b][1];
            Zh += zz[b] * e;
          }
        }
        Mh = Mb;
      }
    }
    __syncthreads();                              // LDS reuse across units
    if (hf == 1) {
      float* x = xch + (threadIdx.x & 255) * 8;
      x[0] = Mh;
      x[1] = Lh;
      *reinterpret_cast<f32x4*>(x + 4) = Zh;
    }
    __syncthreads();
    if (hf == 0 && (int)threadIdx.x < nt * D4) {
      const float* x = xch + threadIdx.x * 8;
      const float M1 = x[0], L1 = x[1];
      const f32x4 Z1 = *reinterpret_cast<const f32x4*>(x + 4);
      const float M = fmaxf(Mh, M1);
      const float a0 = Mh == -INFINITY ? 0.f : __expf(Mh - M), a1 = M1 == -INFINITY ? 0.f : __expf(M1 - M);
      const f32x4 zv = (Zh * a0 + Z1 * a1) / (a0 * Lh + a1 * L1);
      store4<A>(zs + ti * XS + 4 * r4, zv);
      *reinterpret_cast<f32x4*>(p.z + (long long)q * dc + 4 * r4) = zv;
    }
    __syncthreads();
    // (3) o rows of head h for the group: wave w multiplies row tile w
    if (w < RT) {
      const int jj = j < nt ? j : nt - 1;
      const A* bp = zs + jj * XS + g * (TK / 4);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KTMAX; ++kt)
        if (kt < KT) acc = tile_mma<AF>(wt[kt], bp + kt * TK, acc);
      if (j < nt) {
        A* o = reinterpret_cast<A*>(p.o);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[(long long)(t0 + j) * nh * dh + h * dh + w * 16 + 4 * g + e] = to_act<A>(acc[e]);
      }
    }
  }
}

// ------------------------------------------------------------------ P4  H' = H + W_O o
template <int AF>
__device__ __forceinline__ void phase_wo(const LayerParams& p, char* smem) {
  typedef typename Act<AF>::T A;
  constexpr int TK = tile_k(AF);
  const int T = p.T, K = p.nh * p.dh, XS = K + kXPad;
  LdsPlan lp(p, sizeof(A));
  A* xs = reinterpret_cast<A*>(smem);
  float* red = reinterpret_cast<float*>(smem + lp.xb);
  const int KT = K / TK, U = p.d / 16;
  int u0, u1;
  split_range(U, gridDim.x, blockIdx.x, u0, u1);
  if (u1 <= u0) return;
  const A* bl = b_lane<A>(xs, XS, T, TK);
  struct Src {
    const uint8_t* wo; int KT; const A* bl;
    __device__ const uint8_t* base(int u) const { return wo + (long long)u * KT * 1024; }
    __device__ const A* bbase(int) const { return bl; }
    __device__ const float* sbase(int) const { return nullptr; }
    __device__ const float* sbase2(int) const { return nullptr; }
  } src{p.wo, KT, bl};
  const float* H = p.H;
  float* hp = p.hp;
  const int d = p.d;
  auto epi = [=](int u, int row, int col, float v, float) {
    const long long i = (long long)col * d + u * 16 + row;
    hp[i] = ldg(H + i) + v;
  };
  RowCopier<A> rc;
  rc.issue(reinterpret_cast<const A*>(p.o), T, K);
  Chunk<AF, false, 16> ck;
  const bool pr = wg_primable(KT, false);
  stream_prime<AF, false, true, 16, kPrimeTiles>(ck, u0, u1, KT, src, p.dummy, pr);
  rc.finish(T, K, xs, XS);
  trace_x(p, 6);
  stream_units_wg_primed<AF, false, false, kPrimeTiles>(u0, u1, KT, T, src, epi, red, p.dummy, ck, pr);
}

// ------------------------------------------------------------------ routing
struct RouteLds {
  float* lg;       // [T][E]
  int* sel;        // [T][topk]
  float* gate;     // [T][topk]
  int* slot_of;    // [T][topk]
  int* slots;      // [slots]
  int* flags;      // [E]
  int* nslots;     // [1]
  const uint8_t** blk;   // [slots] packed expert block of each slot
};
__device__ __forceinline__ RouteLds route_lds(const LayerParams& p, char* smem, int xb) {
  char* b = smem + xb + 32768;
  RouteLds r;
  r.lg = reinterpret_cast<float*>(b);
  b += (size_t)kMaxT * p.E * 4;
  r.sel = reinterpret_cast<int*>(b);
  b += kMaxT * kMaxTopK * 4;
  r.gate = reinterpret_cast<float*>(b);
  b += kMaxT * kMaxTopK * 4;
  r.slot_of = reinterpret_cast<int*>(b);
  b += kMaxT * kMaxTopK * 4;
  r.slots = reinterpret_cast<int*>(b);
  b += (kMaxT * kMaxTopK + 8) * 4;
  r.flags = reinterpret_cast<int*>(b);
  b += (size_t)p.E * 4;
  r.nslots = reinterpret_cast<int*>(b);
  b += 16;
  r.blk = reinterpret_cast<const uint8_t**>(b);
  return r;
}

// Orderable key of a float: a > b  <=>  fkey(a) > fkey(b) (for non-NaN values).
__device__ __forceinline__ uint32_t fkey(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Top-k by logit (ties to the lower index) and gates = selected softmax
// probabilities renormalised (the normaliser over all experts cancels, so the
// gates are exp(l - m) / sum over the selection of exp(l' - m), m the largest
// selected logit).  Wave t < T handles token t: lane u < E/16 holds the
// candidates its router unit kept (the top min(k, 16) of 16 experts, which
// together contain the overall top k), in descending order, and k rounds each
// take the largest head among the lanes (the lowest lane on ties: lower units
// hold lower experts) and advance that lane's list.  The selection is written
// in descending order of logit.
template <int K8M>
__device__ __forceinline__ void route_cands(const LayerParams& p, const RouteLds& r) {
  const int K = p.topk, K8 = min(K, 16), RT = p.E / 16;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* cv = p.route_cand + ((long long)w * RT + min(lane, RT - 1)) * 16;
  const int* ci = reinterpret_cast<const int*>(p.route_cand) + ((long long)(p.T + w) * RT + min(lane, RT - 1)) * 16;
  float lv[K8M];
  int id[K8M];
  uint32_t key[K8M];
#pragma unroll
  for (int i = 0; i < K8M; ++i) {
    lv[i] = ldg(cv + min(i, K8 - 1));
    id[i] = ldg(ci + min(i, K8 - 1));
  }
#pragma unroll
  for (int i = 0; i < K8M; ++i) key[i] = lane < RT && i < K8 ? fkey(lv[i]) : 0u;   // 0: below every logit
  trace_x(p, 12);
  float m0 = 0.f, ps = 0.f, myv = 0.f;
  for (int k = 0; k < K; ++k) {
    const uint32_t hk = key[0];
    uint32_t mx = hk;
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x124, 0xF, 0xF, false));  // row_ror:4
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x128, 0xF, 0xF, false));  // row_ror:8
    // every lane of a 16-lane row now holds the row's maximum: the four rows
    // are combined through lane reads (scalar, no LDS round trip), and the
    // winner's logit and expert are read from its lane the same way
    mx = max(max((uint32_t)__builtin_amdgcn_readlane((int)mx, 0), (uint32_t)__builtin_amdgcn_readlane((int)mx, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)mx, 32), (uint32_t)__builtin_amdgcn_readlane((int)mx, 48)));
    const int wl = __ffsll((long long)__ballot(hk == mx)) - 1;
    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv[0]), wl));
    const int e = __builtin_amdgcn_readlane(id[0], wl);
    if (k == 0) m0 = v;
    const float ex = __expf(v - m0);
    ps += ex;
    if (lane == k) myv = ex;
    if (lane == 0) r.sel[w * kMaxTopK + k] = e;
    // the winning lane's next candidate moves up
    const bool win = lane == wl;
#pragma unroll
    for (int i = 0; i < K8M - 1; ++i) {
      key[i] = win ? key[i + 1] : key[i];
      lv[i] = win ? lv[i + 1] : lv[i];
      id[i] = win ? id[i + 1] : id[i];
    }
    if (win) key[K8M - 1] = 0u;
  }
  if (lane < K) r.gate[w * kMaxTopK + lane] = myv / ps;
}

// Router workgroup, after its units: for every unit (16 experts) and token,
// the biased logits (also written to the logits tap) and the top min(k, 16)
// of the 16 by (logit, lower index), stored in that order (rank r at r).
// lgl[unit - u0][t][16] holds the unit's unbiased logits.
__device__ __forceinline__ void router_candidates(const LayerParams& p, const float* lgl, int u0, int u1) {
  const int T = p.T, E = p.E, K8 = min(p.topk, 16), RT = E / 16;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int u = u0; u < u1; ++u) {
    if (w < T && lane < 16) {
      const int e = u * 16 + lane;
      const float v = lgl[((u - u0) * kMaxT + w) * 16 + lane] + (p.rbias ? ldg(p.rbias + e) : 0.f);
      p.logits[(long long)w * E + e] = v;
      const uint32_t k = fkey(v);
      int rank = 0;
      for (int j = 0; j < 16; ++j) {
        const uint32_t kj = __shfl(k, j, 16);
        rank += (kj > k || (kj == k && j < lane)) ? 1 : 0;
      }
      if (rank < K8) {
        const long long o = ((long long)w * RT + u) * 16 + rank;
        p.route_cand[o] = v;
        reinterpret_cast<int*>(p.route_cand)[(long long)T * RT * 16 + o] = e;
      }
    }
  }
}

// Every workgroup, at the start of the expert phases: the routing computed
// into its own LDS tables from the router workgroups' candidates -- the top k
// and gates per token (route_cands), then the slot list: the shared experts
// first, then the distinct selected experts in ascending order, each with its
// packed block.  Workgroup 0 also writes the selection and gates out (debug
// taps) and counts the experts streamed.
__device__ __forceinline__ void route_local(const LayerParams& p, const RouteLds& r) {
  const int T = p.T, E = p.E, K = p.topk, S0 = p.nshared;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the expert block table, requested into registers together with the token
  // waves' candidates (one round trip for both) and stored into LDS (the logit
  // area is free) afterwards
  constexpr int kEt = (kMaxExperts + 1 + kThreads - 1) / kThreads;
  const uint8_t** etab = reinterpret_cast<const uint8_t**>(r.lg);
  const uint8_t* ev[kEt];
#pragma unroll
  for (int j = 0; j < kEt; ++j) ev[j] = p.experts[min((int)threadIdx.x + j * kThreads, E + S0 - 1)];
  for (int i = threadIdx.x; i < E; i += kThreads) r.flags[i] = 0;
  if (w < T) {
    if (K <= 8) route_cands<8>(p, r);
    else route_cands<16>(p, r);
  }
#pragma unroll
  for (int j = 0; j < kEt; ++j)
    if ((int)threadIdx.x + j * kThreads < E + S0) etab[threadIdx.x + j * kThreads] = ev[j];
  __syncthreads();
  trace_x(p, 13);
  if (threadIdx.x < T * K) {
    const int t = threadIdx.x / K, k = threadIdx.x - t * K;
    r.flags[r.sel[t * kMaxTopK + k]] = 1;
  }
  __syncthreads();
  if (w == 0) {
    if (lane < S0) r.slots[lane] = E + lane;
    int base = S0;
    for (int c0 = 0; c0 < E; c0 += 64) {
      const int e = c0 + lane;
      const int f = e < E ? r.flags[e] : 0;
      const unsigned long long m = __ballot(f);
      if (f) {
        const int idx = base + __popcll(m & ((1ull << lane) - 1ull));
        r.slots[idx] = e;
        r.flags[e] = idx + 1;          // slot + 1
      }
      base += __popcll(m);
    }
    if (lane == 0) *r.nslots = base;
  }
  __syncthreads();
  const int ns = *r.nslots;
  if (threadIdx.x < T * K) {
    const int t = threadIdx.x / K, k = threadIdx.x - t * K;
    r.slot_of[t * kMaxTopK + k] = r.flags[r.sel[t * kMaxTopK + k]] - 1;
  }
  if ((int)threadIdx.x < ns) r.blk[threadIdx.x] = etab[r.slots[threadIdx.x]];
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < T * K; i += kThreads) {
      const int t = i / K, k = i - t * K;
      p.route_sel[i] = r.sel[t * kMaxTopK + k];
      p.route_gate[i] = r.gate[t * kMaxTopK + k];
    }
    if (threadIdx.x == 0) {
      p.bar->slots_sum += (unsigned long long)ns;
      p.bar->launches += 1ull;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ gate/up units
// Unit u = (slot s0 + u / RT, 16 rows rt = u % RT of d_ff): h = silu(W1 x') * W3 x'
// for all T rows, W1 and W3 tiles interleaved in the packed expert block.
// blk[i] is the packed block of slot s0 + i.
struct NoStage {
  __device__ void issue() {}
  __device__ void finish() {}
};
// Scales of a packed expert block (formats with scales), after the W1/W3 and W2 tiles.
//  fp8: fp32 [ceil(rows/128)][ceil(cols/128)] per matrix, W1 then W3 then W2;
//       a unit of 16 rows starting at row tile rt reads block row rt / 8.
//  MXFP4: E8M0 bytes in tile order, 64 per tile (byte l for lane l: the scale
//       of row l % 16 over columns (l / 16) * 32 ... of the tile), the W1 and
//       W3 tiles' 64 bytes alternating (128 per W1/W3 tile pair), then W2's.
template <int EF>
struct ExpScales {
  long long sc13, sc3, sc2;   // byte offsets: W1 (and, for fp8, W3) and W2 scales
  int n13, n2;                // fp8: blocks per block row (W1/W3, W2); MXFP4: tiles per row tile
  __device__ explicit ExpScales(const LayerParams& p) {
    sc13 = p.exp_w13_bytes + p.exp_w2_bytes;
    if constexpr (EF == MK_FMT_MXFP4) {
      n13 = p.d / 128;
      n2 = p.f / 128;
      sc3 = sc13 + 64;
      sc2 = sc13 + (long long)(p.f / 16) * n13 * 128;
    } else {
      n13 = (p.d + 127) / 128;
      n2 = (p.f + 127) / 128;
      const long long nb = (long long)((p.f + 127) / 128) * n13;
      sc3 = sc13 + nb * 4;
      sc2 = sc13 + 2 * nb * 4;
    }
  }
  // the scales of row tile rt of W1 (W3 with w3), of W2
  __device__ const float* w13(const uint8_t* blk, int rt, bool w3 = false) const {
    const uint8_t* b = blk + (w3 ? sc3 : sc13);
    if constexpr (EF == MK_FMT_MXFP4) return reinterpret_cast<const float*>(b + (long long)rt * n13 * 128);
    else return reinterpret_cast<const float*>(b) + (rt >> 3) * n13;
  }
  __device__ const float* w2(const uint8_t* blk, int rt) const {
    if constexpr (EF == MK_FMT_MXFP4) return reinterpret_cast<const float*>(blk + sc2 + (long long)rt * n2 * 64);
    else return reinterpret_cast<const float*>(blk + sc2) + (rt >> 3) * n2;
  }
};
// Shapes of the ticket-fed expert streams.  An MXFP4 tile holds twice the
// columns of an fp8 tile, so a row of d_model or d_ff has half as many tiles;
// to keep as many bytes per wave in flight, MXFP4 gate/up units go two to a
// workgroup (four waves each), and MXFP4 down-projection units are eight row
// tiles with each wave streaming one of them over all of d_ff.
constexpr int kGateDepth = 8;                      // gate/up tiles per chunk (two matrices each)
__host__ __device__ constexpr int gateup_split(int fmt) { return fmt == MK_FMT_MXFP4 ? 2 : 1; }
__host__ __device__ constexpr bool gateup_dyn_fits(int KT, int fmt) {
  return KT % (kWaves / gateup_split(fmt)) == 0 && (KT / (kWaves / gateup_split(fmt))) % kGateDepth == 0;
}
__host__ __device__ constexpr int down_rtu(int tk) { return tk >= 128 ? 8 : 4; }   // row tiles per unit
__host__ __device__ constexpr int down_kp(int tk) { return kWaves / down_rtu(tk); }  // k parts per row tile
constexpr int kDownDepth = 16;                     // down-projection tiles per chunk

// MODE 0: workgroup units [u0, u1); 1: wave units [u0, u1); 2: workgroup units
// 0 .. u1-1 handed out at run time by the ticket counters; 3: as 2, and every
// completed unit counted on its slot's completion counter.  `stage` requests
// the activation operand (issue) before the first weight chunk is requested
// and stores it (finish) before that chunk is used (workgroup mode).
template <int EF, int MODE, class Stage = NoStage>
__device__ __forceinline__ void gateup_units(const LayerParams& p, const uint8_t* const* blk, int s0, int u0, int u1,
                                             const typename Act<EF>::T* xs, float* red, Stage stage = Stage()) {
  typedef typename Act<EF>::T A;
  constexpr int TK = tile_k(EF);
  const int T = p.T, XS = p.d + kXPad;
  const int RT = p.f / 16, KT = p.d / TK;
  const A* bl = b_lane<A>(xs, XS, T, TK);
  struct Src {
    const uint8_t* const* blk; int RT, KT; const A* bl; ExpScales<EF> es;
    __device__ const uint8_t* base(int u) const {
      const int sl = u / RT, rt = u - sl * RT;
      return blk[sl] + (long long)rt * KT * 2048;
    }
    __device__ const A* bbase(int) const { return bl; }
    __device__ const float* sbase(int u) const {
      const int sl = u / RT, rt = u - sl * RT;
      return es.w13(blk[sl], rt);
    }
    __device__ const float* sbase2(int u) const {
      const int sl = u / RT, rt = u - sl * RT;
      return es.w13(blk[sl], rt, true);
    }
  };
  Src src{blk, RT, KT, bl, ExpScales<EF>(p)};
  A* hb = reinterpret_cast<A*>(p.hbuf);
  const int f = p.f;
  const float* rsc = rsc_lds();       // the staged rows are h * gamma: scale by 1/rms
  auto epi = [=](int u, int row, int col, float v, float v2) {
    v *= rsc[col];
    v2 *= rsc[col];
    const int sl = s0 + u / RT, rt = u % RT;
    const float sg = v / (1.0f + expf(-v));
    hb[((long long)sl * T + col) * f + rt * 16 + row] = to_act<A>(sg * v2);
  };
  if constexpr (MODE == 3) {
    // row pairs written with agent-scope exchanges (they pass this XCD's L2,
    // so a down projection on any XCD reads them once the slot's counter is
    // full); the reply tells the stream engine when the write has completed
    auto epi2 = [=](int u, int row, int col, float v0, float w0, float v1, float w1) -> uint32_t {
      const float rc = rsc[col];
      v0 *= rc;
      w0 *= rc;
      v1 *= rc;
      w1 *= rc;
      const int sl = s0 + u / RT, rt = u % RT;
      const float h0 = (v0 / (1.0f + expf(-v0))) * w0, h1 = (v1 / (1.0f + expf(-v1))) * w1;
      A* dst = hb + ((long long)sl * T + col) * f + rt * 16 + row;
      if constexpr (sizeof(A) == 2) {
        const bf16x2 pr = {(__bf16)h0, (__bf16)h1};
        return __hip_atomic_exchange(reinterpret_cast<uint32_t*>(dst), __builtin_bit_cast(uint32_t, pr),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const uint32_t r0 = __hip_atomic_exchange(reinterpret_cast<uint32_t*>(dst), __builtin_bit_cast(uint32_t, h0),
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t r1 = __hip_atomic_exchange(reinterpret_cast<uint32_t*>(dst) + 1,
                                                  __builtin_bit_cast(uint32_t, h1), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        return r0 ^ r1;
      }
    };
    uint32_t* scnt = p.att_cnt + kSlotCnt;
    auto done = [=](int u) {
      __hip_atomic_fetch_add(scnt + kSlotStride * (s0 + u / RT), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    stage.issue();
    stage.finish();
    run_stream_dyn<EF, true, kGateDepth, gateup_split(EF)>(u1, KT, T, src, epi2, red, p.dummy, p.att_cnt + kGateCnt,
                                                           seq_lds(), done);
  } else if constexpr (MODE == 2) {
    stage.issue();
    stage.finish();
    run_stream_dyn<EF, true, kGateDepth, gateup_split(EF)>(u1, KT, T, src, epi, red, p.dummy, p.att_cnt + kGateCnt,
                                                           seq_lds());
  } else if constexpr (MODE == 1) {
    stage.issue();
    stage.finish();
    stream_units_wave<EF, true>(u0, u1, KT, T, src, epi, p.dummy);
  } else {
    stage.issue();
    Chunk<EF, true, 8> ck;
    const bool pr = wg_primable(KT, true);
    stream_prime<EF, true, true, 8, kPrimeTiles / 2>(ck, u0, u1, KT, src, p.dummy, pr);
    stage.finish();
    stream_units_wg_primed<EF, true, false, kPrimeTiles / 2>(u0, u1, KT, T, src, epi, red, p.dummy, ck, pr);
  }
}

// The shared experts do not depend on routing: when the grid has workgroups
// beyond the router's E/16 units, those run the shared experts' gate/up in the
// router phase (into slots 0 .. n_shared-1).
__device__ __forceinline__ bool shared_early(const LayerParams& p) {
  return p.nshared > 0 && (p.sch.grid_min > p.E / 16 || (int)gridDim.x > p.E / 16);
}

// ------------------------------------------------------------------ P5 router
template <int AF, int EF>
__device__ __forceinline__ void phase_router(const LayerParams& p, char* smem) {
  typedef typename Act<AF>::T A;
  constexpr int TK = tile_k(AF);
  const int T = p.T, XS = p.d + kXPad;
  LdsPlan lp(p, sizeof(A));
  A* xs = reinterpret_cast<A*>(smem);
  const int RT = p.E / 16;              // router units: 16 experts, all of d_model
  const bool early = shared_early(p);
  if (early && (int)blockIdx.x >= RT) {
    const int nwg = (int)gridDim.x - RT, U = p.nshared * (p.f / 16);
    int u0, u1;
    split_range(U, nwg, (int)blockIdx.x - RT, u0, u1);
    // RMSNorm-2 of H' into LDS, requested ahead of the first weight chunk
    struct Stage {
      const LayerParams& p;
      A* xs;
      int XS;
      RowStager<A, true> rs;
      __device__ void issue() { rs.issue(p.hp, p.T, p.d, p.g2); }
      __device__ void finish() {
        rs.finish(p.T, p.d, xs, (A*)nullptr, XS, p.eps);
        trace_x(p, 7);
      }
    } stage{p, xs, XS};
    if (u1 > u0) {
      gateup_units<EF, 0>(p, p.experts + p.E, 0, u0, u1, xs, reinterpret_cast<float*>(smem + lp.xb), stage);
    } else {
      stage.issue();
      stage.finish();
    }
    return;
  }
  A* xlo = AF == MK_FMT_F32 ? (A*)nullptr : reinterpret_cast<A*>(smem + lp.xb);
  float* red = reinterpret_cast<float*>(smem + 2 * lp.xb);
  const int KT = p.d / TK;
  int u0, u1;
  if (early) {
    u0 = blockIdx.x;
    u1 = u0 + 1;
  } else {
    split_range(RT, gridDim.x, blockIdx.x, u0, u1);
  }
  const A* bl = b_lane<A>(xs, XS, T, TK);
  struct Src {
    const uint8_t* wr; int KT; const A* bl; long long lo_off;
    __device__ const uint8_t* base(int u) const { return wr + (long long)u * KT * 1024; }
    __device__ const A* bbase(int) const { return bl; }
    __device__ const float* sbase(int) const { return nullptr; }
    __device__ const float* sbase2(int) const { return nullptr; }
  } src{p.wr, KT, bl, (long long)(lp.xb / (int)sizeof(A))};
  float* lgl = reinterpret_cast<float*>(smem + 2 * lp.xb + 2 * kWaves * 64 * 4 * 4);   // [4][kMaxT][16]
  const float* rsc = rsc_lds();       // the staged rows are h * gamma: scale by 1/rms
  auto epi = [=](int u, int row, int col, float v, float) { lgl[((u - u0) * kMaxT + col) * 16 + row] = v * rsc[col]; };
  RowStager<A, true> rs;
  rs.issue(p.hp, T, p.d, p.g2);
  Chunk<AF, false, 16> ck;
  const bool pr = wg_primable(KT, false);
  stream_prime<AF, false, true, 16, kPrimeTiles>(ck, u0, u1, KT, src, p.dummy, pr);
  rs.finish(T, p.d, xs, xlo, XS, p.eps);
  trace_x(p, 7);
  stream_units_wg_primed<AF, false, AF != MK_FMT_F32, kPrimeTiles>(u0, u1, KT, T, src, epi, red, p.dummy, ck, pr);
  if (u1 <= u0) return;
  __syncthreads();
  router_candidates(p, lgl, u0, u1);
}

// ------------------------------------------------------------------ P6 gate/up
template <int AF, int EF>
__device__ __forceinline__ void phase_route_gateup(const LayerParams& p, char* smem) {
  typedef typename Act<EF>::T A;
  static_assert((AF == MK_FMT_F32) == (EF == MK_FMT_F32), "activation types must agree");
  LdsPlan lp(p, sizeof(A));
  const A* xs = reinterpret_cast<const A*>(smem);      // x' (hi part) from P5
  float* red = reinterpret_cast<float*>(smem + lp.xb);
  RouteLds r = route_lds(p, smem, lp.xb);
  route_local(p, r);
  trace_x(p, 8);
  const int s0 = shared_early(p) ? p.nshared : 0;     // slots whose gate/up ran in P5
  const int ns = *r.nslots;
  const int U = (ns - s0) * (p.f / 16);
  const int KT = p.d / tile_k(EF);
  if (gateup_dyn_fits(KT, EF)) {
    // units handed out at run time (ticket counter), 8 waves per unit
    gateup_units<EF, 2>(p, r.blk + s0, s0, 0, U, xs, red);
    return;
  }
  int u0, u1;
  split_range(U, gridDim.x, blockIdx.x, u0, u1);
  if (U >= 2 * (int)gridDim.x * kWaves)
    gateup_units<EF, 1>(p, r.blk + s0, s0, u0, u1, xs, red);
  else
    gateup_units<EF, 0>(p, r.blk + s0, s0, u0, u1, xs, red);
}

// ------------------------------------------------------------------ P7 down projections (ticket-fed)
// Unit u = (slot u / QP, row tiles RTU (u % QP) ... RTU (u % QP) + RTU - 1 of
// d_model), QP = d_model / (16 RTU): RTU row tiles times all KT tiles of W2.
// Wave w streams row tile RTU (u % QP) + w % RTU over k part w / RTU (KT / KP
// tiles, KP = 8 / RTU, in chunks of D, the next chunk requested while the
// current one is multiplied, across unit boundaries); with two k parts the
// waves w and w + 4 add their blocks in LDS.  RTU = 4 (two k parts), or 8 (one
// k part, each wave's sums final) for MXFP4, whose rows hold half as many
// tiles.  Workgroup b
// first takes a run of R = min(8, units / nwg) consecutive units starting at
// b R (one slot, so its rows are loaded once), then draws tickets for the rest
// as run_stream_dyn does, so workgroups on faster XCDs take more units and the
// last units are spread over the grid.
//
// The rows of a unit's slot (h, T x d_ff in the operand type) sit in one of two
// LDS buffers.  When the next unit's slot differs, its rows are requested at the
// end of the current unit and stored into the other buffer when the next unit
// starts.  Slots from `s_wait` on may still be in their gate/up phase (no grid
// barrier in between): their rows are read only after the slot's completion
// counter has reached d_ff / 16 (thread 0 requests the counter when a unit
// starts and checks it, waiting if needed, when the unit ends), and they are read
// with agent-scope loads, which do not return stale lines of this XCD's L2.
__host__ __device__ constexpr bool down_dyn_fits(int d, int f, int tk, int es, int xb) {
  return d % (16 * down_rtu(tk)) == 0 && (f / tk) % (down_kp(tk) * kDownDepth) == 0 &&
         2 * kMaxT * (f + kXPad) * es <= xb &&
         kMaxT * f * es <= 16 * kThreads * 4;
}

// Whether the expert phases run fused: ticket-fed gate/up units whose slot
// completion counters let ticket-fed down projections start without a grid
// barrier in between.
template <int EF>
__device__ __forceinline__ bool experts_fused(const LayerParams& p, int xb) {
  constexpr int TK = tile_k(EF);
  const int KT = p.d / TK;
  return gateup_dyn_fits(KT, EF) &&
         down_dyn_fits(p.d, p.f, TK, (int)sizeof(typename Act<EF>::T), xb);
}

template <int EF>
__device__ __forceinline__ bool phase_down_dyn(const LayerParams& p, char* smem, int xb, const RouteLds& r,
                                               int s_wait) {
  typedef typename Act<EF>::T A;
  constexpr int TK = tile_k(EF);
  constexpr int D = kDownDepth;
  constexpr int RTU = down_rtu(TK), KP = down_kp(TK);
  constexpr int HW = 16;                                   // dwords of expert rows per thread, at most
  const int T = p.T, f = p.f, d = p.d, HS = f + kXPad;
  const int ns = *r.nslots;
  const int QP = d / (16 * RTU), KT = f / TK, NTh = KT / KP, cps = NTh / D;
  const int U = ns * QP;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = w % RTU, kp = w / RTU;
  const int nwg = (int)gridDim.x;
  const long long w2_off = p.exp_w13_bytes;
  const ExpScales<EF> es(p);
  // the two row buffers: hls + 0 and hls + hsz (offsets rather than an array of
  // pointers, so that every access stays an LDS access and never becomes FLAT)
  A* const hls = reinterpret_cast<A*>(smem);
  const int hsz = kMaxT * HS;
  float* red = reinterpret_cast<float*>(smem + xb);        // [2][8 waves][64][4]
  uint32_t* ctr = p.att_cnt + kDownCnt;
  const uint32_t* scnt = p.att_cnt + kSlotCnt;
  const uint32_t need = (uint32_t)(f / 16);                // gate/up units of one slot
  int* seq = seq_lds();
  int* flag = reinterpret_cast<int*>(smem + kFlagOff);
  const float* dsc = reinterpret_cast<const float*>(p.dummy);
  // This workgroup's first RS units are fixed: a run of R consecutive units
  // (all in one slot when R divides QP) when
  // there are at least two per workgroup, else units b and b + nwg; the rest
  // come from the tickets.  Consecutive units of one slot share its rows.
  const int R = min(8, U / nwg);
  const int RS = R >= 2 ? R : 2;
  auto static_unit = [&](int k) {
    const int u = R >= 2 ? (int)blockIdx.x * R + k : (int)blockIdx.x + k * nwg;
    return u < U ? u : -1;
  };
  int cur = static_unit(0);
  int nxt = static_unit(1);
  int kk = 0;                                              // cur's place in this workgroup's sequence
  if (cur < 0 || cps <= 0) return true;
  const int n32 = T * f * (int)sizeof(A) / 4;             // dwords of one slot's rows
  const int rw = f * (int)sizeof(A) / 4;                  // dwords of one row
  const int hw = (kMaxT * f * (int)sizeof(A) / 4 + kThreads - 1) / kThreads;
  // When a row is a whole number of kThreads-dword blocks (per of them),
  // thread block c of a slot's rows lies in row c / per, so the row test and
  // the block's offset are the same for the whole workgroup.  Otherwise the
  // index is taken through an opaque move, so that the addresses are formed
  // where they are used rather than hoisted out of the unit loop into
  // registers that would stay occupied while the tiles stream.
  const bool blk = rw % kThreads == 0;
  const int per = blk ? rw / kThreads : 1;
  auto h_load = [&](int sl, uint32_t* hv) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(reinterpret_cast<const A*>(p.hbuf) + (long long)sl * T * f);
    if (blk) {
#pragma unroll
      for (int c = 0; c < HW; ++c)
        if (c < hw) {
          const int t = c / per;
          hv[c] = __hip_atomic_load(src + min(t, T - 1) * rw + (c - t * per) * kThreads + (int)threadIdx.x,
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      return;
    }
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
#pragma unroll
    for (int c = 0; c < HW; ++c)
      if (c < hw)
        hv[c] = __hip_atomic_load(src + min(tid + kThreads * c, n32 - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto h_store = [&](A* buf, const uint32_t* hv) {
    if (blk) {
#pragma unroll
      for (int c = 0; c < HW; ++c) {
        const int t = c / per;
        if (c < hw && t < T)
          reinterpret_cast<uint32_t*>(buf + (long long)t * HS)[(c - t * per) * kThreads + (int)threadIdx.x] = hv[c];
      }
      return;
    }
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
#pragma unroll
    for (int c = 0; c < HW; ++c) {
      const int i = tid + kThreads * c;
      if (c < hw && i < n32) {
        const int t = i / rw;
        reinterpret_cast<uint32_t*>(buf + (long long)t * HS)[i - t * rw] = hv[c];
      }
    }
  };
  // thread 0: waits (bounded) until slot sl's gate/up units are all complete;
  // false when the wait timed out or another workgroup reported a fault
  auto slot_ready = [&](int sl, uint32_t seen) -> int {
    if (sl < s_wait || seen >= need) return 1;
    const uint64_t t0 = clock100();
    while (__hip_atomic_load(scnt + kSlotStride * sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
      __builtin_amdgcn_s_sleep(1);
      if ((long long)(clock100() - t0) > p.timeout_ticks) {
        __hip_atomic_store(&p.bar->fault, kFaultTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
      }
      if (__hip_atomic_load(&p.bar->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return 0;
    }
    return 1;
  };
  auto wbase = [&](int u) {
    const int sl = u / QP, rt = RTU * (u - sl * QP) + sub;
    return r.blk[sl] + w2_off + (long long)rt * KT * 1024 + lane * 16 + (long long)kp * NTh * 1024;
  };
  auto sbase = [&](int u) {
    const int sl = u / QP, rt = RTU * (u - sl * QP) + sub;
    return es.w2(r.blk[sl], rt);
  };
  u32x4 buf[D];
  float sc[D];
  {
    // issued as the loop issues a chunk (see run_stream_dyn)
    const uint8_t* cb = wbase(cur);
    const float* sp = scaled_fmt(EF) ? sbase(cur) : dsc;
    const int vz = vzero();
#pragma unroll
    for (int rr = 0; rr < D; ++rr) {
      buf[rr] = ld_stream16(cb + rr * 1024);
      if constexpr (scaled_fmt(EF)) sc[rr] = tile_scale<EF, false>(sp, kp * NTh + rr, lane, vz);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the first unit's rows, staged synchronously (its first weight chunk, which
  // does not depend on the slot's gate/up units, is already on its way)
  if (threadIdx.x == 0) *flag = slot_ready(cur / QP, 0);
  __syncthreads();
  if (!*flag) return false;
  uint32_t hv[HW];
  h_load(cur / QP, hv);
  h_store(hls, hv);
  __syncthreads();
  trace_x(p, 15);
  uint32_t tk = 0, cseen = 0;
  int cq = (int)blockIdx.x & 7;
  int cc = 0, par = 0, hb = 0;
  bool hpend = false;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  BPair bn;
  f32x4 tp = zero;
  float sp = 0.f;
  const int j = lane & 15, g = lane >> 4, jj = j < T ? j : T - 1;
  float* yb = p.ybuf;
  while (true) {
    if (cc == 0) {
      if (hpend) {
        // this unit's rows, requested when the previous unit ended
        h_store(hls + (hb ^ 1) * hsz, hv);
        __syncthreads();
        hb ^= 1;
      }
      if (threadIdx.x == 0) {
        if (kk + 2 >= RS)
          tk = __hip_atomic_fetch_add(ctr + kCntStride * cq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int ns2 = nxt >= 0 ? nxt / QP : 0;
        cseen = (nxt >= 0 && ns2 != cur / QP && ns2 >= s_wait)
                    ? __hip_atomic_load(scnt + kSlotStride * ns2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : need;
      }
    }
    int ncc = cc + 1, un = cur;
    if (ncc == cps) {
      ncc = 0;
      un = nxt;
    }
    const bool has_next = un >= 0;
    const uint8_t* nb = has_next ? wbase(un) + (long long)ncc * D * 1024 : p.dummy + lane * 16;
    const float* nsp = dsc;
    if constexpr (scaled_fmt(EF)) {
      if (has_next) nsp = sbase(un);
    }
    const A* bp = hls + hb * hsz + jj * HS + g * (TK / 4) + (kp * NTh + cc * D) * TK;
    // fp8: B read one tile ahead, scaled products added one tile later (see
    // run_stream_dyn); a chunk's first B is read here, after the rows' barrier
    if constexpr (EF == MK_FMT_FP8_B128) bn = b_pair(bp);
#pragma unroll
    for (int rr = 0; rr < D; ++rr) {
      if constexpr (EF == MK_FMT_FP8_B128) {
        const BPair b = bn;
        if (rr + 1 < D) bn = b_pair(bp + (rr + 1) * TK);
        const f32x4 tmp = tile_mma_fp8(buf[rr], b, zero);
        acc += tp * sp;
        tp = tmp;
        sp = keep_copy(sc[rr]);
      } else if constexpr (EF == MK_FMT_MXFP4) {
        acc = tile_mma_mx(buf[rr], bp + rr * TK, sc[rr], acc);
      } else {
        acc = tile_mma<EF>(buf[rr], bp + rr * TK, acc);
      }
      buf[rr] = ld_stream16(nb + rr * 1024);
      if constexpr (scaled_fmt(EF))
        sc[rr] = tile_scale<EF, false>(nsp, has_next ? kp * NTh + ncc * D + rr : 0, lane);
      __builtin_amdgcn_sched_barrier(0);   // loads in consumption order (see run_stream_dyn)
    }
    cc = ncc;
    if (ncc != 0) continue;
    // unit `cur` complete: the blocks of waves w and w + 4 added (two k
    // parts), the unit after nxt published, the next slot's completion confirmed
    if constexpr (EF == MK_FMT_FP8_B128) {
      acc += tp * sp;
      tp = zero;
      sp = 0.f;
    }
    float* rb = red + par * (kWaves * 64 * 4);
    if constexpr (KP == 2) {
      *reinterpret_cast<f32x4*>(rb + (w * 64 + lane) * 4) = acc;
    } else {
      // one k part: this wave's sums are final (lane: rows 4 g + e, column j)
      if (j < T) {
        const int sl = cur / QP, rt = RTU * (cur - sl * QP) + sub;
#pragma unroll
        for (int e = 0; e < 4; ++e) yb[((long long)sl * T + j) * d + rt * 16 + 4 * g + e] = acc[e];
      }
    }
    if (threadIdx.x == 0) {
      if (kk + 2 < RS) {
        seq[par] = static_unit(kk + 2);
      } else {
        long long un2 = (long long)RS * nwg + 8LL * tk + cq;
        for (int tries = 1; un2 >= U && tries < 8; ++tries) {
          cq = (cq + 1) & 7;
          tk = __hip_atomic_fetch_add(ctr + kCntStride * cq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          un2 = (long long)RS * nwg + 8LL * tk + cq;
        }
        seq[par] = un2 < U ? (int)un2 : -1;
      }
      *flag = (nxt >= 0 && nxt / QP != cur / QP) ? slot_ready(nxt / QP, cseen) : 1;
    }
    __syncthreads();
    if (!*flag) return false;
    if (kk == 0) trace_x(p, 4);
    if constexpr (KP == 2) {
      const int s4 = threadIdx.x >> 7, rem = threadIdx.x & 127, row = rem >> 3, col = rem & 7;
      if (col < T) {
        const int l = (row >> 2) * 16 + col, e = row & 3;
        const float v = rb[(s4 * 64 + l) * 4 + e] + rb[((s4 + 4) * 64 + l) * 4 + e];
        const int sl = cur / QP, rt = RTU * (cur - sl * QP) + s4;
        yb[((long long)sl * T + col) * d + rt * 16 + row] = v;
      }
    }
    // the next unit's rows, when its slot differs (they are waited for when
    // it starts, together with every older load)
    hpend = nxt >= 0 && nxt / QP != cur / QP;
    if (hpend) {
      h_load(nxt / QP, hv);
    } else {
      // defined on both paths, so that the registers are free while the tiles stream
#pragma unroll
      for (int c = 0; c < HW; ++c) hv[c] = 0u;
    }
    acc = zero;
    cur = nxt;
    nxt = nxt >= 0 ? seq[par] : -1;
    par ^= 1;
    ++kk;
    if (cur < 0) break;
  }
  __syncthreads();
  return true;
}

// ------------------------------------------------------------------ P7 down projections
template <int EF>
__device__ __forceinline__ void phase_down(const LayerParams& p, char* smem) {
  typedef typename Act<EF>::T A;
  constexpr int TK = tile_k(EF);
  const int T = p.T, XS = p.f + kXPad;
  LdsPlan lp(p, sizeof(A));
  A* xs = reinterpret_cast<A*>(smem);
  float* red = reinterpret_cast<float*>(smem + lp.xb);
  RouteLds r = route_lds(p, smem, lp.xb);
  const int ns = *r.nslots;
  const int RT = p.d / 16, KT = p.f / TK, U = ns * RT;
  int u0, u1;
  split_range(U, gridDim.x, blockIdx.x, u0, u1);
  const A* bl = b_lane<A>(xs, XS, T, TK);
  const ExpScales<EF> es(p);
  struct Src {
    const uint8_t* blk; int RT, KT; const A* bl; long long w2_off; ExpScales<EF> es;
    __device__ const uint8_t* base(int u) const { return blk + w2_off + (long long)(u % RT) * KT * 1024; }
    __device__ const A* bbase(int) const { return bl; }
    __device__ const float* sbase(int u) const { return es.w2(blk, u % RT); }
    __device__ const float* sbase2(int) const { return nullptr; }
  };
  // several slots per source: each unit finds its slot's block and staged operand
  struct SrcMulti {
    const uint8_t* const* blk; int RT, KT, sa; const A* bl; long long slot_elems, w2_off; ExpScales<EF> es;
    __device__ const uint8_t* base(int u) const {
      return blk[u / RT] + w2_off + (long long)(u % RT) * KT * 1024;
    }
    __device__ const A* bbase(int u) const { return bl + (u / RT - sa) * slot_elems; }
    __device__ const float* sbase(int u) const { return es.w2(blk[u / RT], u % RT); }
    __device__ const float* sbase2(int) const { return nullptr; }
  };
  float* yb = p.ybuf;
  const int d = p.d, f = p.f;
  auto epi = [=](int uu, int row, int col, float v, float) {
    const int sl = uu / RT, rt = uu - sl * RT;
    yb[((long long)sl * T + col) * d + rt * 16 + row] = v;
  };
  if (down_dyn_fits(p.d, p.f, TK, (int)sizeof(A), lp.xb)) {
    phase_down_dyn<EF>(p, smem, lp.xb, r, 1 << 30);
    return;
  }
  if (U >= 2 * (int)gridDim.x * kWaves) {
    // wave-level units; stage up to two slots' activations at a time
    const long long slot_elems = (long long)kMaxT * XS;
    int u = u0;
    while (u < u1) {
      const int sa = u / RT;
      const int ue = min(u1, (sa + 2) * RT);
      const int sb = (ue - 1) / RT;
      for (int sl = sa; sl <= sb; ++sl)
        rows_copy_lds<A>(reinterpret_cast<const A*>(p.hbuf) + (long long)sl * T * f, T, f, xs + (sl - sa) * slot_elems,
                         XS);
      if (u == u0) trace_x(p, 9);
      SrcMulti src{r.blk, RT, KT, sa, bl, slot_elems, p.exp_w13_bytes, es};
      stream_units_wave<EF, false>(u, ue, KT, T, src, epi, p.dummy);
      __syncthreads();
      u = ue;
    }
  } else {
    int u = u0;
    while (u < u1) {
      const int sl = u / RT;
      const int ue = min(u1, (sl + 1) * RT);
      rows_copy_lds<A>(reinterpret_cast<const A*>(p.hbuf) + (long long)sl * T * f, T, f, xs, XS);
      Src src{r.blk[sl], RT, KT, bl, p.exp_w13_bytes, es};
      stream_units_wg<EF, false, false>(u, ue, KT, T, src, epi, red, p.dummy);
      u = ue;
    }
  }
}

// The fused expert phases: routing, ticket-fed gate/up (counted per slot), then
// ticket-fed down projections, which wait per slot instead of at a grid barrier.
template <int AF, int EF>
__device__ __forceinline__ void phase_experts_fused(const LayerParams& p, char* smem) {
  typedef typename Act<EF>::T A;
  LdsPlan lp(p, sizeof(A));
  const A* xs = reinterpret_cast<const A*>(smem);      // x' (hi part) from P5
  float* red = reinterpret_cast<float*>(smem + lp.xb);
  RouteLds r = route_lds(p, smem, lp.xb);
  route_local(p, r);
  trace_x(p, 8);
  const int s0 = shared_early(p) ? p.nshared : 0;     // slots whose gate/up ran in P5
  const int ns = *r.nslots;
  gateup_units<EF, 3>(p, r.blk + s0, s0, 0, (ns - s0) * (p.f / 16), xs, red);
  __syncthreads();
  trace_x(p, 9);
  phase_down_dyn<EF>(p, smem, lp.xb, r, s0);
}

// ------------------------------------------------------------------ P8 combine
__device__ __forceinline__ void phase_combine(const LayerParams& p, char* smem, int xb) {
  RouteLds r = route_lds(p, smem, xb);
  const int T = p.T, d = p.d, K = p.topk;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < T * d; i += gridDim.x * kThreads) {
    const int t = i / d, c = i - t * d;
    float v = ldg(p.hp + i);
    for (int k = 0; k < K; ++k)
      v += r.gate[t * kMaxTopK + k] * ldg(p.ybuf + ((long long)r.slot_of[t * kMaxTopK + k] * T + t) * d + c);
    for (int s = 0; s < p.nshared; ++s) v += ldg(p.ybuf + ((long long)s * T + t) * d + c);
    p.out[i] = v;
  }
}

// ------------------------------------------------------------------ the kernel
// Layer shapes with an instance of their own, where every dimension (and the
// projection's split-K factor, 1) is a compile-time constant: address
// arithmetic folds, the ragged-shape engines drop out, and fewer values stay
// live across phases.
struct SpecShape {
  int d, nh, dh, dc, dr, E, topk, nshared, f, s_q;
};
constexpr SpecShape kSpecShapes[] = {
    {0, 0, 0, 0, 0, 0, 0, 0, 0, 0},                 // 0: dimensions read from the parameters
    {4096, 32, 128, 512, 64, 128, 8, 1, 1024, 1},   // 1: 128 experts of width 1024
    {4096, 32, 128, 512, 64, 384, 8, 1, 2048, 1},   // 2: 384 experts of width 2048
};
template <int SPEC>
__device__ __forceinline__ void specialise(LayerParams& p) {
  if constexpr (SPEC > 0) {
    constexpr SpecShape s = kSpecShapes[SPEC];
    p.d = s.d; p.nh = s.nh; p.dh = s.dh; p.dc = s.dc; p.dr = s.dr;
    p.qw = s.dh + s.dr; p.kvw = s.dc + s.dr; p.nq = s.nh * (s.dh + s.dr);
    p.E = s.E; p.topk = s.topk; p.nshared = s.nshared; p.f = s.f;
    p.sch.s_q = s.s_q;
    p.sch.grid_min = kSpecMinGrid;
    if (p.itopk == 0) p.kv_row = s.dc + s.dr;
  }
}

// A workgroup leaving the launch because a barrier failed passes the layer's
// fault on to the stack's fault word (so that later layers skip their work and
// the stack's head commits nothing).
__device__ __forceinline__ void raise_model_fault(const LayerParams& p) {
  if (p.model_fault && threadIdx.x == 0) {
    const uint32_t f = __hip_atomic_load(&p.bar->fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.model_fault, f ? f : kFaultTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// LR: the layer has a low-rank query (W_DQ, q-norm, W_UQ; phase P0b between
// P0 and P1, one grid barrier more) and may normalise its cached latent.
// SP: sparse attention (indexer projections in P0, index keys cached in P1,
// index scores P1b and top-k P1c, each followed by a grid barrier; attention
// over the kept rows).
template <int AF, int EF, int KF, int KBMAX, int DBMAX, bool EXACT, int SPEC, bool LR = false, bool SP = false>
__global__ __launch_bounds__(kThreads, 1) void layer_kernel(LayerParams p) {
  specialise<SPEC>(p);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int* flag = reinterpret_cast<int*>(smem + kFlagOff);
  // a stack step that already failed (an earlier layer, a bad token id) does
  // no further work; every workgroup reads the same word (written by earlier
  // launches on the stream) and leaves before the first barrier
  if (p.model_fault && __hip_atomic_load(p.model_fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  const int L = p.L_dev ? ldg(p.L_dev) : p.L;
  if (L < 0 || (long long)L + p.T > p.kv_capacity || (SP && (long long)L + p.T > p.imax)) {
    // every workgroup reads the same L and leaves before the first barrier
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      __hip_atomic_store(&p.bar->fault, kFaultKvRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.model_fault) __hip_atomic_store(p.model_fault, kFaultKvRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (p.trace && threadIdx.x == 0) {
    long long* tl = trace_lds();
    for (int i = 1; i < kTraceStride; ++i) tl[i] = 0;
    tl[0] = (long long)clock100();
  }
  // ticket counters of the expert phases: cleared here, used after several grid barriers
  if (blockIdx.x == 0 && threadIdx.x < 16)
    __hip_atomic_store(&p.att_cnt[kGateCnt + kCntStride * threadIdx.x], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);   // gate/up and down ticket counters
  if (blockIdx.x == 0 && threadIdx.x < kMaxSlots)
    __hip_atomic_store(&p.att_cnt[kSlotCnt + kSlotStride * threadIdx.x], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);   // slot completion counters
  phase_qkv<AF, LR, SP>(p, smem);
  if (!grid_barrier(p, 0, flag)) return raise_model_fault(p);
  if constexpr (LR) {
    phase_uq<AF, SP>(p, smem);
    if (!grid_barrier(p, 8, flag)) return raise_model_fault(p);
  }
  if constexpr (SP) {
    stage_index_queries<LR>(p, blockIdx.x * kThreads + threadIdx.x, gridDim.x * kThreads);
    // the top-k's row histograms and part counters start at zero
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < kMaxT * (kTopkBins + kIdxCtrStride); i += gridDim.x * kThreads)
      __hip_atomic_store(i < kMaxT * kTopkBins ? p.ihist + i : p.ictr + (i - kMaxT * kTopkBins), 0u,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  {
    // absorbed-query units on waves [0, wa) of every workgroup; when they fit
    // in half the waves, RoPE / KV insert runs on the other half meanwhile
    const int gs = p.sch.grid_min > 0 ? p.sch.grid_min : (int)gridDim.x;   // never above the grid
    const int wa = (p.nh * (p.dc / 16) + gs - 1) / gs;
    if (wa <= kWaves / 2) {
      if ((int)threadIdx.x < kThreads / 2) phase_absorb<AF, LR, SP>(p);
      else phase_rope_kv<KF, LR, SP>(p, L, blockIdx.x * (kThreads / 2) + threadIdx.x - kThreads / 2,
                                     gridDim.x * (kThreads / 2));
    } else {
      phase_rope_kv<KF, LR, SP>(p, L, blockIdx.x * kThreads + threadIdx.x, gridDim.x * kThreads);
      phase_absorb<AF, LR, SP>(p);
    }
  }
  if (!grid_barrier(p, 1, flag)) return raise_model_fault(p);
  if constexpr (SP) {
    phase_iscore<KF == MK_FMT_FP8_ROW>(p, L, smem);
    if (!grid_barrier(p, 9, flag)) return raise_model_fault(p);
    phase_topk(p, L, smem);
    if (!grid_barrier(p, 10, flag)) return raise_model_fault(p);
  }
  // long contexts: four query tiles per unit (the instance for the dense bf16
  // cache of the 512 + 64 latent shape only); P3 merges the same plan
  bool att_sh = false;
  if constexpr (KF == MK_FMT_BF16 && EXACT && !SP && KBMAX == 18 && DBMAX == 32)
    att_sh = attn_shared(p, (p.T * p.nh + 15) / 16, L + p.T);
  if (att_sh) phase_attention_shared(p, L, smem);
  else phase_attention<KF, KBMAX, DBMAX, EXACT, SP>(p, L, smem);
  if (!grid_barrier(p, 2, flag)) return raise_model_fault(p);
  phase_merge_uv<AF, SP>(p, L, smem, att_sh);
  if (!grid_barrier(p, 3, flag)) return raise_model_fault(p);
  phase_wo<AF>(p, smem);
  if (!grid_barrier(p, 4, flag)) return raise_model_fault(p);
  phase_router<AF, EF>(p, smem);
  if (!grid_barrier(p, 5, flag)) return raise_model_fault(p);
  if (experts_fused<EF>(p, LdsPlan(p, EF == MK_FMT_F32 ? 4 : 2).xb)) {
    phase_experts_fused<AF, EF>(p, smem);
  } else {
    phase_route_gateup<AF, EF>(p, smem);
    if (!grid_barrier(p, 6, flag)) return raise_model_fault(p);
    phase_down<EF>(p, smem);
  }
  if (!grid_barrier(p, 7, flag)) return raise_model_fault(p);
  LdsPlan lp(p, EF == MK_FMT_F32 ? 4 : 2);
  phase_combine(p, smem, lp.xb);
  if (p.trace && threadIdx.x == 0) {
    long long* tl = trace_lds();
    tl[1 + 2 * kBarriers] = (long long)clock100();
    for (int i = 0; i < kTraceStride; ++i) p.trace[(long long)blockIdx.x * kTraceStride + i] = tl[i];
  }
}

}  // namespace mk
