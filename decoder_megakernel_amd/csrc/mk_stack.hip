// Stack pieces around the layer kernel: embedding gather, and one launch that
// does the final RMSNorm, the LM-head projection (bf16, or fp8 E4M3 with
// 128x128 block scales), and the verification of the drafts -- greedy (argmax
// per verify row) or sampled at a temperature -- with the device-side
// bookkeeping (the lm_head and rejection-kernel rows of the per-step kernel
// table in "Why one GB300 doesn't beat 4x RTX PRO 6000 at single-stream
// decode", section "Where the 11.2 ms goes", and the fp8 head of its section
// "Three readings"; greedy decoding as the engine gate uses it and sampling
// with matched random draws, "DeepSeek-V4.1-Flash breaks 1,000 tokens per
// second for one user", section "The safety layer").
#include "mk_device.h"
#include "mk_host.h"

namespace mk {

// A token id outside [0, V) is not clamped: its row is left as zeros and the
// stack's fault word is set, so the layers skip their work and the head
// commits nothing.
__global__ __launch_bounds__(256) void embed_kernel(const uint16_t* emb, int V, int d, const int32_t* tokens, int T,
                                                    float* h, uint32_t* fault) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < T * d; i += gridDim.x * 256) {
    const int t = i / d, k = i - t * d;
    const int tok = tokens[t];
    if (tok < 0 || tok >= V) {
      h[i] = 0.f;
      if (k == 0) __hip_atomic_store(fault, kFaultToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    h[i] = __uint_as_float((uint32_t)emb[(long long)tok * d + k] << 16);
  }
}

int launch_embed(const uint16_t* emb, int V, int d, const int32_t* tokens, int T, float* h, uint32_t* fault,
                 hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(64), dim3(256), 0, s, emb, V, d, tokens, T, h, fault);
  return (int)hipGetLastError();
}

struct HeadArgs {
  const uint8_t* head; int V, d; const float* gamma; float eps; const float* h; int T;
  float* logits; float* best_val; int32_t* best_idx; uint32_t* counter; int32_t* tokens;
  const int32_t* next_drafts; int32_t* argmax; int32_t* committed; int32_t* kv_len; const uint8_t* dummy;
  const uint32_t* fault;   // the stack's fault word
  uint32_t* tickets;       // 8 ticket counters, kCntStride words apart (zero between launches)
  const float* scales;     // fp8 head: fp32 block scales [ceil(V/128)][ceil(d/128)]
  float inv_tau;           // sampled verification: 1 / temperature
  uint64_t seed;           // sampled verification: the draws of step s are keyed by (seed, s)
  uint32_t* step;          // sampled verification: s, advanced by every step that commits
  float* part;             // sampled verification: per-workgroup row states [nwg][8][8]
};

// ---- sampled verification
// Speculative sampling with the drafts as point proposals: row i's target is
// p_i = softmax(logits_i / tau); draft i+1 is accepted when the row's
// acceptance draw is below p_i(draft); the first rejection commits a draw from
// p_i without the draft, T-1 acceptances a draw from p_{T-1}.  Token draws are
// Gumbel-max (argmax of logit / tau - ln(-ln u), ties to the lower id).
// Draws: SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) outputs from the
// step's key mix(seed + (s + 1) gamma): u(i) = ((mix(key + (i + 1) gamma) >> 41)
// + 1/2) 2^-23, token draw (row r, id v) at i = r (V + 1) + v, the row's
// acceptance draw at i = r (V + 1) + V.
constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;
__device__ __forceinline__ uint64_t splitmix_out(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ float draw_uniform(uint64_t key, uint64_t i) {
  const uint64_t r = splitmix_out(key + (i + 1) * kGolden);
  return ((float)(uint32_t)(r >> 41) + 0.5f) * 0x1p-23f;     // exact: 24 significant bits
}
// A row's running state over a set of vocabulary ids: the maximum m of
// x = logit / tau and the sum s of exp(x - m), the best Gumbel-perturbed id and
// the best one other than the row's next draft, and x of that draft.
struct RowState {
  float m, s, yb, yx, xd;
  int ib, ix;
};
__device__ __forceinline__ RowState row_state_empty() {
  return RowState{-INFINITY, 0.f, -INFINITY, -INFINITY, -INFINITY, 0x7fffffff, 0x7fffffff};
}
__device__ __forceinline__ void row_state_merge(RowState& a, const RowState& b) {
  const float M = fmaxf(a.m, b.m);
  const float sa = a.m == -INFINITY ? 0.f : a.s * __expf(a.m - M);
  const float sb = b.m == -INFINITY ? 0.f : b.s * __expf(b.m - M);
  a.m = M;
  a.s = sa + sb;
  if (b.yb > a.yb || (b.yb == a.yb && b.ib < a.ib)) { a.yb = b.yb; a.ib = b.ib; }
  if (b.yx > a.yx || (b.yx == a.yx && b.ix < a.ix)) { a.yx = b.yx; a.ix = b.ix; }
  a.xd = fmaxf(a.xd, b.xd);
}

constexpr int kHeadLds = 8 * (8192 + kXPad) * 2 + 2 * kWaves * 64 * 4 * 4 + 1024;
constexpr int kHeadMergeB = 4;           // per-workgroup states loaded together per thread in the grid merge

__device__ __forceinline__ RowState rs_shfl_xor(const RowState& r, int m) {
  return RowState{__shfl_xor(r.m, m), __shfl_xor(r.s, m), __shfl_xor(r.yb, m), __shfl_xor(r.yx, m),
                  __shfl_xor(r.xd, m), __shfl_xor(r.ib, m), __shfl_xor(r.ix, m)};
}
// LDS slots of RowState for kThreads threads (7 arrays of kThreads words)
__device__ __forceinline__ void rs_put(char* base, int i, const RowState& r) {
  float* f = reinterpret_cast<float*>(base);
  int* n = reinterpret_cast<int*>(base);
  f[i] = r.m; f[kThreads + i] = r.s; f[2 * kThreads + i] = r.yb; f[3 * kThreads + i] = r.yx;
  f[4 * kThreads + i] = r.xd; n[5 * kThreads + i] = r.ib; n[6 * kThreads + i] = r.ix;
}
__device__ __forceinline__ RowState rs_get(const char* base, int i) {
  const float* f = reinterpret_cast<const float*>(base);
  const int* n = reinterpret_cast<const int*>(base);
  return RowState{f[i], f[kThreads + i], f[2 * kThreads + i], f[3 * kThreads + i], f[4 * kThreads + i],
                  n[5 * kThreads + i], n[6 * kThreads + i]};
}

// After the stream of a sampled step: the workgroup's state per row to memory,
// and in the last workgroup the grid-wide states, the acceptance decisions and
// the bookkeeping.  cvb: LDS free for 7 * kThreads words; misc: 1 KiB of LDS.
__device__ __forceinline__ void head_sample_tail(const HeadArgs& a, const RowState& mine, uint64_t key, char* cvb, float* misc) {
  const int T = a.T, V = a.V;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the four lanes of a wave that hold one column, then the 8 waves (LDS)
  RowState r0 = mine;
  row_state_merge(r0, rs_shfl_xor(r0, 16));
  row_state_merge(r0, rs_shfl_xor(r0, 32));
  if (lane < 16) rs_put(cvb, w * 16 + lane, r0);
  __syncthreads();
  if ((int)threadIdx.x < T) {
    RowState r = rs_get(cvb, threadIdx.x);
    for (int q = 1; q < kWaves; ++q) row_state_merge(r, rs_get(cvb, q * 16 + threadIdx.x));
    // agent-scope stores pass this XCD's L2 (read by the merging workgroup on any XCD)
    float* dst = a.part + ((long long)blockIdx.x * 8 + threadIdx.x) * 8;
    const float wd[7] = {r.m, r.s, r.yb, r.yx, r.xd, __int_as_float(r.ib), __int_as_float(r.ix)};
#pragma unroll
    for (int k = 0; k < 7; ++k) __hip_atomic_store(dst + k, wd[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wg_release_begin();
  int* flag = reinterpret_cast<int*>(misc + 250);
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == gridDim.x - 1;
    if (last) {
      __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int c = 0; c < 8; ++c)
        __hip_atomic_store(a.tickets + kCntStride * c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  // grid-wide state per row: thread x takes row x % 8 of workgroups x / 8,
  // x / 8 + 64, ... (loads issued in batches), then the 64 partial states of a
  // row are merged in LDS in a fixed order
  {
    const int t = threadIdx.x & 7, b0 = threadIdx.x >> 3;
    RowState r = row_state_empty();
    if (t < T) {
      for (int bb = b0; bb < (int)gridDim.x; bb += 64 * kHeadMergeB) {
        float wd[kHeadMergeB][7];
#pragma unroll
        for (int i = 0; i < kHeadMergeB; ++i) {
          const int b = bb + 64 * i;
          const float* src = a.part + ((long long)min(b, (int)gridDim.x - 1) * 8 + t) * 8;
#pragma unroll
          for (int k = 0; k < 7; ++k) wd[i][k] = __hip_atomic_load(src + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < kHeadMergeB; ++i)
          if (bb + 64 * i < (int)gridDim.x)
            row_state_merge(r, RowState{wd[i][0], wd[i][1], wd[i][2], wd[i][3], wd[i][4], __float_as_int(wd[i][5]),
                                        __float_as_int(wd[i][6])});
      }
    }
    // the eight lanes of a wave that hold one row, then the 8 waves (LDS)
    row_state_merge(r, rs_shfl_xor(r, 8));
    row_state_merge(r, rs_shfl_xor(r, 16));
    row_state_merge(r, rs_shfl_xor(r, 32));
    if (lane < 8) rs_put(cvb, w * 8 + lane, r);
  }
  int* am = reinterpret_cast<int*>(misc + 200);
  int* tk = reinterpret_cast<int*>(misc + 208);
  int* rx = reinterpret_cast<int*>(misc + 216);
  float* pa = misc + 224;
  if ((int)threadIdx.x < T) tk[threadIdx.x] = a.tokens[threadIdx.x];
  __syncthreads();
  if ((int)threadIdx.x < T) {
    RowState r = rs_get(cvb, threadIdx.x);
    for (int q = 1; q < kWaves; ++q) row_state_merge(r, rs_get(cvb, q * 8 + threadIdx.x));
    am[threadIdx.x] = r.ib;
    rx[threadIdx.x] = r.ix;
    pa[threadIdx.x] = r.xd == -INFINITY ? 0.f : expf(r.xd - r.m) / r.s;   // p_i(next draft)
    a.argmax[threadIdx.x] = r.ib;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0, fin = -1;
    for (; n + 1 <= T - 1; ++n) {
      const float ua = draw_uniform(key, (uint64_t)n * (uint64_t)(V + 1) + (uint64_t)V);
      if (!(ua < pa[n])) {
        fin = rx[n];
        break;
      }
    }
    if (n == T - 1) fin = am[T - 1];
    a.committed[0] = n + 1;
    for (int i = 1; i <= n; ++i) a.committed[i] = tk[i];
    a.committed[n + 1] = fin;
    if (a.kv_len) a.kv_len[0] += n + 1;
    a.step[0] += 1u;
    a.tokens[0] = fin;
    if (a.next_drafts)
      for (int i = 1; i < T; ++i) a.tokens[i] = a.next_drafts[i - 1];
  }
}
constexpr int kHeadNormB = 16;           // float4 loads per lane in flight while normalising a row

template <int HF, bool SAMPLE>
__global__ __launch_bounds__(kThreads, 1) void head_kernel(HeadArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int T = a.T, d = a.d, XS = d + kXPad;
  // a step in which a layer or the embedding failed commits nothing: no
  // token, no KV length change, the token buffer left as it was (every
  // workgroup reads the same word, written by earlier launches on the stream)
  if (__hip_atomic_load(a.fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
    if (blockIdx.x == 0 && (int)threadIdx.x < T) {
      a.argmax[threadIdx.x] = -1;
      if (threadIdx.x == 0) a.committed[0] = 0;
    }
    return;
  }
  __bf16* xs = reinterpret_cast<__bf16*>(smem);
  float* red = reinterpret_cast<float*>(smem + 8 * XS * 2);
  float* misc = reinterpret_cast<float*>(smem + kHeadLds - 1024);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  auto stage = [&]() {
    // final RMSNorm into LDS: wave t < T normalises row t.  The row is read in
    // batches of kHeadNormB float4s per lane, every load of a batch issued
    // before the first is used (one memory round trip per batch, not per element).
    if (w < T) {
      const f32x4* hr = reinterpret_cast<const f32x4*>(a.h + (long long)w * d);
      const f32x4* gr = reinterpret_cast<const f32x4*>(a.gamma);
      const int n4 = d / 4;
      float ss = 0.f;
      for (int b0 = 0; b0 < n4; b0 += 64 * kHeadNormB) {
        f32x4 v[kHeadNormB];
#pragma unroll
        for (int i = 0; i < kHeadNormB; ++i) {
          const int q = b0 + i * 64 + lane;
          v[i] = q < n4 ? ldg(hr + q) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < kHeadNormB; ++i) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      const float rs = 1.0f / sqrtf(ss / (float)d + a.eps);
      for (int b0 = 0; b0 < n4; b0 += 64 * kHeadNormB) {
        f32x4 v[kHeadNormB], gm[kHeadNormB];
#pragma unroll
        for (int i = 0; i < kHeadNormB; ++i) {
          const int q = min(b0 + i * 64 + lane, n4 - 1);
          v[i] = ldg(hr + q);
          gm[i] = ldg(gr + q);
        }
#pragma unroll
        for (int i = 0; i < kHeadNormB; ++i) {
          const int q = b0 + i * 64 + lane;
          if (q < n4) {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)((v[i][e] * rs) * gm[i][e]);
            *reinterpret_cast<bf16x4*>(xs + w * XS + 4 * q) = o;
          }
        }
      }
    }
    __syncthreads();
  };
  constexpr int TK = tile_k(HF);
  constexpr int D = 16;                                  // tiles per wave per chunk
  // fp8 rows are half as long: two row tiles per workgroup at a time, four
  // waves on each, so a wave still streams 16 KiB per chunk
  constexpr int SPLIT = HF == MK_FMT_FP8_B128 ? 2 : 1;
  constexpr int WPU = kWaves / SPLIT;
  const int RT = a.V / 16, KT = d / TK;
  const long long U = RT;
  const int u0 = (int)(U * blockIdx.x / gridDim.x), u1 = (int)(U * (blockIdx.x + 1) / gridDim.x);
  const int j = lane & 15, g = lane >> 4;
  const __bf16* bl = xs + (j < T ? j : T - 1) * XS + g * (TK / 4);
  struct Src {
    const uint8_t* head; int KT; const __bf16* bl; const float* sc; int nbk;
    __device__ const uint8_t* base(int u) const { return head + (long long)u * KT * 1024; }
    __device__ const __bf16* bbase(int) const { return bl; }
    // the unit's 16 rows lie in one 128-row block row of the scales
    __device__ const float* sbase(int u) const { return sc ? sc + (long long)(u >> 3) * nbk : nullptr; }
    __device__ const float* sbase2(int) const { return nullptr; }
  } src{a.head, KT, bl, a.scales, (d + 127) / 128};
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  float* logits = a.logits;
  const int V = a.V;
  // sampled verification: this thread's column (its epilogue values are all
  // of column threadIdx.x % 16), the step's key and the column's next draft
  RowState rs = row_state_empty();
  uint64_t key = 0;
  int dn = -1;
  if constexpr (SAMPLE) {
    key = splitmix_out(a.seed + ((uint64_t)ldg(a.step) + 1) * kGolden);
    const int c = threadIdx.x & 15;
    dn = c + 1 < T ? ldg(a.tokens + c + 1) : -1;
  }
  auto epi = [&](int u, int row, int col, float v, float) {
    const int id = u * 16 + row;
    if (logits) logits[(long long)col * V + id] = v;
    if constexpr (SAMPLE) {
      const float x = v * a.inv_tau;
      if (x > rs.m) {
        rs.s = rs.s * __expf(rs.m - x) + 1.f;
        rs.m = x;
      } else {
        rs.s += __expf(x - rs.m);
      }
      const float y = x - logf(-logf(draw_uniform(key, (uint64_t)col * (uint64_t)(V + 1) + (uint64_t)id)));
      if (y > rs.yb || (y == rs.yb && id < rs.ib)) { rs.yb = y; rs.ib = id; }
      if (id == dn) rs.xd = x;
      else if (y > rs.yx || (y == rs.yx && id < rs.ix)) { rs.yx = y; rs.ix = id; }
    } else {
      if (v > bv || (v == bv && id < bi)) { bv = v; bi = id; }
    }
  };
  if (KT % WPU == 0 && (KT / WPU) % D == 0) {
    // row tiles handed out at run time (workgroups b and b + nwg first, then
    // tickets), the 8 waves of a workgroup on one tile's k slices: workgroups
    // on faster XCDs take more tiles and the last tiles spread over the grid;
    // the rows are normalised while the first tile is on its way
    int* seq = reinterpret_cast<int*>(misc + 230);
    run_stream_dyn<HF, false, D, SPLIT>(RT, KT, T, src, epi, red, a.dummy, a.tickets, seq, NoDone(), stage);
  } else {
    stage();
    stream_units_wave<HF, false>(u0, u1, KT, T, src, epi, a.dummy);
  }
  if constexpr (SAMPLE) {
    head_sample_tail(a, rs, key, smem + 8 * XS * 2, misc);
    return;
  }
  // workgroup best per row: every thread holds a candidate for column lane % 16
  // (the four lanes of a wave that hold a column, then the 8 waves through LDS)
  float* cv = reinterpret_cast<float*>(smem + 8 * XS * 2);
  int* ci = reinterpret_cast<int*>(cv + kThreads);
  auto best_of = [](float& v, int& id, float ov, int oi) {
    if (ov > v || (ov == v && oi < id)) { v = ov; id = oi; }
  };
  best_of(bv, bi, __shfl_xor(bv, 16), __shfl_xor(bi, 16));
  best_of(bv, bi, __shfl_xor(bv, 32), __shfl_xor(bi, 32));
  if (lane < 16) {
    cv[w * 16 + lane] = bv;
    ci[w * 16 + lane] = bi;
  }
  __syncthreads();
  if (threadIdx.x < T) {
    float v = -INFINITY;
    int id = 0x7fffffff;
    for (int r = 0; r < kWaves; ++r) best_of(v, id, cv[r * 16 + threadIdx.x], ci[r * 16 + threadIdx.x]);
    // agent-scope stores pass this XCD's L2, so the merging workgroup (on any
    // XCD) reads them from memory once the store has completed (waited for
    // below) -- no write-back of the whole L2
    __hip_atomic_store(a.best_val + blockIdx.x * 8 + threadIdx.x, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.best_idx + blockIdx.x * 8 + threadIdx.x, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the last workgroup to finish reduces over the grid and verifies the drafts
  wg_release_begin();
  int* flag = reinterpret_cast<int*>(misc + 250);
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == gridDim.x - 1;
    if (last) {
      // every workgroup has left its stream: the counters start the next launch at zero
      __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int c = 0; c < 8; ++c)
        __hip_atomic_store(a.tickets + kCntStride * c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  // grid-wide best per row: thread x takes column x % 8 of workgroups
  // x / 8, x / 8 + 64, ... (its loads issued together), then the 64 partial
  // bests of a column are merged (shuffles, then LDS).  The result does not
  // depend on the order (largest logit, lowest row id among equal ones).
  int* am = reinterpret_cast<int*>(misc + 200);
  int* tk = reinterpret_cast<int*>(misc + 208);
  {
    const int t = threadIdx.x & 7, b0 = threadIdx.x >> 3;
    float v = -INFINITY;
    int id = 0x7fffffff;
    if (t < T) {
      for (int bb = b0; bb < (int)gridDim.x; bb += 64 * kHeadMergeB) {
        float ov[kHeadMergeB];
        int oi[kHeadMergeB];
#pragma unroll
        for (int i = 0; i < kHeadMergeB; ++i) {
          const int b = min(bb + 64 * i, (int)gridDim.x - 1);
          ov[i] = __hip_atomic_load(a.best_val + b * 8 + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          oi[i] = __hip_atomic_load(a.best_idx + b * 8 + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < kHeadMergeB; ++i) best_of(v, id, ov[i], oi[i]);
      }
    }
    // the eight lanes of a wave that hold a row, then the 8 waves (LDS)
    best_of(v, id, __shfl_xor(v, 8), __shfl_xor(id, 8));
    best_of(v, id, __shfl_xor(v, 16), __shfl_xor(id, 16));
    best_of(v, id, __shfl_xor(v, 32), __shfl_xor(id, 32));
    if (lane < 8) {
      cv[w * 8 + lane] = v;
      ci[w * 8 + lane] = id;
    }
    if ((int)threadIdx.x < T) tk[threadIdx.x] = a.tokens[threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x < T) {
    float v = -INFINITY;
    int id = 0x7fffffff;
    for (int r = 0; r < kWaves; ++r) best_of(v, id, cv[r * 8 + threadIdx.x], ci[r * 8 + threadIdx.x]);
    am[threadIdx.x] = id;
    a.argmax[threadIdx.x] = id;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n + 1 <= T - 1 && tk[n + 1] == am[n]) ++n;
    a.committed[0] = n + 1;
    for (int i = 1; i <= n; ++i) a.committed[i] = tk[i];
    a.committed[n + 1] = am[n];
    if (a.kv_len) a.kv_len[0] += n + 1;
    a.tokens[0] = am[n];
    if (a.next_drafts)
      for (int i = 1; i < T; ++i) a.tokens[i] = a.next_drafts[i - 1];
  }
}

typedef void (*HeadKernelFn)(HeadArgs);
static HeadKernelFn head_kernel_for(int head_fmt, bool sample) {
  if (head_fmt == MK_FMT_FP8_B128)
    return sample ? head_kernel<MK_FMT_FP8_B128, true> : head_kernel<MK_FMT_FP8_B128, false>;
  return sample ? head_kernel<MK_FMT_BF16, true> : head_kernel<MK_FMT_BF16, false>;
}

int head_kernel_occupancy(int* wgs_per_cu) {
  int least = 1 << 30;
  for (int f : {MK_FMT_BF16, MK_FMT_FP8_B128})
    for (bool smp : {false, true}) {
      const void* fn = (const void*)head_kernel_for(f, smp);
      hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kHeadLds);
      if (e != hipSuccess) return (int)e;
      int occ = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)fn, kThreads, kHeadLds);
      if (e != hipSuccess) return (int)e;
      least = occ < least ? occ : least;
    }
  *wgs_per_cu = least;
  return 0;
}

int launch_head(const HeadLaunch& h, int T, float* logits, int32_t* tokens, const int32_t* next_drafts,
                int32_t* argmax, int32_t* committed, hipStream_t s) {
  HeadArgs a{(const uint8_t*)h.head_packed, h.V, h.d, h.gamma, h.eps, h.hidden, T, logits, h.best_val,
             h.best_idx, h.counter, tokens, next_drafts, argmax, committed, h.kv_len, h.dummy, h.fault, h.tickets,
             h.scales, h.temperature > 0.f ? 1.0f / h.temperature : 0.f, h.seed, h.step, h.part};
  hipLaunchKernelGGL(head_kernel_for(h.head_fmt, h.temperature > 0.f), dim3(h.nwg), dim3(kThreads), kHeadLds, s, a);
  return (int)hipGetLastError();
}

}  // namespace mk
