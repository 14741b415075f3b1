// Stack pieces around the layer kernel: embedding gather, and one launch that
// does the final RMSNorm, the LM-head projection, the argmax per verify row
// and greedy acceptance of the drafts (the lm_head and rejection-kernel rows of
// the per-step kernel table in "Why one GB300 doesn't beat 4x RTX PRO 6000 at
// single-stream decode", section "Where the 11.2 ms goes"; greedy decoding as
// the engine gate uses it, "DeepSeek-V4.1-Flash breaks 1,000 tokens per second
// for one user", section "The safety layer").
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
};

constexpr int kHeadLds = 8 * (8192 + kXPad) * 2 + 2 * kWaves * 64 * 4 * 4 + 1024;
constexpr int kHeadNormB = 16;           // float4 loads per lane in flight while normalising a row
constexpr int kHeadMergeB = 4;           // per-workgroup bests loaded together per thread in the grid merge

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
  const int RT = a.V / 16, KT = d / 32;
  const long long U = RT;
  const int u0 = (int)(U * blockIdx.x / gridDim.x), u1 = (int)(U * (blockIdx.x + 1) / gridDim.x);
  const int j = lane & 15, g = lane >> 4;
  const __bf16* bl = xs + (j < T ? j : T - 1) * XS + g * 8;
  struct Src {
    const uint8_t* head; int KT; const __bf16* bl;
    __device__ const uint8_t* base(int u) const { return head + (long long)u * KT * 1024; }
    __device__ const __bf16* bbase(int) const { return bl; }
    __device__ const float* sbase(int) const { return nullptr; }
    __device__ const float* sbase2(int) const { return nullptr; }
  } src{a.head, KT, bl};
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  float* logits = a.logits;
  const int V = a.V;
  auto epi = [&](int u, int row, int col, float v, float) {
    const int id = u * 16 + row;
    if (logits) logits[(long long)col * V + id] = v;
    if (v > bv || (v == bv && id < bi)) { bv = v; bi = id; }
  };
  if (KT % kWaves == 0 && (KT / kWaves) % 16 == 0) {
    // row tiles handed out at run time (workgroups b and b + nwg first, then
    // tickets), the 8 waves of a workgroup on one tile's k slices: workgroups
    // on faster XCDs take more tiles and the last tiles spread over the grid;
    // the rows are normalised while the first tile is on its way
    int* seq = reinterpret_cast<int*>(misc + 230);
    run_stream_dyn<MK_FMT_BF16, false, 16>(RT, KT, T, src, epi, red, a.dummy, a.tickets, seq, NoDone(), stage);
  } else {
    stage();
    stream_units_wave<MK_FMT_BF16, false>(u0, u1, KT, T, src, epi, a.dummy);
  }
  // workgroup best per row: every thread holds a candidate for column lane % 16
  float* cv = reinterpret_cast<float*>(smem + 8 * XS * 2);
  int* ci = reinterpret_cast<int*>(cv + kThreads);
  cv[threadIdx.x] = bv;
  ci[threadIdx.x] = bi;
  __syncthreads();
  if (threadIdx.x < T) {
    float v = -INFINITY;
    int id = 0x7fffffff;
    for (int r = 0; r < kThreads / 16; ++r) {
      const float ov = cv[r * 16 + threadIdx.x];
      const int oi = ci[r * 16 + threadIdx.x];
      if (ov > v || (ov == v && oi < id)) { v = ov; id = oi; }
    }
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
  // bests of a column are merged in LDS.  The result does not depend on the
  // order (largest logit, lowest row id among equal ones).
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
        for (int i = 0; i < kHeadMergeB; ++i)
          if (ov[i] > v || (ov[i] == v && oi[i] < id)) { v = ov[i]; id = oi[i]; }
      }
    }
    cv[threadIdx.x] = v;
    ci[threadIdx.x] = id;
    if ((int)threadIdx.x < T) tk[threadIdx.x] = a.tokens[threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x < T) {
    float v = -INFINITY;
    int id = 0x7fffffff;
    for (int r = 0; r < kThreads / 8; ++r) {
      const float ov = cv[r * 8 + threadIdx.x];
      const int oi = ci[r * 8 + threadIdx.x];
      if (ov > v || (ov == v && oi < id)) { v = ov; id = oi; }
    }
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

int head_kernel_occupancy(int* wgs_per_cu) {
  hipError_t e = hipFuncSetAttribute((const void*)head_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kHeadLds);
  if (e != hipSuccess) return (int)e;
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(wgs_per_cu, head_kernel, kThreads, kHeadLds);
}

int launch_head(const void* head_packed, int V, int d, const float* gamma, float eps, const float* h, int T,
                float* logits, float* best_val, int32_t* best_idx, uint32_t* counter, uint32_t* tickets,
                int32_t* tokens, const int32_t* next_drafts, int32_t* argmax, int32_t* committed, int32_t* kv_len,
                const uint8_t* dummy, const uint32_t* fault, int nwg, hipStream_t s) {
  HeadArgs a{(const uint8_t*)head_packed, V, d, gamma, eps, h, T, logits, best_val, best_idx, counter, tokens,
             next_drafts, argmax, committed, kv_len, dummy, fault, tickets};
  hipLaunchKernelGGL(head_kernel, dim3(nwg), dim3(kThreads), kHeadLds, s, a);
  return (int)hipGetLastError();
}

}  // namespace mk
