// Host-side entry points into the kernel translation units.
#pragma once
#include "mk_common.h"

namespace mk {

typedef void (*LayerKernelFn)(LayerParams);
// The kernel instance for a layer's formats and dimensions (null if none).
// s_q is the schedule's split-K factor of the projection and nwg its grid size
// (0: not known yet; an instance is returned whenever one exists for some
// factor and grid).
LayerKernelFn layer_kernel_for(int af, int ef, int kf, int d, int nh, int dh, int dc, int dr, int E, int topk,
                               int nshared, int f, int s_q, int nwg);
// The instance for a layer with sparse attention (null if none).
// spec: the 384-expert layer's dimensions (fixed-shape instances for fp8 experts).
LayerKernelFn layer_kernel_sparse_for(int af, int ef, int kf, bool lowrank, bool spec);
// The instance for a layer with a low-rank query (null if none); arguments as above.
LayerKernelFn layer_kernel_lowrank_for(int af, int ef, int kf, int d, int nh, int dh, int dc, int dr, int E, int topk,
                                       int nshared, int f, int s_q, int nwg);

int launch_pack(const void* src, int fmt, int nb, int R, int K, long long sb, long long sr, long long sk,
                void* dst, long long dst_stride, long long dst_off, hipStream_t stream);

int launch_pack_mx_scales(const void* src, int R, int K, void* dst, long long tile_stride, long long dst_off,
                          hipStream_t stream);

int launch_embed(const uint16_t* emb, int V, int d, const int32_t* tokens, int T, float* h, uint32_t* fault,
                 hipStream_t s);
// Everything the head launch takes that does not change from step to step.
struct HeadLaunch {
  const void* head_packed; int head_fmt; const float* scales;   // scales: fp8 head only
  int V, d; const float* gamma; float eps; const float* hidden;
  float* best_val; int32_t* best_idx; uint32_t* counter; uint32_t* tickets; int32_t* kv_len;
  const uint8_t* dummy; const uint32_t* fault; int nwg;
  float temperature; uint64_t seed; uint32_t* step; float* part;   // temperature 0: greedy
};
int launch_head(const HeadLaunch& h, int T, float* logits, int32_t* tokens, const int32_t* next_drafts,
                int32_t* argmax, int32_t* committed, hipStream_t s);
int head_kernel_occupancy(int* wgs_per_cu);

}  // namespace mk
