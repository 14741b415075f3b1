// The C ABI (include/mk.h): validation, sizing, packing launches, layer and
// stack set-up, step launches.  No device memory is allocated here: every
// buffer is the caller's.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "mk_common.h"
#include "mk_host.h"

using namespace mk;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_OK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(MK_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Dims {
  int d, nh, dh, dc, dr, qw, kvw, nq, E, topk, nshared, f;
  int af, ef, kf;
  int ql, kvn;       // low-rank query rank (0: one W_Q), latent norm
  int ih, idm, ik, imax;   // sparse attention: indexer heads, key dim, rows kept, largest L + T
  int kvmax;               // the largest L + T the caller expects (0: not stated)
  // long contexts may take the four-tile attention units (their partials are sized for it)
  bool att_share() const { return kf == MK_FMT_BF16 && dc == 512 && dr == 64 && ik == 0 && kvmax >= 16384; }
  int nqp() const { return ql > 0 ? ql : nq; }   // rows of the first projection's query part
  int nidx() const { return ik > 0 ? ih * idm + ih + idm : 0; }   // indexer rows of the first projection
  int kvrow() const { return kvw + (ik > 0 ? idm : 0); }           // values per cache row
};

// s_q: the projection's split-K factor of the schedule (0 when not known yet).
LayerKernelFn kernel_of(const Dims& D, int s_q = 0, int nwg = 0) {
  if (D.ik > 0) {
    const bool spec = D.d == 4096 && D.nh == 32 && D.dh == 128 && D.dc == 512 && D.dr == 64 && D.E == 384 &&
                      D.topk == 8 && D.nshared == 1 && D.f == 2048 && (s_q == 0 || s_q == 1) &&
                      (nwg == 0 || nwg >= kSpecMinGrid);
    return layer_kernel_sparse_for(D.af, D.ef, D.kf, D.ql > 0, spec);
  }
  if (D.ql > 0)
    return layer_kernel_lowrank_for(D.af, D.ef, D.kf, D.d, D.nh, D.dh, D.dc, D.dr, D.E, D.topk, D.nshared, D.f, s_q,
                                    nwg);
  return layer_kernel_for(D.af, D.ef, D.kf, D.d, D.nh, D.dh, D.dc, D.dr, D.E, D.topk, D.nshared, D.f, s_q, nwg);
}

Dims dims_of(const mk_layer_config* c) {
  Dims D;
  D.d = c->d_model; D.nh = c->n_heads; D.dh = c->d_head; D.dc = c->d_latent; D.dr = c->d_rope;
  D.qw = D.dh + D.dr; D.kvw = D.dc + D.dr; D.nq = D.nh * D.qw; D.E = c->n_experts; D.topk = c->top_k;
  D.nshared = c->n_shared; D.f = c->d_ff; D.af = c->attn_format; D.ef = c->expert_format; D.kf = c->kv_format;
  D.ql = c->q_lora_rank; D.kvn = c->kv_norm;
  D.ih = c->idx_heads; D.idm = c->idx_dim; D.ik = c->idx_topk; D.imax = c->idx_max_rows;
  D.kvmax = c->kv_max_rows;
  return D;
}

int check_cfg(const mk_layer_config* c) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "null config");
  if (c->abi_version != MK_ABI_VERSION)
    return fail(MK_ERR_ABI_MISMATCH, "config abi_version %d, library %d", c->abi_version, MK_ABI_VERSION);
  const Dims D = dims_of(c);
  if (D.d <= 0 || D.nh <= 0 || D.dh <= 0 || D.dc <= 0 || D.dr <= 0 || D.E <= 0 || D.topk <= 0 || D.f <= 0)
    return fail(MK_ERR_INVALID_ARG, "non-positive dimension");
  if (D.af < 0 || D.af > 1 || D.ef < 0 || D.ef > 3 || !(D.kf == MK_FMT_F32 || D.kf == MK_FMT_BF16 || D.kf == MK_FMT_FP8_ROW))
    return fail(MK_ERR_INVALID_ARG, "unknown format");
  if (c->has_router_bias != 0 && c->has_router_bias != 1) return fail(MK_ERR_INVALID_ARG, "has_router_bias must be 0 or 1");
  if (D.ql < 0 || (D.kvn != 0 && D.kvn != 1)) return fail(MK_ERR_INVALID_ARG, "q_lora_rank must be >= 0 and kv_norm 0 or 1");
  if (D.ql > 0 && (D.af != MK_FMT_BF16 || D.ql % 32 || D.ql > D.d))
    return fail(MK_ERR_UNSUPPORTED_SHAPE, "a low-rank query needs bf16 attention and a rank that is a multiple of 32, <= d_model");
  if (D.kvn && D.ql == 0) return fail(MK_ERR_UNSUPPORTED_SHAPE, "the latent norm is built with the low-rank query only");
  if (D.kvmax < 0) return fail(MK_ERR_INVALID_ARG, "kv_max_rows must be >= 0");
  if (D.ik < 0) return fail(MK_ERR_INVALID_ARG, "idx_topk must be >= 0");
  if (D.ik > 0) {
    if (D.af != MK_FMT_BF16 || (D.kf != MK_FMT_BF16 && D.kf != MK_FMT_FP8_ROW))
      return fail(MK_ERR_UNSUPPORTED_SHAPE, "sparse attention needs bf16 attention and a bf16 or fp8 cache");
    if (D.nh % 16 || D.ih <= 0 || D.ih % 16 || D.idm <= 0 || D.idm % 32 || D.ih * D.idm > 8192 || D.ik > 8192)
      return fail(MK_ERR_UNSUPPORTED_SHAPE, "sparse attention: n_heads and idx_heads multiples of 16, idx_dim a "
                                            "multiple of 32, idx_heads * idx_dim <= 8192, idx_topk <= 8192");
    if (D.imax < 8 || D.imax > (1 << 24) || D.imax % 8)
      return fail(MK_ERR_INVALID_ARG, "idx_max_rows must be a multiple of 8 in [8, 2^24]");
    // the index-score phase holds a row's index queries in 16 fragments per lane and
    // stages 512 index keys (bf16, 8 pad each) and the head weights in LDS
    if (D.idm > 128) return fail(MK_ERR_UNSUPPORTED_SHAPE, "idx_dim must be <= 128");
  }
  // the one-wave-per-row cache writer (fp8 cache, low-rank variant) forms one key RoPE pair per lane
  if ((D.kf == MK_FMT_FP8_ROW || D.ql > 0) && D.dr > 128)
    return fail(MK_ERR_UNSUPPORTED_SHAPE, "d_rope must be <= 128 with an fp8 cache or a low-rank query");
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f)) return fail(MK_ERR_INVALID_ARG, "bad eps or rope base");
  const bool f32 = D.af == MK_FMT_F32 && D.ef == MK_FMT_F32 && D.kf == MK_FMT_F32;
  const bool bf = D.af == MK_FMT_BF16 && (D.kf == MK_FMT_BF16 || D.kf == MK_FMT_FP8_ROW) &&
                  (D.ef == MK_FMT_BF16 || D.ef == MK_FMT_FP8_B128 || D.ef == MK_FMT_MXFP4);
  if (!f32 && !bf)
    return fail(MK_ERR_UNSUPPORTED_SHAPE,
                "formats must be all F32, or BF16 attention with a BF16 or FP8_ROW cache and BF16, FP8_B128 or MXFP4 experts");
  if (D.d % 128 || D.f % 128) return fail(MK_ERR_UNSUPPORTED_SHAPE, "d_model and d_ff must be multiples of 128");
  if (D.dh % 32 || D.dc % 32 || D.dr % 32) return fail(MK_ERR_UNSUPPORTED_SHAPE, "d_head, d_latent, d_rope must be multiples of 32");
  if (D.E % 16) return fail(MK_ERR_UNSUPPORTED_SHAPE, "n_experts must be a multiple of 16");
  if ((kMaxT * D.nh + 15) / 16 > 64) return fail(MK_ERR_UNSUPPORTED_SHAPE, "n_heads must be <= 128");
  if (D.dh > 16 * kWaves) return fail(MK_ERR_UNSUPPORTED_SHAPE, "d_head must be <= %d", 16 * kWaves);
  if (D.E > kMaxExperts) return fail(MK_ERR_UNSUPPORTED_SHAPE, "n_experts must be <= %d", kMaxExperts);
  if (D.topk > kMaxTopK || D.topk > D.E) return fail(MK_ERR_UNSUPPORTED_SHAPE, "top_k must be <= 16 and <= n_experts");
  if (D.nshared < 0 || D.nshared > 1) return fail(MK_ERR_UNSUPPORTED_SHAPE, "n_shared must be 0 or 1");
  if (f32 && (D.kvw > 160 || D.dc > 128)) return fail(MK_ERR_UNSUPPORTED_SHAPE, "fp32 layers: d_latent <= 128, d_latent + d_rope <= 160");
  if (bf && (D.kvw > 576 || D.dc > 512)) return fail(MK_ERR_UNSUPPORTED_SHAPE, "bf16 layers: d_latent <= 512, d_latent + d_rope <= 576");
  const int es = f32 ? 4 : 2;
  const int dmax = std::max(D.d, std::max(D.nh * D.dh, D.f));
  if (dmax > kMaxStageK)
    return fail(MK_ERR_UNSUPPORTED_SHAPE, "d_model, n_heads*d_head and d_ff must be <= %d", kMaxStageK);
  if (D.d > kMaxModel) return fail(MK_ERR_UNSUPPORTED_SHAPE, "d_model must be <= %d", kMaxModel);
  const long long xb = align256((size_t)kMaxT * (dmax + kXPad) * es);
  const long long lds_router = 2 * xb + 2 * kWaves * 64 * 4 * 4 + 4LL * kMaxT * 16 * 4;
  const long long lds_route = xb + 32768 + (long long)kMaxT * D.E * 4 + 3 * kMaxT * kMaxTopK * 4 +
                              (kMaxT * kMaxTopK + 8) * 4 + (long long)D.E * 4 + 16 + (kMaxT * kMaxTopK + 8) * 8;
  // attention: per-wave value slices (half the latent, key-dim blocks of 16 fp32
  // or 32 bf16 dims), the query tile, two rounds of score halves; then the
  // merge of the four wave pairs
  const int kbw = f32 ? 16 : 32, la = (D.dc / kbw + 1) / 2;
  const long long lds_att =
      std::max(((long long)kWaves * 16 * (la * kbw + 8) * es + 16LL * (D.kvw + 8) * es + 15) / 16 * 16 +
                   2LL * kWaves * 64 * 16,
               4LL * 16 * D.dc * 4 + 8 * 64 * 2 * 4);
  const long long lim = kLdsBytes - 1024;
  // the down projection stages two experts' activations below the routing tables
  if (2LL * kMaxT * (D.f + kXPad) * es > xb + 32768)
    return fail(MK_ERR_UNSUPPORTED_SHAPE, "d_ff too large for the LDS plan");
  if (lds_router > lim || lds_route > lim || lds_att > lim)
    return fail(MK_ERR_UNSUPPORTED_SHAPE, "shape exceeds the LDS plan (router %lld, route %lld, attention %lld > %lld bytes)",
                lds_router, lds_route, lds_att, lim);
  if (!kernel_of(D)) return fail(MK_ERR_UNSUPPORTED_SHAPE, "no kernel for this shape");
  return MK_OK;
}

// packed sizes
long long tiles_bytes(int R, int K, int fmt) { return (long long)((R + 15) / 16) * ((K + tile_k(fmt) - 1) / tile_k(fmt)) * 1024; }
long long exp_w13(const Dims& D) { return 2 * tiles_bytes(D.f, D.d, D.ef); }
long long exp_w2(const Dims& D) { return tiles_bytes(D.d, D.f, D.ef); }
long long exp_scales(const Dims& D) {
  if (D.ef == MK_FMT_MXFP4) return align256((size_t)(3LL * D.f * D.d / 32));   // one byte per 32 elements
  if (D.ef != MK_FMT_FP8_B128) return 0;
  const long long a = (long long)((D.f + 127) / 128) * ((D.d + 127) / 128);
  return align256((size_t)(3 * a * 4));
}

int packed_bytes(const mk_layer_config* c, int tensor, size_t* out) {
  const Dims D = dims_of(c);
  long long b = 0;
  switch (tensor) {
    case MK_T_WQ: b = tiles_bytes(D.nq, D.d, D.af); break;
    case MK_T_WDKV: b = tiles_bytes(D.kvw, D.d, D.af); break;
    case MK_T_WUK: b = (long long)D.nh * tiles_bytes(D.dc, D.dh, D.af); break;
    case MK_T_WUV: b = (long long)D.nh * tiles_bytes(D.dh, D.dc, D.af); break;
    case MK_T_WO: b = tiles_bytes(D.d, D.nh * D.dh, D.af); break;
    case MK_T_WR: b = tiles_bytes(D.E, D.d, D.af); break;
    case MK_T_EXPERT: b = exp_w13(D) + exp_w2(D) + exp_scales(D); break;
    case MK_T_WDQ:
    case MK_T_WUQ:
      if (D.ql == 0) return fail(MK_ERR_INVALID_ARG, "W_DQ / W_UQ need q_lora_rank > 0");
      b = tensor == MK_T_WDQ ? tiles_bytes(D.ql, D.d, D.af) : tiles_bytes(D.nq, D.ql, D.af);
      break;
    case MK_T_WIDX:
      if (D.ik == 0) return fail(MK_ERR_INVALID_ARG, "the indexer's weights need idx_topk > 0");
      b = tiles_bytes(D.nidx(), D.d, D.af);
      break;
    default: return fail(MK_ERR_INVALID_ARG, "unknown tensor id %d", tensor);
  }
  *out = (size_t)b;
  return MK_OK;
}

// Choose the k-split S (a divisor of KT leaving >= 2 tiles per wave per unit)
// that minimises the busiest workgroup's time: units x (tile slots per wave +
// a fixed per-unit cost of about two tile slots for the reduction).
int choose_split(int RT, int KT, int nwg) {
  int best = 1;
  long long best_cost = -1;
  for (int S = 1; S <= KT; ++S) {
    if (KT % S) continue;
    const int NT = KT / S;
    if (NT < 2 * kWaves && S > 1) break;
    const long long U = (long long)RT * S;
    const long long cost = ((U + nwg - 1) / nwg) * ((NT + kWaves - 1) / kWaves + 2);
    if (best_cost < 0 || cost < best_cost) { best = S; best_cost = cost; }
  }
  return best;
}

struct DevInfo {
  int cus = 0, wgs_per_cu = 0, nwg = 0;
  bool gfx950 = false;
  char name[64] = {0};
  long long mem = 0;
};

int device_info(int dev, DevInfo* di, LayerKernelFn fn) {
  hipDeviceProp_t prop;
  HIP_OK(hipGetDeviceProperties(&prop, dev));
  di->cus = prop.multiProcessorCount;
  di->mem = (long long)prop.totalGlobalMem;
  std::strncpy(di->name, prop.gcnArchName, sizeof(di->name) - 1);
  di->gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (!di->gfx950) return fail(MK_ERR_UNSUPPORTED_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  if (fn) {
    int cur = 0;
    HIP_OK(hipGetDevice(&cur));
    HIP_OK(hipSetDevice(dev));
    HIP_OK(hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes));
    int n = 0;
    HIP_OK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, kLdsBytes));
    HIP_OK(hipSetDevice(cur));
    di->wgs_per_cu = n;
    if (n < 1) return fail(MK_ERR_NOT_CORESIDENT, "layer kernel cannot be resident (occupancy %d)", n);
    di->nwg = di->cus;   // one workgroup per compute unit
    if (di->nwg > kBarGroup * kMaxBarGroups)
      return fail(MK_ERR_UNSUPPORTED_DEVICE, "%d compute units exceed the barrier's %d workgroups", di->nwg,
                  kBarGroup * kMaxBarGroups);
  }
  return MK_OK;
}

struct WsLayout {
  size_t qkv_part, qrope, qabs, att_part, att_ml, z, o, hp, route_sel, route_gate, route_cand, logits, hbuf,
      ybuf, dummy, qbuf, iq, iw, iscore, ik16, isel, ihist, ictr, icnt, icand,
      total;
};
struct StLayout {
  size_t bar, att_cnt, experts, trace, total;
};

WsLayout ws_layout(const Dims& D, const Schedule& s) {
  WsLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const int T = kMaxT;
  const int nqt = (T * D.nh + 15) / 16;
  // attention partials: one per (query tile, key split); four-tile units take
  // grid / ceil(tiles / 4) splits, so up to four partials per workgroup
  const int units = D.att_share() ? 4 * s.nwg + nqt : std::max(s.nwg, nqt);
  const int slots = std::min(D.E, T * D.topk) + D.nshared;
  w.qkv_part = take((size_t)s.s_q * T * (D.nqp() + D.kvw + D.nidx()) * 4);
  w.qrope = take((size_t)T * D.nh * D.dr * 4);
  w.qabs = take((size_t)T * D.nh * D.dc * 4);
  w.att_part = take((size_t)units * 16 * D.dc * 4);
  w.att_ml = take((size_t)units * 16 * 2 * 4);
  w.z = take((size_t)T * D.nh * D.dc * 4);
  w.o = take((size_t)T * D.nh * D.dh * 4);
  w.hp = take((size_t)T * D.d * 4);
  w.route_sel = take((size_t)T * kMaxTopK * 4);
  w.route_gate = take((size_t)T * kMaxTopK * 4);
  w.route_cand = take((size_t)2 * T * (D.E / 16) * 16 * 4);
  w.logits = take((size_t)T * D.E * 4);
  w.hbuf = take((size_t)slots * T * D.f * 4);
  w.ybuf = take((size_t)slots * T * D.d * 4);
  w.dummy = take(32768);
  w.qbuf = D.ql > 0 ? take((size_t)T * D.nq * 4) : 0;
  w.iq = D.ik > 0 ? take((size_t)T * D.ih * D.idm * 2) : 0;
  w.iw = D.ik > 0 ? take((size_t)T * D.ih * 4) : 0;
  w.iscore = D.ik > 0 ? take((size_t)T * D.imax * 4) : 0;
  w.ik16 = D.ik > 0 ? take((size_t)T * D.imax * 2) : 0;
  w.ihist = D.ik > 0 ? take((size_t)T * 2048 * 4) : 0;
  w.ictr = D.ik > 0 ? take((size_t)T * kIdxCtrStride * 4) : 0;
  w.icnt = D.ik > 0 ? take((size_t)T * kThreads * 4) : 0;
  w.icand = D.ik > 0 ? take((size_t)T * D.imax * 8) : 0;
  w.isel = D.ik > 0 ? take((size_t)T * D.ik * 4) : 0;
  w.total = off;
  return w;
}

StLayout st_layout(const Dims& D, const Schedule& s) {
  StLayout l;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  l.bar = take(sizeof(BarrierState));
  l.att_cnt = take(kCntWords * 4);
  l.experts = take((size_t)(D.E + D.nshared) * 8);
  l.trace = take((size_t)s.nwg * kTraceStride * 8);
  l.total = off;
  return l;
}

// Points the workspace fields of `p` into the workspace at `ws` (layout `wl`).
void bind_workspace(LayerParams& p, const WsLayout& wl, char* ws) {
  p.qkv_part = (float*)(ws + wl.qkv_part);
  p.qrope = (float*)(ws + wl.qrope);
  p.qabs = (float*)(ws + wl.qabs);
  p.att_part = (float*)(ws + wl.att_part);
  p.att_ml = (float*)(ws + wl.att_ml);
  p.z = (float*)(ws + wl.z);
  p.o = (float*)(ws + wl.o);
  p.hp = (float*)(ws + wl.hp);
  p.route_sel = (int32_t*)(ws + wl.route_sel);
  p.route_gate = (float*)(ws + wl.route_gate);
  p.route_cand = (float*)(ws + wl.route_cand);
  p.logits = (float*)(ws + wl.logits);
  p.hbuf = (float*)(ws + wl.hbuf);
  p.ybuf = (float*)(ws + wl.ybuf);
  p.dummy = (const uint8_t*)(ws + wl.dummy);
  p.qbuf = wl.qbuf ? (float*)(ws + wl.qbuf) : nullptr;
  p.iq = wl.iq ? (void*)(ws + wl.iq) : nullptr;
  p.iw = wl.iw ? (float*)(ws + wl.iw) : nullptr;
  p.iscore = wl.iscore ? (float*)(ws + wl.iscore) : nullptr;
  p.ik16 = wl.ik16 ? (uint16_t*)(ws + wl.ik16) : nullptr;
  p.ihist = wl.ihist ? (uint32_t*)(ws + wl.ihist) : nullptr;
  p.ictr = wl.ictr ? (uint32_t*)(ws + wl.ictr) : nullptr;
  p.icnt = wl.icnt ? (uint32_t*)(ws + wl.icnt) : nullptr;
  p.icand = wl.icand ? (uint32_t*)(ws + wl.icand) : nullptr;
  p.isel = wl.isel ? (int32_t*)(ws + wl.isel) : nullptr;
}

// ------------------------------------------------------------------ static scratch
// The scratch of mk_decode_step_static: a file-scope device array that every
// GPU the library runs on holds until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device (hipGetSymbolAddress, with that device current,
// in mk_layer_init) and only that address is ever passed to a kernel.
constexpr size_t kStaticScratchBytes = MK_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];        // device address of `scratch` per device (null: not looked up)
hipError_t g_scratch_err[kMaxDevices];   // the lookup's result per device

// With `dev` current: looks up the device address of `scratch` once per device.
void scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev]) return;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  g_scratch_err[dev] = e;
  if (e == hipSuccess && ptr) g_scratch_ptr[dev] = (char*)ptr;
}

Schedule make_schedule(const Dims& D, int nwg) {
  Schedule s;
  s.nwg = nwg;
  s.grid_min = 0;
  const int KTa = D.d / tile_k(D.af);
  s.s_q = choose_split(D.nqp() / 16 + (D.kvw + 15) / 16 + D.nidx() / 16, KTa, nwg);
  return s;
}

}  // namespace

struct mk_layer {
  mk_layer_config cfg;
  Dims D;
  int dev;
  DevInfo di;
  Schedule sch;
  WsLayout wl;
  StLayout sl;
  char* state;
  char* ws;
  LayerKernelFn fn;
  LayerParams base;
  LayerParams last;    // the workspace pointers of the last launch (the debug taps read these)
  int trace_on;
  long long timeout_us;
  long long steps, launches;
  int last_T;
};

struct mk_model {
  mk_layer* const* layers_host;
  mk_layer** layers;
  int n_layers;
  const uint16_t* emb;
  const void* head;
  const float* gamma_f;
  int V;
  void** kv;
  int capacity;
  char* state;
  float* hidden;       // [2][kMaxT][d]
  int32_t* kv_len;
  uint32_t* fault;     // the stack's fault word
  float* hidden_rec;   // when set: [n_layers + 1][kMaxT][d], layer l reads slot l and writes slot l + 1
  float* best_val;
  int32_t* best_idx;
  uint32_t* counter;
  uint32_t* tickets;   // the head's ticket counters
  const uint8_t* dummy;
  int nwg_head;
  int head_fmt;              // MK_FMT_BF16 or MK_FMT_FP8_B128
  const float* head_scales;  // fp8 head: its block scales (inside the packed head)
  float temperature;         // 0: greedy verification
  uint64_t seed;             // sampled verification: draws keyed by (seed, step)
  uint32_t* step;            // sampled verification: device step counter
  float* part;               // sampled verification: per-workgroup row states
};

extern "C" {

int mk_abi_version(void) { return MK_ABI_VERSION; }
const char* mk_last_error(void) { return g_err.c_str(); }

int mk_query_device(int hip_device, mk_device_info* out) {
  if (!out) return fail(MK_ERR_INVALID_ARG, "null output");
  std::memset(out, 0, sizeof *out);
  int n = 0;
  HIP_OK(hipGetDeviceCount(&n));
  if (hip_device < 0 || hip_device >= n) return fail(MK_ERR_INVALID_ARG, "no HIP device %d", hip_device);
  DevInfo di;
  LayerKernelFn fn = layer_kernel_for(MK_FMT_BF16, MK_FMT_FP8_B128, MK_FMT_BF16, 4096, 32, 128, 512, 64, 384, 8, 1, 2048, 0, 0);
  hipDeviceProp_t prop;
  HIP_OK(hipGetDeviceProperties(&prop, hip_device));
  out->hip_device = hip_device;
  out->n_cus = prop.multiProcessorCount;
  out->hbm_bytes = (int64_t)prop.totalGlobalMem;
  std::strncpy(out->arch_name, prop.gcnArchName, sizeof(out->arch_name) - 1);
  int rc = device_info(hip_device, &di, fn);
  out->is_gfx950 = di.gfx950 ? 1 : 0;
  if (rc != MK_OK) return rc;
  out->wgs_per_cu = di.wgs_per_cu;
  out->grid_wgs = di.nwg;
  out->threads_per_wg = kThreads;
  out->lds_bytes_per_wg = kLdsBytes;
  return MK_OK;
}

int mk_check_config(const mk_layer_config* cfg) { return check_cfg(cfg); }

int mk_packed_bytes(const mk_layer_config* cfg, int tensor, size_t* bytes) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!bytes) return fail(MK_ERR_INVALID_ARG, "null output");
  return packed_bytes(cfg, tensor, bytes);
}

int mk_kv_bytes(const mk_layer_config* cfg, int32_t capacity, size_t* bytes) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!bytes || capacity < 0) return fail(MK_ERR_INVALID_ARG, "bad arguments");
  *bytes = (size_t)capacity * kv_row_bytes(cfg->kv_format, dims_of(cfg).kvrow());
  return MK_OK;
}

static int sizes_for(const mk_layer_config* cfg, int dev, WsLayout* wl, StLayout* sl) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  const Dims D = dims_of(cfg);
  DevInfo di;
  rc = device_info(dev, &di, kernel_of(D));
  if (rc) return rc;
  const Schedule s = make_schedule(D, di.nwg);
  if (wl) *wl = ws_layout(D, s);
  if (sl) *sl = st_layout(D, s);
  return MK_OK;
}

int mk_layer_state_bytes(const mk_layer_config* cfg, int hip_device, size_t* bytes) {
  if (!bytes) return fail(MK_ERR_INVALID_ARG, "null output");
  StLayout sl;
  int rc = sizes_for(cfg, hip_device, nullptr, &sl);
  if (rc) return rc;
  *bytes = sl.total;
  return MK_OK;
}

int mk_layer_workspace_bytes(const mk_layer_config* cfg, int hip_device, size_t* bytes) {
  if (!bytes) return fail(MK_ERR_INVALID_ARG, "null output");
  WsLayout wl;
  int rc = sizes_for(cfg, hip_device, &wl, nullptr);
  if (rc) return rc;
  *bytes = wl.total;
  return MK_OK;
}

int mk_pack_tensor(const mk_layer_config* cfg, int tensor, const void* src, void* dst, void* stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!src || !dst) return fail(MK_ERR_INVALID_ARG, "null tensor");
  const Dims D = dims_of(cfg);
  hipStream_t s = (hipStream_t)stream;
  const int f = D.af;
  switch (tensor) {
    case MK_T_WQ: rc = launch_pack(src, f, 1, D.nq, D.d, 0, D.d, 1, dst, 1024, 0, s); break;
    case MK_T_WDKV: rc = launch_pack(src, f, 1, D.kvw, D.d, 0, D.d, 1, dst, 1024, 0, s); break;
    // per head, rows m (d_latent) and columns e (d_head): element = W_UK[h][e][m]
    case MK_T_WUK: rc = launch_pack(src, f, D.nh, D.dc, D.dh, (long long)D.dh * D.dc, 1, D.dc, dst, 1024, 0, s); break;
    case MK_T_WUV: rc = launch_pack(src, f, D.nh, D.dh, D.dc, (long long)D.dh * D.dc, D.dc, 1, dst, 1024, 0, s); break;
    case MK_T_WO: rc = launch_pack(src, f, 1, D.d, D.nh * D.dh, 0, D.nh * D.dh, 1, dst, 1024, 0, s); break;
    case MK_T_WR: rc = launch_pack(src, f, 1, D.E, D.d, 0, D.d, 1, dst, 1024, 0, s); break;
    case MK_T_WDQ:
      if (D.ql == 0) return fail(MK_ERR_INVALID_ARG, "W_DQ needs q_lora_rank > 0");
      rc = launch_pack(src, f, 1, D.ql, D.d, 0, D.d, 1, dst, 1024, 0, s);
      break;
    case MK_T_WUQ:
      if (D.ql == 0) return fail(MK_ERR_INVALID_ARG, "W_UQ needs q_lora_rank > 0");
      rc = launch_pack(src, f, 1, D.nq, D.ql, 0, D.ql, 1, dst, 1024, 0, s);
      break;
    case MK_T_WIDX:
      if (D.ik == 0) return fail(MK_ERR_INVALID_ARG, "the indexer's weights need idx_topk > 0");
      rc = launch_pack(src, f, 1, D.nidx(), D.d, 0, D.d, 1, dst, 1024, 0, s);
      break;
    default: return fail(MK_ERR_INVALID_ARG, "tensor %d is not packed with mk_pack_tensor", tensor);
  }
  if (rc) return fail(MK_ERR_HIP, "pack launch failed: %s", hipGetErrorString((hipError_t)rc));
  return MK_OK;
}

int mk_pack_expert(const mk_layer_config* cfg, const void* w1, const void* w3, const void* w2, const float* s1,
                   const float* s3, const float* s2, void* dst, void* stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  const Dims D = dims_of(cfg);
  if (!w1 || !w3 || !w2 || !dst) return fail(MK_ERR_INVALID_ARG, "null tensor");
  const bool fp8 = D.ef == MK_FMT_FP8_B128, mx = D.ef == MK_FMT_MXFP4;
  if ((fp8 || mx) && (!s1 || !s3 || !s2)) return fail(MK_ERR_INVALID_ARG, "fp8 and MXFP4 experts need three scale arrays");
  hipStream_t s = (hipStream_t)stream;
  const long long w13 = exp_w13(D), w2b = exp_w2(D);
  // row strides in bytes for MXFP4 (two codes per byte), in elements otherwise
  const int rd = mx ? D.d / 2 : D.d, rf = mx ? D.f / 2 : D.f;
  rc = launch_pack(w1, D.ef, 1, D.f, D.d, 0, rd, 1, dst, 2048, 0, s);
  if (!rc) rc = launch_pack(w3, D.ef, 1, D.f, D.d, 0, rd, 1, dst, 2048, 1024, s);
  if (!rc) rc = launch_pack(w2, D.ef, 1, D.d, D.f, 0, rf, 1, dst, 1024, w13, s);
  if (!rc && mx) {
    const long long sc13 = w13 + w2b, sc2 = sc13 + (long long)(D.f / 16) * (D.d / 128) * 128;
    rc = launch_pack_mx_scales(s1, D.f, D.d, dst, 128, sc13, s);
    if (!rc) rc = launch_pack_mx_scales(s3, D.f, D.d, dst, 128, sc13 + 64, s);
    if (!rc) rc = launch_pack_mx_scales(s2, D.d, D.f, dst, 64, sc2, s);
  }
  if (rc) return fail(MK_ERR_HIP, "pack launch failed: %s", hipGetErrorString((hipError_t)rc));
  if (fp8) {
    const size_t a = (size_t)((D.f + 127) / 128) * ((D.d + 127) / 128) * 4;
    char* sc = (char*)dst + w13 + w2b;
    HIP_OK(hipMemcpyAsync(sc, s1, a, hipMemcpyDeviceToDevice, s));
    HIP_OK(hipMemcpyAsync(sc + a, s3, a, hipMemcpyDeviceToDevice, s));
    HIP_OK(hipMemcpyAsync(sc + 2 * a, s2, a, hipMemcpyDeviceToDevice, s));
  }
  return MK_OK;
}

int mk_layer_init(const mk_layer_config* cfg, const mk_layer_weights* w, void* state_dev, void* workspace_dev,
                  int hip_device, mk_layer** out) {
  if (!out) return fail(MK_ERR_INVALID_ARG, "null output");
  *out = nullptr;
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!w || !state_dev || !workspace_dev) return fail(MK_ERR_INVALID_ARG, "null weights, state or workspace");
  if (!w->gamma1 || !w->gamma2 || !w->wdkv || !w->wuk || !w->wuv || !w->wo || !w->wr || !w->experts)
    return fail(MK_ERR_INVALID_ARG, "null weight tensor");
  if (cfg->q_lora_rank > 0 ? (!w->wdq || !w->wuq || !w->gamma_q) : !w->wq)
    return fail(MK_ERR_INVALID_ARG, "null query projection (W_Q, or W_DQ, W_UQ and gamma_q with a low-rank query)");
  if (cfg->kv_norm && !w->gamma_kv) return fail(MK_ERR_INVALID_ARG, "kv_norm needs gamma_kv");
  if (cfg->idx_topk > 0 && !w->widx) return fail(MK_ERR_INVALID_ARG, "sparse attention needs the indexer's weights");
  if ((cfg->has_router_bias != 0) != (w->router_bias != nullptr))
    return fail(MK_ERR_INVALID_ARG, "router_bias must be given iff has_router_bias");
  const Dims D = dims_of(cfg);
  for (int e = 0; e < D.E + D.nshared; ++e)
    if (!w->experts[e]) return fail(MK_ERR_INVALID_ARG, "expert block %d is null", e);
  LayerKernelFn fn = kernel_of(D);
  DevInfo di;
  rc = device_info(hip_device, &di, fn);
  if (rc) return rc;
  if ((D.E / 16 + di.nwg - 1) / di.nwg > 4)
    return fail(MK_ERR_UNSUPPORTED_SHAPE, "n_experts / 16 exceeds 4 router units per workgroup on %d workgroups",
                di.nwg);
  if (D.ik > 0 && di.nwg < kMaxT)
    return fail(MK_ERR_UNSUPPORTED_SHAPE, "sparse attention needs at least %d workgroups (one per verify row)", kMaxT);
  mk_layer* L = new (std::nothrow) mk_layer();
  if (!L) return fail(MK_ERR_INVALID_ARG, "out of host memory");
  L->cfg = *cfg;
  L->D = D;
  L->dev = hip_device;
  L->di = di;
  L->sch = make_schedule(D, di.nwg);
  L->wl = ws_layout(D, L->sch);
  L->sl = st_layout(D, L->sch);
  L->state = (char*)state_dev;
  L->ws = (char*)workspace_dev;
  L->fn = kernel_of(D, L->sch.s_q, L->sch.nwg);   // the instance for this schedule (same occupancy)
  L->trace_on = 0;
  L->timeout_us = 2000000;
  L->steps = L->launches = 0;
  L->last_T = 0;
  int cur = 0;
  hipGetDevice(&cur);
  hipSetDevice(hip_device);
  hipError_t e1 = hipMemset(L->state, 0, L->sl.total);
  hipError_t e2 = hipMemcpy(L->state + L->sl.experts, w->experts, (size_t)(D.E + D.nshared) * 8, hipMemcpyHostToDevice);
  hipError_t e3 = hipDeviceSynchronize();
  scratch_setup(hip_device);
  hipSetDevice(cur);
  if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess) {
    delete L;
    return fail(MK_ERR_HIP, "state initialisation failed: %s", hipGetErrorString(e1 != hipSuccess ? e1 : (e2 != hipSuccess ? e2 : e3)));
  }
  LayerParams& p = L->base;
  std::memset(&p, 0, sizeof p);
  p.d = D.d; p.nh = D.nh; p.dh = D.dh; p.dc = D.dc; p.dr = D.dr; p.qw = D.qw; p.kvw = D.kvw; p.nq = D.nq;
  p.E = D.E; p.topk = D.topk; p.nshared = D.nshared; p.f = D.f;
  p.eps = cfg->rms_eps;
  p.scale = (float)(1.0 / std::sqrt((double)(D.dh + D.dr)));
  p.rope_base = (double)cfg->rope_base;
  p.rope_step = std::pow((double)cfg->rope_base, -2.0 / (double)D.dr);
  p.g1 = w->gamma1; p.g2 = w->gamma2;
  p.wq = (const uint8_t*)w->wq; p.wdkv = (const uint8_t*)w->wdkv; p.wuk = (const uint8_t*)w->wuk;
  p.wuv = (const uint8_t*)w->wuv; p.wo = (const uint8_t*)w->wo; p.wr = (const uint8_t*)w->wr;
  p.rbias = w->router_bias;
  p.ql = D.ql; p.kv_norm = D.kvn;
  p.wdq = (const uint8_t*)w->wdq; p.wuq = (const uint8_t*)w->wuq; p.gq = w->gamma_q; p.gkv = w->gamma_kv;
  p.ihead = D.ih; p.idim = D.idm; p.itopk = D.ik; p.imax = D.imax; p.kv_row = D.kvrow();
  p.att_share = D.att_share() ? 1 : 0;
  p.widx = (const uint8_t*)w->widx;
  p.experts = (const uint8_t* const*)(L->state + L->sl.experts);
  p.exp_w13_bytes = exp_w13(D);
  p.exp_w2_bytes = exp_w2(D);
  bind_workspace(p, L->wl, L->ws);
  p.bar = (BarrierState*)(L->state + L->sl.bar);
  p.att_cnt = (uint32_t*)(L->state + L->sl.att_cnt);
  p.trace = nullptr;
  // MI355X runs workgroup b of a launch on XCD b % 8 (checked by the kernel at every barrier)
  p.xcd_release = L->sch.nwg % 8 == 0 ? 1 : 0;
  p.sch = L->sch;
  L->last = p;
  *out = L;
  return MK_OK;
}

// ws: the workspace to use (null: the layer's own).
static int launch_layer(mk_layer* L, const float* hin, int T, void* kv_rows, int capacity, int length,
                        const int32_t* len_dev, float* hout, uint32_t* model_fault, hipStream_t s,
                        char* ws = nullptr) {
  LayerParams p = L->base;
  if (ws) bind_workspace(p, L->wl, ws);
  p.model_fault = model_fault;
  p.T = T;
  p.L = length;
  p.L_dev = len_dev;
  p.H = hin;
  p.out = hout;
  p.kv = kv_rows;
  p.kv_capacity = capacity;
  p.trace = L->trace_on ? (long long*)(L->state + L->sl.trace) : nullptr;
  p.timeout_ticks = L->timeout_us * 100;
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel((const void*)L->fn, dim3(L->sch.nwg), dim3(kThreads), args, kLdsBytes, s);
  if (e != hipSuccess) return fail(MK_ERR_HIP, "layer launch: %s", hipGetErrorString(e));
  L->steps++;
  L->launches++;
  L->last_T = T;
  L->last = p;
  return MK_OK;
}

int mk_decode_step(mk_layer* L, const float* hidden_in, int T, const mk_kv_cache* kv, float* hidden_out, void* stream) {
  if (!L || !hidden_in || !kv || !kv->rows || !hidden_out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (L->D.ik > 0 && (long long)kv->length + T > L->D.imax)
    return fail(MK_ERR_INVALID_ARG, "KV length %d + T %d exceeds idx_max_rows %d", kv->length, T, L->D.imax);
  if (T < 1 || T > kMaxT) return fail(MK_ERR_INVALID_ARG, "T=%d outside [1, %d]", T, kMaxT);
  if (kv->length < 0 || kv->capacity < 0 || (long long)kv->length + T > kv->capacity)
    return fail(MK_ERR_INVALID_ARG, "KV length %d + T %d exceeds capacity %d", kv->length, T, kv->capacity);
  if (hidden_in == hidden_out) return fail(MK_ERR_INVALID_ARG, "hidden_out may not alias hidden_in");
  return launch_layer(L, hidden_in, T, kv->rows, kv->capacity, kv->length, nullptr, hidden_out, nullptr,
                      (hipStream_t)stream);
}

int mk_decode_step_static(mk_layer* L, const float* hidden_in, int T, const mk_kv_cache* kv, float* hidden_out,
                          void* stream) {
  if (!L || !hidden_in || !kv || !kv->rows || !hidden_out) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (T < 1 || T > kMaxT) return fail(MK_ERR_INVALID_ARG, "T=%d outside [1, %d]", T, kMaxT);
  if (kv->length < 0 || kv->capacity < 0 || (long long)kv->length + T > kv->capacity)
    return fail(MK_ERR_INVALID_ARG, "KV length %d + T %d exceeds capacity %d", kv->length, T, kv->capacity);
  if (hidden_in == hidden_out) return fail(MK_ERR_INVALID_ARG, "hidden_out may not alias hidden_in");
  if (L->wl.total > kStaticScratchBytes)
    return fail(MK_ERR_UNSUPPORTED_SHAPE, "the layer's scratch (%zu bytes) exceeds the static scratch of %zu bytes",
                L->wl.total, kStaticScratchBytes);
  char* ptr = (L->dev >= 0 && L->dev < kMaxDevices) ? g_scratch_ptr[L->dev] : nullptr;
  if (!ptr)
    return fail(MK_ERR_HIP, "static scratch of device %d unavailable: %s", L->dev,
                hipGetErrorString(L->dev >= 0 && L->dev < kMaxDevices ? g_scratch_err[L->dev] : hipErrorInvalidDevice));
  return launch_layer(L, hidden_in, T, kv->rows, kv->capacity, kv->length, nullptr, hidden_out, nullptr,
                      (hipStream_t)stream, ptr);
}

int mk_debug_tap(mk_layer* L, int tap, void* host_dst, size_t bytes, void* stream) {
  if (!L || !host_dst) return fail(MK_ERR_INVALID_ARG, "null argument");
  const Dims& D = L->D;
  const int T = L->last_T;
  if (T <= 0) return fail(MK_ERR_INVALID_ARG, "no step has run on this layer");
  const char* src = nullptr;
  size_t need = 0;
  const LayerParams& p = L->last;
  switch (tap) {
    case 1: src = (const char*)p.qabs; need = (size_t)T * D.nh * D.dc * 4; break;
    case 2: src = (const char*)p.z; need = (size_t)T * D.nh * D.dc * 4; break;
    case 3: src = (const char*)p.o; need = (size_t)T * D.nh * D.dh * (D.af == MK_FMT_F32 ? 4 : 2); break;
    case 4: src = (const char*)p.hp; need = (size_t)T * D.d * 4; break;
    case 5: src = (const char*)p.logits; need = (size_t)T * D.E * 4; break;
    case 6: src = (const char*)p.route_sel; need = (size_t)T * D.topk * 4; break;
    case 7: src = (const char*)p.route_gate; need = (size_t)T * D.topk * 4; break;
    case 8:   // sparse attention: kept cache rows [T][idx_topk] (ascending; entries past a row's count unspecified)
    case 9:   // sparse attention: index scores [T][idx_max_rows] (row t: columns 0 .. L + T - 1)
      if (D.ik == 0) return fail(MK_ERR_INVALID_ARG, "tap %d needs sparse attention", tap);
      src = tap == 8 ? (const char*)p.isel : (const char*)p.iscore;
      need = (size_t)T * (tap == 8 ? D.ik : D.imax) * 4;
      break;
    case 0: {
      // Q with rotated q^R: rebuild [T][nh][qw] from the split-K partials and the rotated part
      if (bytes < (size_t)T * D.nh * D.qw * 4) return fail(MK_ERR_INVALID_ARG, "tap buffer too small");
      // (a low-rank query is kept whole in qbuf: one "partial" of row length nq)
      const bool lr = D.ql > 0;
      const int S = lr ? 1 : L->sch.s_q, nrow = lr ? D.nq : D.nq + D.kvw;
      std::string tmp((size_t)S * T * nrow * 4, '\0');
      std::string rq((size_t)T * D.nh * D.dr * 4, '\0');
      HIP_OK(hipStreamSynchronize((hipStream_t)stream));
      HIP_OK(hipMemcpy(&tmp[0], lr ? p.qbuf : p.qkv_part, tmp.size(), hipMemcpyDeviceToHost));
      HIP_OK(hipMemcpy(&rq[0], p.qrope, rq.size(), hipMemcpyDeviceToHost));
      const float* pt = (const float*)tmp.data();
      const float* pr = (const float*)rq.data();
      float* o = (float*)host_dst;
      for (int t = 0; t < T; ++t)
        for (int h = 0; h < D.nh; ++h)
          for (int e = 0; e < D.qw; ++e) {
            float v;
            if (e < D.dh) {
              v = 0.f;
              for (int s = 0; s < S; ++s) v += pt[((size_t)s * T + t) * nrow + h * D.qw + e];
            } else {
              v = pr[((size_t)t * D.nh + h) * D.dr + (e - D.dh)];
            }
            o[((size_t)t * D.nh + h) * D.qw + e] = v;
          }
      return MK_OK;
    }
    default: return fail(MK_ERR_INVALID_ARG, "unknown tap %d", tap);
  }
  if (bytes < need) return fail(MK_ERR_INVALID_ARG, "tap buffer too small (%zu < %zu)", bytes, need);
  HIP_OK(hipStreamSynchronize((hipStream_t)stream));
  HIP_OK(hipMemcpy(host_dst, src, need, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_get_stats(const mk_layer* L, mk_stats* out) {
  if (!L || !out) return fail(MK_ERR_INVALID_ARG, "null argument");
  out->steps = L->steps;
  out->launches = L->launches;
  out->grid_wgs = L->sch.nwg;
  out->threads_per_wg = kThreads;
  out->barriers_per_step = kBarriers;
  out->trace_enabled = L->trace_on;
  unsigned long long dv[2] = {0, 0};
  HIP_OK(hipMemcpy(dv, L->state + L->sl.bar + offsetof(BarrierState, slots_sum), 16, hipMemcpyDeviceToHost));
  out->expert_blocks_sum = (int64_t)dv[0];
  out->device_launches = (int64_t)dv[1];
  return MK_OK;
}

int mk_set_trace(mk_layer* L, int enabled) {
  if (!L) return fail(MK_ERR_INVALID_ARG, "null layer");
  if (enabled && !L->trace_on) {
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemset(L->state + L->sl.trace, 0, (size_t)L->sch.nwg * kTraceStride * 8));
    HIP_OK(hipDeviceSynchronize());
  }
  L->trace_on = enabled ? 1 : 0;
  return MK_OK;
}

int mk_read_trace(mk_layer* L, int64_t* host_dst, size_t bytes, void* stream) {
  if (!L || !host_dst) return fail(MK_ERR_INVALID_ARG, "null argument");
  const size_t need = (size_t)L->sch.nwg * kTraceStride * 8;
  if (bytes < need) return fail(MK_ERR_INVALID_ARG, "trace buffer too small (%zu < %zu)", bytes, need);
  HIP_OK(hipStreamSynchronize((hipStream_t)stream));
  HIP_OK(hipMemcpy(host_dst, L->state + L->sl.trace, need, hipMemcpyDeviceToHost));
  return MK_OK;
}

int mk_set_barrier_timeout_us(mk_layer* L, int64_t us) {
  if (!L || us <= 0) return fail(MK_ERR_INVALID_ARG, "bad argument");
  L->timeout_us = us;
  return MK_OK;
}

static int status_of_fault(uint32_t fault) {
  if (fault == kFaultTimeout) return fail(MK_ERR_TIMEOUT, "a bounded device wait exceeded its limit");
  if (fault == kFaultKvRange) return fail(MK_ERR_INVALID_ARG, "device KV length + T exceeded the cache capacity");
  if (fault == kFaultToken) return fail(MK_ERR_INVALID_ARG, "a token id was outside [0, vocab)");
  if (fault == kFaultXcd)
    return fail(MK_ERR_DEVICE_FAULT, "a workgroup ran on another XCD than its barrier group assumes");
  if (fault != 0) return fail(MK_ERR_DEVICE_FAULT, "device fault word %u", fault);
  return MK_OK;
}

int mk_sync_status(mk_layer* L) {
  if (!L) return fail(MK_ERR_INVALID_ARG, "null layer");
  uint32_t fault = 0;
  HIP_OK(hipMemcpy(&fault, L->state + L->sl.bar + offsetof(BarrierState, fault), 4, hipMemcpyDeviceToHost));
  return status_of_fault(fault);
}

int mk_layer_reset(mk_layer* L) {
  if (!L) return fail(MK_ERR_INVALID_ARG, "null layer");
  int cur = 0;
  hipGetDevice(&cur);
  hipSetDevice(L->dev);
  hipError_t e1 = hipMemset(L->state + L->sl.bar, 0, sizeof(BarrierState));
  hipError_t e2 = hipMemset(L->state + L->sl.att_cnt, 0, L->sl.experts - L->sl.att_cnt);
  hipError_t e3 = hipDeviceSynchronize();
  hipSetDevice(cur);
  if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess) return fail(MK_ERR_HIP, "reset failed");
  return MK_OK;
}

void mk_layer_destroy(mk_layer* L) { delete L; }

// ------------------------------------------------------------------ stack
// fp8 head: the E4M3 tiles, then (at a 256-byte boundary) the fp32 block scales
static long long head_scales_offset(int32_t vocab, int32_t d_model) {
  return (long long)align256((size_t)tiles_bytes(vocab, d_model, MK_FMT_FP8_B128));
}

int mk_head_packed_bytes_fmt(int32_t vocab, int32_t d_model, int32_t format, size_t* bytes) {
  if (!bytes || vocab <= 0 || d_model <= 0 || vocab % 16 || d_model % 128)
    return fail(MK_ERR_INVALID_ARG, "vocab must be a positive multiple of 16 and d_model of 128");
  if (format == MK_FMT_BF16) {
    *bytes = (size_t)tiles_bytes(vocab, d_model, MK_FMT_BF16);
  } else if (format == MK_FMT_FP8_B128) {
    *bytes = (size_t)head_scales_offset(vocab, d_model) +
             (size_t)((vocab + 127) / 128) * (size_t)((d_model + 127) / 128) * 4;
  } else {
    return fail(MK_ERR_INVALID_ARG, "head format must be BF16 or FP8_B128");
  }
  return MK_OK;
}

int mk_head_packed_bytes(int32_t vocab, int32_t d_model, size_t* bytes) {
  return mk_head_packed_bytes_fmt(vocab, d_model, MK_FMT_BF16, bytes);
}

int mk_pack_head_fp8(int32_t vocab, int32_t d_model, const uint8_t* codes, const float* scales, void* dst,
                     void* stream) {
  size_t b;
  int rc = mk_head_packed_bytes_fmt(vocab, d_model, MK_FMT_FP8_B128, &b);
  if (rc) return rc;
  if (!codes || !scales || !dst) return fail(MK_ERR_INVALID_ARG, "null tensor");
  hipStream_t s = (hipStream_t)stream;
  rc = launch_pack(codes, MK_FMT_FP8_B128, 1, vocab, d_model, 0, d_model, 1, dst, 1024, 0, s);
  if (rc) return fail(MK_ERR_HIP, "pack launch failed");
  const size_t nsc = (size_t)((vocab + 127) / 128) * (size_t)((d_model + 127) / 128) * 4;
  if (hipMemcpyAsync((char*)dst + head_scales_offset(vocab, d_model), scales, nsc, hipMemcpyDeviceToDevice, s) !=
      hipSuccess)
    return fail(MK_ERR_HIP, "copy of the head scales failed");
  return MK_OK;
}

int mk_pack_head(int32_t vocab, int32_t d_model, const uint16_t* src_bf16, void* dst, void* stream) {
  size_t b;
  int rc = mk_head_packed_bytes(vocab, d_model, &b);
  if (rc) return rc;
  if (!src_bf16 || !dst) return fail(MK_ERR_INVALID_ARG, "null tensor");
  rc = launch_pack(src_bf16, MK_FMT_BF16, 1, vocab, d_model, 0, d_model, 1, dst, 1024, 0, (hipStream_t)stream);
  if (rc) return fail(MK_ERR_HIP, "pack launch failed");
  return MK_OK;
}

struct ModelStLayout {
  size_t len, counter, fault, best_val, best_idx, tickets, dummy, step, part, total;
};
static ModelStLayout model_layout(int nwg) {
  ModelStLayout l;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  l.len = take(4);
  l.counter = take(4);
  l.fault = take(4);
  l.best_val = take((size_t)nwg * 8 * 4);
  l.best_idx = take((size_t)nwg * 8 * 4);
  l.tickets = take((size_t)8 * kCntStride * 4);
  l.dummy = take(32768);
  l.step = take(4);
  l.part = take((size_t)nwg * 8 * 8 * 4);
  l.total = off;
  return l;
}

static int head_grid(int dev, int* nwg) {
  hipDeviceProp_t prop;
  HIP_OK(hipGetDeviceProperties(&prop, dev));
  int cur = 0;
  HIP_OK(hipGetDevice(&cur));
  HIP_OK(hipSetDevice(dev));
  int occ = 0;
  int rc = head_kernel_occupancy(&occ);
  HIP_OK(hipSetDevice(cur));
  if (rc) return fail(MK_ERR_HIP, "head kernel occupancy query failed");
  if (occ < 1) return fail(MK_ERR_NOT_CORESIDENT, "head kernel cannot be resident");
  *nwg = prop.multiProcessorCount;
  return MK_OK;
}

int mk_model_state_bytes(int32_t n_layers, int32_t vocab, int hip_device, size_t* bytes) {
  if (!bytes || n_layers <= 0 || vocab <= 0) return fail(MK_ERR_INVALID_ARG, "bad arguments");
  int nwg = 0;
  int rc = head_grid(hip_device, &nwg);
  if (rc) return rc;
  *bytes = model_layout(nwg).total;
  return MK_OK;
}

int mk_model_init(mk_layer* const* layers, int32_t n_layers, const uint16_t* embedding, const void* head_packed,
                  const float* gamma_final, int32_t vocab, void* const* kv_rows, int32_t capacity, void* state_dev,
                  void* hidden_dev, mk_model** out) {
  return mk_model_init_ex(layers, n_layers, embedding, head_packed, MK_FMT_BF16, gamma_final, vocab, kv_rows,
                          capacity, state_dev, hidden_dev, out);
}

int mk_model_init_ex(mk_layer* const* layers, int32_t n_layers, const uint16_t* embedding, const void* head_packed,
                     int32_t head_format, const float* gamma_final, int32_t vocab, void* const* kv_rows,
                     int32_t capacity, void* state_dev, void* hidden_dev, mk_model** out) {
  if (!out) return fail(MK_ERR_INVALID_ARG, "null output");
  *out = nullptr;
  if (!layers || n_layers <= 0 || !embedding || !head_packed || !gamma_final || !kv_rows || !state_dev || !hidden_dev)
    return fail(MK_ERR_INVALID_ARG, "null argument");
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l] || !kv_rows[l]) return fail(MK_ERR_INVALID_ARG, "layer %d or its KV rows are null", l);
    if (std::memcmp(&layers[l]->cfg, &layers[0]->cfg, sizeof(mk_layer_config)) != 0)
      return fail(MK_ERR_INVALID_ARG, "layer %d has a different config", l);
  }
  size_t hb;
  int rc = mk_head_packed_bytes_fmt(vocab, layers[0]->D.d, head_format, &hb);
  if (rc) return rc;
  int nwg = 0;
  rc = head_grid(layers[0]->dev, &nwg);
  if (rc) return rc;
  mk_model* m = new (std::nothrow) mk_model();
  if (!m) return fail(MK_ERR_INVALID_ARG, "out of host memory");
  m->layers = new mk_layer*[n_layers];
  m->kv = new void*[n_layers];
  for (int l = 0; l < n_layers; ++l) {
    m->layers[l] = layers[l];
    m->kv[l] = kv_rows[l];
  }
  m->n_layers = n_layers;
  m->emb = embedding;
  m->head = head_packed;
  m->gamma_f = gamma_final;
  m->V = vocab;
  m->capacity = capacity;
  m->state = (char*)state_dev;
  m->hidden = (float*)hidden_dev;
  const ModelStLayout ml = model_layout(nwg);
  m->kv_len = (int32_t*)(m->state + ml.len);
  m->counter = (uint32_t*)(m->state + ml.counter);
  m->fault = (uint32_t*)(m->state + ml.fault);
  m->hidden_rec = nullptr;
  m->best_val = (float*)(m->state + ml.best_val);
  m->best_idx = (int32_t*)(m->state + ml.best_idx);
  m->tickets = (uint32_t*)(m->state + ml.tickets);
  m->dummy = (const uint8_t*)(m->state + ml.dummy);
  m->nwg_head = nwg;
  m->head_fmt = head_format;
  m->head_scales = head_format == MK_FMT_FP8_B128
                       ? (const float*)((const char*)head_packed + head_scales_offset(vocab, layers[0]->D.d))
                       : nullptr;
  m->temperature = 0.f;
  m->seed = 0;
  m->step = (uint32_t*)(m->state + ml.step);
  m->part = (float*)(m->state + ml.part);
  hipError_t e = hipMemset(m->state, 0, ml.total);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    delete[] m->layers;
    delete[] m->kv;
    delete m;
    return fail(MK_ERR_HIP, "model state initialisation: %s", hipGetErrorString(e));
  }
  *out = m;
  return MK_OK;
}

int mk_model_set_length(mk_model* m, int32_t length) {
  if (!m || length < 0 || length > m->capacity) return fail(MK_ERR_INVALID_ARG, "bad length");
  HIP_OK(hipMemcpy(m->kv_len, &length, 4, hipMemcpyHostToDevice));
  return MK_OK;
}

const int32_t* mk_model_length_ptr(const mk_model* m) { return m ? m->kv_len : nullptr; }

int mk_model_step(mk_model* m, int32_t* tokens_dev, int T, const int32_t* next_drafts_dev, int32_t* argmax_dev,
                  int32_t* committed_dev, float* logits_dev, void* stream) {
  if (!m || !tokens_dev || !argmax_dev || !committed_dev) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (T < 1 || T > kMaxT) return fail(MK_ERR_INVALID_ARG, "T=%d outside [1, %d]", T, kMaxT);
  hipStream_t s = (hipStream_t)stream;
  const int d = m->layers[0]->D.d;
  // hidden rows of layer l's input: two buffers in turn, or slot l of the record
  const size_t rows = (size_t)kMaxT * d;
  auto hid = [&](int l) -> float* {
    return m->hidden_rec ? m->hidden_rec + (size_t)l * rows : m->hidden + (size_t)(l & 1) * rows;
  };
  int rc = launch_embed(m->emb, m->V, d, tokens_dev, T, hid(0), m->fault, s);
  if (rc) return fail(MK_ERR_HIP, "embedding launch failed");
  for (int l = 0; l < m->n_layers; ++l) {
    // the KV length lives in device memory; a step that would pass the capacity faults on the device
    rc = launch_layer(m->layers[l], hid(l), T, m->kv[l], m->capacity, 0, m->kv_len, hid(l + 1), m->fault, s);
    if (rc) return rc;
  }
  HeadLaunch h;
  h.head_packed = m->head; h.head_fmt = m->head_fmt; h.scales = m->head_scales;
  h.V = m->V; h.d = d; h.gamma = m->gamma_f; h.eps = m->layers[0]->cfg.rms_eps; h.hidden = hid(m->n_layers);
  h.best_val = m->best_val; h.best_idx = m->best_idx; h.counter = m->counter; h.tickets = m->tickets;
  h.kv_len = m->kv_len; h.dummy = m->dummy; h.fault = m->fault; h.nwg = m->nwg_head;
  h.temperature = m->temperature; h.seed = m->seed; h.step = m->step; h.part = m->part;
  rc = launch_head(h, T, logits_dev, tokens_dev, next_drafts_dev, argmax_dev, committed_dev, s);
  if (rc) return fail(MK_ERR_HIP, "head launch failed");
  return MK_OK;
}

int mk_model_set_sampling(mk_model* m, float temperature, uint64_t seed) {
  if (!m) return fail(MK_ERR_INVALID_ARG, "null model");
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(MK_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  int cur = 0;
  hipGetDevice(&cur);
  hipSetDevice(m->layers[0]->dev);
  hipError_t e = hipMemset(m->step, 0, 4);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  hipSetDevice(cur);
  if (e != hipSuccess) return fail(MK_ERR_HIP, "sampling reset failed");
  m->temperature = temperature;
  m->seed = seed;
  return MK_OK;
}

int mk_model_set_hidden_record(mk_model* m, float* record_dev) {
  if (!m) return fail(MK_ERR_INVALID_ARG, "null model");
  m->hidden_rec = record_dev;
  return MK_OK;
}

int mk_model_sync_status(mk_model* m) {
  if (!m) return fail(MK_ERR_INVALID_ARG, "null model");
  uint32_t fault = 0;
  HIP_OK(hipMemcpy(&fault, m->fault, 4, hipMemcpyDeviceToHost));
  return status_of_fault(fault);
}

int mk_model_reset(mk_model* m) {
  if (!m) return fail(MK_ERR_INVALID_ARG, "null model");
  for (int l = 0; l < m->n_layers; ++l) {
    const int rc = mk_layer_reset(m->layers[l]);
    if (rc) return rc;
  }
  int cur = 0;
  hipGetDevice(&cur);
  hipSetDevice(m->layers[0]->dev);
  hipError_t e1 = hipMemset(m->fault, 0, 4);
  hipError_t e2 = hipMemset(m->counter, 0, 4);
  if (e2 == hipSuccess) e2 = hipMemset(m->tickets, 0, (size_t)8 * kCntStride * 4);
  hipError_t e3 = hipDeviceSynchronize();
  hipSetDevice(cur);
  if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess) return fail(MK_ERR_HIP, "model reset failed");
  return MK_OK;
}

void mk_model_destroy(mk_model* m) {
  if (!m) return;
  delete[] m->layers;
  delete[] m->kv;
  delete m;
}

}  // extern "C"
