// Instantiations of the layer kernel (mk_layer_kernel.h) for layers with a
// low-rank query (W_DQ, q-norm, W_UQ; optionally an RMSNorm of the cached
// latent): bf16 attention with bf16, fp8 or MXFP4 experts and a bf16 or fp8
// cache, general shapes (d_latent + d_rope <= 576, d_latent <= 512), and the
// choice between them and the fixed-shape instances.
#include "mk_host.h"
#include "mk_layer_kernel.h"

namespace mk {

LayerKernelFn layer_kernel_lowrank_spec(int ef, int kf);

LayerKernelFn layer_kernel_lowrank_for(int af, int ef, int kf, int d, int nh, int dh, int dc, int dr, int E, int topk,
                                       int nshared, int f, int s_q, int nwg) {
  if (af != MK_FMT_BF16 || dc + dr > 576 || dc > 512) return nullptr;
  // the 384-expert layer's dimensions fixed at compile time (instances in mk_layer_lr_spec.hip)
  const SpecShape& sp = kSpecShapes[2];
  if (d == sp.d && nh == sp.nh && dh == sp.dh && dc == sp.dc && dr == sp.dr && E == sp.E && topk == sp.topk &&
      nshared == sp.nshared && f == sp.f && (s_q == 0 || s_q == sp.s_q) && (nwg == 0 || nwg >= kSpecMinGrid)) {
    LayerKernelFn fn = layer_kernel_lowrank_spec(ef, kf);
    if (fn) return fn;
  }
  constexpr int A = MK_FMT_BF16;
  if (kf == MK_FMT_BF16) {
    if (ef == MK_FMT_BF16) return layer_kernel<A, MK_FMT_BF16, MK_FMT_BF16, 18, 32, false, 0, true>;
    if (ef == MK_FMT_FP8_B128) return layer_kernel<A, MK_FMT_FP8_B128, MK_FMT_BF16, 18, 32, false, 0, true>;
    if (ef == MK_FMT_MXFP4) return layer_kernel<A, MK_FMT_MXFP4, MK_FMT_BF16, 18, 32, false, 0, true>;
  }
  if (kf == MK_FMT_FP8_ROW) {
    if (ef == MK_FMT_BF16) return layer_kernel<A, MK_FMT_BF16, MK_FMT_FP8_ROW, 18, 32, false, 0, true>;
    if (ef == MK_FMT_FP8_B128) return layer_kernel<A, MK_FMT_FP8_B128, MK_FMT_FP8_ROW, 18, 32, false, 0, true>;
    if (ef == MK_FMT_MXFP4) return layer_kernel<A, MK_FMT_MXFP4, MK_FMT_FP8_ROW, 18, 32, false, 0, true>;
  }
  return nullptr;
}

}  // namespace mk
