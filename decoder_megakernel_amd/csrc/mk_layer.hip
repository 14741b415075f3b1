// Instantiations of the layer kernel (mk_layer_kernel.h) for the f32 and bf16
// caches, and the choice of kernel for a layer's formats and shape.  The fp8
// cache instances are built in mk_layer_kv8.hip (a separate unit, so the two
// sets compile in parallel).
#include "mk_host.h"
#include "mk_layer_kernel.h"

namespace mk {

LayerKernelFn layer_kernel_kv8(int ef, bool spec);

// Instantiations: all-fp32 (d_latent + d_rope <= 160, d_latent <= 128),
// bf16 attention with a bf16 or fp8 cache and bf16, fp8 or MXFP4 experts
// (d_latent + d_rope <= 576, d_latent <= 512), and the two fixed shapes of
// kSpecShapes (512 + 64 latent dims, so the attention loop bounds are
// constants too).
LayerKernelFn layer_kernel_for(int af, int ef, int kf, int d, int nh, int dh, int dc, int dr, int E, int topk,
                               int nshared, int f, int s_q, int nwg) {
  const int kvw = dc + dr;
  auto is = [&](int i) {
    const SpecShape& s = kSpecShapes[i];
    return d == s.d && nh == s.nh && dh == s.dh && dc == s.dc && dr == s.dr && E == s.E && topk == s.topk &&
           nshared == s.nshared && f == s.f && (s_q == 0 || s_q == s.s_q) && (nwg == 0 || nwg >= kSpecMinGrid);
  };
  if (af == MK_FMT_F32 && ef == MK_FMT_F32 && kf == MK_FMT_F32 && kvw <= 160 && dc <= 128)
    return layer_kernel<MK_FMT_F32, MK_FMT_F32, MK_FMT_F32, 10, 8, false, 0>;
  if (af == MK_FMT_BF16 && kf == MK_FMT_FP8_ROW && kvw <= 576 && dc <= 512)
    return layer_kernel_kv8(ef, is(2));
  if (af == MK_FMT_BF16 && kf == MK_FMT_BF16 && kvw <= 576 && dc <= 512) {
    if (ef == MK_FMT_BF16)
      return is(1) ? layer_kernel<MK_FMT_BF16, MK_FMT_BF16, MK_FMT_BF16, 18, 32, true, 1>
                   : layer_kernel<MK_FMT_BF16, MK_FMT_BF16, MK_FMT_BF16, 18, 32, false, 0>;
    if (ef == MK_FMT_FP8_B128)
      return is(2) ? layer_kernel<MK_FMT_BF16, MK_FMT_FP8_B128, MK_FMT_BF16, 18, 32, true, 2>
                   : layer_kernel<MK_FMT_BF16, MK_FMT_FP8_B128, MK_FMT_BF16, 18, 32, false, 0>;
    if (ef == MK_FMT_MXFP4)
      return is(2) ? layer_kernel<MK_FMT_BF16, MK_FMT_MXFP4, MK_FMT_BF16, 18, 32, true, 2>
                   : layer_kernel<MK_FMT_BF16, MK_FMT_MXFP4, MK_FMT_BF16, 18, 32, false, 0>;
  }
  return nullptr;
}

}  // namespace mk
