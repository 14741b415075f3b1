// Instantiations of the layer kernel (mk_layer_kernel.h) for layers with a
// low-rank query (W_DQ, q-norm, W_UQ; optionally an RMSNorm of the cached
// latent): bf16 attention with bf16, fp8 or MXFP4 experts and a bf16 or fp8
// cache, general shapes (d_latent + d_rope <= 576, d_latent <= 512).
#include "mk_host.h"
#include "mk_layer_kernel.h"

namespace mk {

LayerKernelFn layer_kernel_lowrank_for(int af, int ef, int kf, int dc, int dr) {
  if (af != MK_FMT_BF16 || dc + dr > 576 || dc > 512) return nullptr;
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
