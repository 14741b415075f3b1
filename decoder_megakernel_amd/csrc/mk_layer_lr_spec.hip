// Instances of the layer kernel (mk_layer_kernel.h) with a low-rank query at
// the 384-expert layer's dimensions (d_model 4096, 32 heads of 128, latent
// 512 + 64, experts of width 2048), fixed at compile time: fp8 or MXFP4
// experts, bf16 cache, and MXFP4 experts with the fp8 cache.
#include "mk_host.h"
#include "mk_layer_kernel.h"

namespace mk {

LayerKernelFn layer_kernel_lowrank_spec(int ef, int kf) {
  constexpr int A = MK_FMT_BF16;
  if (ef == MK_FMT_FP8_B128 && kf == MK_FMT_BF16)
    return layer_kernel<A, MK_FMT_FP8_B128, MK_FMT_BF16, 18, 32, true, 2, true>;
  if (ef == MK_FMT_MXFP4 && kf == MK_FMT_BF16) return layer_kernel<A, MK_FMT_MXFP4, MK_FMT_BF16, 18, 32, true, 2, true>;
  if (ef == MK_FMT_MXFP4 && kf == MK_FMT_FP8_ROW)
    return layer_kernel<A, MK_FMT_MXFP4, MK_FMT_FP8_ROW, 18, 32, true, 2, true>;
  return nullptr;
}

}  // namespace mk
