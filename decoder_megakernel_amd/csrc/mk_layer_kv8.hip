// Instantiations of the layer kernel (mk_layer_kernel.h) for the fp8 (E4M3,
// one scale per row) cache: bf16 attention with bf16, fp8 or MXFP4 experts,
// generic and at the fixed 512 + 64 latent shape.
#include "mk_host.h"
#include "mk_layer_kernel.h"

namespace mk {

LayerKernelFn layer_kernel_kv8(int ef, bool spec) {
  constexpr int KF = MK_FMT_FP8_ROW;
  if (ef == MK_FMT_BF16) return layer_kernel<MK_FMT_BF16, MK_FMT_BF16, KF, 18, 32, false, 0>;
  if (ef == MK_FMT_FP8_B128)
    return spec ? layer_kernel<MK_FMT_BF16, MK_FMT_FP8_B128, KF, 18, 32, true, 2>
                : layer_kernel<MK_FMT_BF16, MK_FMT_FP8_B128, KF, 18, 32, false, 0>;
  if (ef == MK_FMT_MXFP4)
    return spec ? layer_kernel<MK_FMT_BF16, MK_FMT_MXFP4, KF, 18, 32, true, 2>
                : layer_kernel<MK_FMT_BF16, MK_FMT_MXFP4, KF, 18, 32, false, 0>;
  return nullptr;
}

}  // namespace mk
