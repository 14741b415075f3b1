// Instantiations of the layer kernel (mk_layer_kernel.h) with sparse attention
// over an fp8 (E4M3 row) cache whose rows carry the index key under the row's
// scale: bf16 attention, bf16, fp8 or MXFP4 experts, with one W_Q or a
// low-rank query; general shapes, and the 384-expert layer's dimensions fixed at
// compile time (fp8 or MXFP4 experts, one W_Q).
#include "mk_host.h"
#include "mk_layer_kernel.h"

namespace mk {

LayerKernelFn layer_kernel_sparse_kv8_for(int ef, bool lowrank, bool spec) {
  constexpr int A = MK_FMT_BF16, K = MK_FMT_FP8_ROW;
  if (spec && !lowrank) {
    if (ef == MK_FMT_FP8_B128) return layer_kernel<A, MK_FMT_FP8_B128, K, 18, 32, true, 2, false, true>;
    if (ef == MK_FMT_MXFP4) return layer_kernel<A, MK_FMT_MXFP4, K, 18, 32, true, 2, false, true>;
  }
  if (ef == MK_FMT_BF16)
    return lowrank ? layer_kernel<A, MK_FMT_BF16, K, 18, 32, false, 0, true, true>
                   : layer_kernel<A, MK_FMT_BF16, K, 18, 32, false, 0, false, true>;
  if (ef == MK_FMT_FP8_B128)
    return lowrank ? layer_kernel<A, MK_FMT_FP8_B128, K, 18, 32, false, 0, true, true>
                   : layer_kernel<A, MK_FMT_FP8_B128, K, 18, 32, false, 0, false, true>;
  if (ef == MK_FMT_MXFP4)
    return lowrank ? layer_kernel<A, MK_FMT_MXFP4, K, 18, 32, false, 0, true, true>
                   : layer_kernel<A, MK_FMT_MXFP4, K, 18, 32, false, 0, false, true>;
  return nullptr;
}

}  // namespace mk
