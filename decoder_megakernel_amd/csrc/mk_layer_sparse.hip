// Instantiations of the layer kernel (mk_layer_kernel.h) with sparse attention
// (indexer, top-k kept rows per verify row): bf16 attention and cache, bf16,
// fp8 or MXFP4 experts, with one W_Q or a low-rank query; general shapes, and
// the 384-expert layer's dimensions fixed at compile time for fp8 experts.
#include "mk_host.h"
#include "mk_layer_kernel.h"

namespace mk {

LayerKernelFn layer_kernel_sparse_kv8_for(int ef, bool lowrank, bool spec);

LayerKernelFn layer_kernel_sparse_for(int af, int ef, int kf, bool lowrank, bool spec) {
  if (af != MK_FMT_BF16) return nullptr;
  if (kf == MK_FMT_FP8_ROW) return layer_kernel_sparse_kv8_for(ef, lowrank, spec);   // mk_layer_sparse_kv8.hip
  if (kf != MK_FMT_BF16) return nullptr;
  constexpr int A = MK_FMT_BF16, K = MK_FMT_BF16;
  if (spec && ef == MK_FMT_FP8_B128)
    return lowrank ? layer_kernel<A, MK_FMT_FP8_B128, K, 18, 32, true, 2, true, true>
                   : layer_kernel<A, MK_FMT_FP8_B128, K, 18, 32, true, 2, false, true>;
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
