// Instantiations of the MoE layer's combined launches for bf16 weights, 1 token(s).
#include "moe_layer_impl.hpp"

namespace as {
hipError_t launch_moe_route_gu_m1(const MoeLayerCfg& c, const GemvParams& pr, const GemvParams& pg, size_t smem,
                                  hipStream_t s) {
  return moe_route_gu_pick<DT_BF16, 1>(c, pr, pg, smem, s);
}
hipError_t launch_moe_gu_down_m1(const MoeLayerCfg& c, const MoeParams& pm, int n_u, int n_gu, const GemvParams& pd,
                                 size_t smem, hipStream_t s) {
  return moe_gu_down_pick<DT_BF16, 1>(c, pm, n_u, n_gu, pd, smem, s);
}
}  // namespace as
