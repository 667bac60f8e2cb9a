// Instantiations of the row-gather GEMV for bf16 weights, 4 token(s).
#include "gather_gemv_impl.hpp"

namespace as {
hipError_t launch_gemv_bf16_m4(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  return pick_lpr<DT_BF16, 4>(c, p, smem, s);
}
hipError_t launch_fused_bf16_m4(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s) {
  return fused_pick<DT_BF16, 4>(c, f, smem, s);
}
}  // namespace as
