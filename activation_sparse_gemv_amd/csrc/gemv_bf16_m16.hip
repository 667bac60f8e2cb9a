// Instantiations of the row-gather GEMV for bf16 weights, 9..16 tokens (MFMA main loop).
#include "gather_gemv_impl.hpp"

namespace as {
hipError_t launch_gemv_bf16_m16(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  return pick_lpr<DT_BF16, 16>(c, p, smem, s);
}
}  // namespace as
