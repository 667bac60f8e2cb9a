// Instantiations of the row-gather GEMV for f16 weights, 1 token(s).
#include "gather_gemv_impl.hpp"

namespace as {
hipError_t launch_gemv_f16_m1(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  return pick_lpr<DT_F16, 1>(c, p, smem, s);
}
}  // namespace as
