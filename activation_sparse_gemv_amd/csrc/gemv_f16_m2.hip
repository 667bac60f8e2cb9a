// Instantiations of the row-gather GEMV for f16 weights, 2 token(s).
#include "gather_gemv_impl.hpp"

namespace as {
hipError_t launch_gemv_f16_m2(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  return pick_lpr<DT_F16, 2>(c, p, smem, s);
}
}  // namespace as
