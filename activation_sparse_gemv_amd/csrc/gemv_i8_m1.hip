// Instantiations of the row-gather GEMV for int8 weights with a per-row scale, 1 token.
#include "gather_gemv_impl.hpp"

namespace as {
hipError_t launch_gemv_i8_m1(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  if (c.mt != 1) return hipErrorInvalidValue;
  switch (c.lpr) {
    case 16: return pick_i8_mode<16>(c, p, smem, s);
    case 32: return pick_i8_mode<32>(c, p, smem, s);
    case 64: return pick_i8_mode<64>(c, p, smem, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace as
