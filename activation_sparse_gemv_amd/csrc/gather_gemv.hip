// Row-gather GEMV launch entry: picks the instantiation (weights dtype, tokens) and
// the threshold-prologue chunk width.  The kernel itself is in gather_gemv_impl.hpp.
#include "common.hpp"
#include "internal.hpp"

namespace as {

constexpr int kThreadsHost = 256;

size_t gemv_smem_bytes(const GemvConfig& c, int cap, int n_lt) {
  auto a16 = [](size_t b) { return (b + 15) & ~size_t(15); };
  const int nslot = 4 * (64 / c.lpr), tn = c.lpr * 8;
  size_t b = a16(size_t(cap) * 4) + a16(size_t(cap) * c.mt * 4);
  // slot reduction of the VALU loop (the MFMA loop stages its output in the chunk buffer)
  if (c.mt != 16) b += a16(size_t(nslot > c.mt ? nslot : c.mt) * tn * 4);
  if (c.in == IN_LISTS || c.in == IN_TILES) b += a16(size_t(n_lt + 1) * 4);
  // staging region: IN_TILES raw candidate entries (index + M values, cap of them)
  // or the IN_RANGE input range during the prologue; the MFMA weight chunk and
  // output tile afterwards
  size_t stage = 0;
  if (c.in == IN_TILES) stage = size_t(cap) * (1 + c.mt) * 4;
  // IN_RANGE, several tokens, and IN_PARTS: the slice's range of every token, fp32
  if ((c.in == IN_RANGE && c.mt > 1) || c.in == IN_PARTS) stage = size_t(cap) * c.mt * 4;
  if (c.mt == 16) {
    const size_t rows = size_t(32) * (512 / tn);
    const size_t chunk = rows * (tn + 4) * 2, out = size_t(16) * tn * 4;
    const size_t m = chunk > out ? chunk : out;
    if (m > stage) stage = m;
  }
  return b + stage;
}

hipError_t launch_gemv_bf16_m16(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
hipError_t launch_gemv_bf16_m1(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
hipError_t launch_gemv_bf16_m2(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
hipError_t launch_gemv_bf16_m4(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
hipError_t launch_gemv_bf16_m8(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
hipError_t launch_gemv_f16_m1(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
hipError_t launch_gemv_f16_m2(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
hipError_t launch_gemv_f16_m4(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
hipError_t launch_gemv_f16_m8(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);

// Chunk width (16-byte vectors of 8 inputs per thread) of the vectorised
// threshold prologue over `len` inputs, or 0 for the element-wise one.
int pick_chunk_vectors(const void* x, int x_dt, int len, long ldx) {
  const int es = x_dt == DT_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0 || (ldx * es) % 16 != 0) return 0;
  const int per = (len + kThreadsHost - 1) / kThreadsHost;
  if (per <= 16) return 2;
  if (per <= 64) return 8;
  return 0;
}

hipError_t launch_fused_bf16_m1(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s);
hipError_t launch_fused_bf16_m2(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s);
hipError_t launch_fused_bf16_m4(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s);
hipError_t launch_fused_bf16_m8(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s);
hipError_t launch_fused_f16_m1(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s);
hipError_t launch_fused_f16_m2(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s);
hipError_t launch_fused_f16_m4(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s);
hipError_t launch_fused_f16_m8(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s);

hipError_t launch_fused_mlp(const FusedCfg& c, const FusedMlpParams& f, size_t smem, hipStream_t s) {
  const bool bf = c.wdt == DT_BF16;
  switch (c.mt) {
    case 1: return bf ? launch_fused_bf16_m1(c, f, smem, s) : launch_fused_f16_m1(c, f, smem, s);
    case 2: return bf ? launch_fused_bf16_m2(c, f, smem, s) : launch_fused_f16_m2(c, f, smem, s);
    case 4: return bf ? launch_fused_bf16_m4(c, f, smem, s) : launch_fused_f16_m4(c, f, smem, s);
    case 8: return bf ? launch_fused_bf16_m8(c, f, smem, s) : launch_fused_f16_m8(c, f, smem, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gather_gemv(const GemvConfig& c, const GemvParams& p, hipStream_t s) {
  const size_t smem = gemv_smem_bytes(c, p.cap, p.n_lt);
  GemvConfig cc = c;
  if ((cc.in == IN_THRESH || cc.in == IN_RANGE) && cc.nv < 0) {
    if (cc.in == IN_RANGE && cc.mt > 1) {
      // staged range prologue: 16-byte vectors whenever rows are aligned
      cc.nv = (p.K % 8 == 0 && pick_chunk_vectors(p.x, p.x_dt, 1, p.ldx) > 0) ? 2 : 0;
    } else {
      // the chunk prologue covers the whole input (IN_THRESH) or one slice's range
      cc.nv = pick_chunk_vectors(p.x, p.x_dt, cc.in == IN_RANGE ? p.cap : p.K, p.ldx);
      if (cc.mt > 1 && cc.nv > 2) cc.nv = 0;     // wide register chunks only for one token
    }
  }
  const bool bf = cc.wdt == DT_BF16;
  switch (cc.mt) {
    case 1: return bf ? launch_gemv_bf16_m1(cc, p, smem, s) : launch_gemv_f16_m1(cc, p, smem, s);
    case 2: return bf ? launch_gemv_bf16_m2(cc, p, smem, s) : launch_gemv_f16_m2(cc, p, smem, s);
    case 4: return bf ? launch_gemv_bf16_m4(cc, p, smem, s) : launch_gemv_f16_m4(cc, p, smem, s);
    case 8: return bf ? launch_gemv_bf16_m8(cc, p, smem, s) : launch_gemv_f16_m8(cc, p, smem, s);
    case 16: return bf ? launch_gemv_bf16_m16(cc, p, smem, s) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace as
