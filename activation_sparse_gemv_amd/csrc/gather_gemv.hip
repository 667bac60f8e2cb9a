// Row-gather GEMV launch entry: picks the instantiation (weights dtype, tokens) and
// the threshold-prologue chunk width.  The kernel itself is in gather_gemv_impl.hpp.
#include "common.hpp"
#include "internal.hpp"

namespace as {

constexpr int kThreadsHost = 256;

int device_cus() {
  static const int cus = [] {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      return prop.multiProcessorCount;
    return 256;
  }();
  return cus;
}

size_t gemv_smem_bytes(const GemvConfig& c, int cap, int n_lt) {
  auto a16 = [](size_t b) { return (b + 15) & ~size_t(15); };
  const int nslot = 4 * (64 / c.lpr), tn = c.lpr * 8;
  size_t b = a16(size_t(cap) * 4) + a16(size_t(cap) * c.mt * 4);
  // slot reduction of the VALU loop (the MFMA loop stages its output in the chunk buffer)
  if (c.mt != 16) b += a16(size_t(nslot > c.mt ? nslot : c.mt) * tn * 4);
  if (c.in == IN_LISTS) b += a16(size_t(n_lt + 1) * 4);
  // staging region: the IN_RANGE / IN_PARTS input range during the prologue; the
  // MFMA weight chunk and output tile afterwards
  size_t stage = 0;
  // IN_RANGE, several tokens, and IN_PARTS: the slice's range of every token, fp32
  if ((c.in == IN_RANGE && c.mt > 1) || c.in == IN_PARTS) stage = size_t(cap) * c.mt * 4;
  if (c.mt == 16) {
    const size_t rows = size_t(32) * (512 / tn);
    const size_t chunk = size_t(tn) * (rows + 8) * 2, out = size_t(16) * tn * 4;
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


// y[m][c] = sum over slices s = 0, 1, ... of partials[s][m][c], in that order from
// 0, then + y (accumulate), then + res: the additions of the in-kernel last-workgroup
// combine, so results are bitwise the same.  One thread per output element, the
// slices' loads issued in batches of eight.
__global__ __launch_bounds__(kThreadsHost) void sum_slices_kernel(const GemvParams p) {
  const long i = (long)blockIdx.x * kThreadsHost + threadIdx.x;
  if (i >= (long)p.M * p.N) return;
  const int m = (int)(i / p.N), c = (int)(i % p.N);
  const float* src = p.partials + (long)m * p.part_ld + c;
  const long stride = (long)p.M * p.part_ld;
  float v = 0.f;
  for (int s0 = 0; s0 < p.S; s0 += 8) {
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = src[(long)min(s0 + k, p.S - 1) * stride];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < p.S) v += t[k];
  }
  if (p.accumulate) v += load_elem(p.y, p.y_dt, m * p.ldy + c);
  if (p.res != nullptr) v += load_elem(p.res, p.res_dt, m * p.ldres + c);
  store_elem(p.y, p.y_dt, m * p.ldy + c, v);
}

// The SwiGLU epilogue of a gate/up launch whose slices stored their partials: for
// token m = blockIdx.y and neuron n, g and u are the slice-order sums of the gate
// (column n) and up (column N + n) partials, h = silu(g) * u, and the |h| > t_h
// mask bits and counts are exported when asked for; the y the next launch adds into
// is cleared.  The same operations in the same order as the in-kernel epilogue.
__global__ __launch_bounds__(kThreadsHost) void sum_swiglu_kernel(const GemvParams p) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * kThreadsHost + threadIdx.x;
  const bool valid = n < p.N;
  if (p.zero_y != nullptr) {
    const long nth = (long)gridDim.x * gridDim.y * kThreadsHost;
    for (long i = ((long)blockIdx.y * gridDim.x + blockIdx.x) * kThreadsHost + threadIdx.x; i < p.zero_n; i += nth)
      p.zero_y[i] = 0.f;
  }
  const int nc = valid ? n : 0;
  const float* src = p.partials + (long)m * p.part_ld;
  const long stride = (long)p.M * p.part_ld;
  float g = 0.f, u = 0.f;
  for (int s0 = 0; s0 < p.S; s0 += 8) {
    float tg[8], tu[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float* ps = src + (long)min(s0 + k, p.S - 1) * stride;
      tg[k] = ps[nc];
      tu[k] = ps[(long)p.N + nc];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < p.S) {
        g += tg[k];
        u += tu[k];
      }
  }
  const float hv = valid ? silu_f32(g) * u : 0.f;
  if (valid) p.h[(long)m * p.ldh + n] = hv;
  if (p.h_bits != nullptr || p.h_nnz != nullptr) {
    const uint64_t bits = __ballot(valid && fabsf(hv) > p.t_h);
    if ((threadIdx.x & 63) == 0 && valid) {
      if (p.h_bits != nullptr) p.h_bits[(long)m * p.h_bits_ld + n / 64] = bits;
      // the mask's count: integer adds, exact in any order (cleared by the host)
      if (p.h_nnz != nullptr && bits) atomicAdd(p.h_nnz + m, (int)__popcll(bits));
    }
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
  if (cc.wdt == DT_I8) return launch_gemv_i8_m1(cc, p, smem, s);
  const bool bf = cc.wdt == DT_BF16;
  switch (cc.mt) {
    case 1: return bf ? launch_gemv_bf16_m1(cc, p, smem, s) : launch_gemv_f16_m1(cc, p, smem, s);
    case 2: return bf ? launch_gemv_bf16_m2(cc, p, smem, s) : launch_gemv_f16_m2(cc, p, smem, s);
    case 4: return bf ? launch_gemv_bf16_m4(cc, p, smem, s) : launch_gemv_f16_m4(cc, p, smem, s);
    case 8: return bf ? launch_gemv_bf16_m8(cc, p, smem, s) : launch_gemv_f16_m8(cc, p, smem, s);
    case 16: {
      if (!bf) return hipErrorInvalidValue;
      // 9..16 tokens, split rows, deterministic sum: a 16-token tile of every slice
      // is 16x larger than one token's, and one workgroup per tile loading all of
      // them sets the launch's tail; the slices are summed by a launch of its own
      // that spreads the loads over the chip
      if (cc.out == OUT_Y && p.S > 1 && !p.atomic_y) {
        GemvParams q = p;
        q.defer_sum = 1;
        hipError_t e = launch_gemv_bf16_m16(cc, q, smem, s);
        if (e != hipSuccess) return e;
        const long n = (long)p.M * p.N;
        hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((n + kThreadsHost - 1) / kThreadsHost)),
                           dim3(kThreadsHost), 0, s, p);
        return hipGetLastError();
      }
      // the gate/up stage likewise, unless it writes per-tile row lists
      if (cc.out == OUT_SWIGLU && p.S > 1 && p.o_cnt == nullptr) {
        GemvParams q = p;
        q.defer_sum = 1;
        q.zero_y = nullptr;
        hipError_t e = launch_gemv_bf16_m16(cc, q, smem, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(sum_swiglu_kernel, dim3((unsigned)((p.N + kThreadsHost - 1) / kThreadsHost), (unsigned)p.M),
                           dim3(kThreadsHost), 0, s, p);
        return hipGetLastError();
      }
      return launch_gemv_bf16_m16(cc, p, smem, s);
    }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace as
