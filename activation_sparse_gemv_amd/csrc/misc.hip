// Workspace fill, cache flush and threshold calibration kernels.
#include "common.hpp"
#include "internal.hpp"

namespace as {

__global__ void fill_kernel(u32x4* p, size_t n16, uint32_t v) {
  const u32x4 val{v, v, v, v};
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = val;
}

__global__ void fill_tail_kernel(unsigned char* p, size_t n, unsigned char v) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_pattern(void* p, size_t bytes, uint32_t v, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 > 0) {
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<u32x4*>(p), n16, v);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t tail = bytes - n16 * 16;
  if (tail > 0) {
    hipLaunchKernelGGL(fill_tail_kernel, dim3(1), dim3(16), 0, s,
                       reinterpret_cast<unsigned char*>(p) + n16 * 16, tail, (unsigned char)(v & 0xff));
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) { return launch_fill_pattern(p, bytes, 0u, s); }

// ---------------------------------------------------------------- calibration
// TEAL slides, method slide: t_p is decided from calibration data for the target
// sparsity.  Nearest-rank order statistic of |pool| by an MSB-first radix select
// over the fp32 bit pattern of |v| (for non-negative floats the bit pattern
// orders like the value; NaN patterns order above +inf).  One workgroup of 1024
// threads, four 8-bit passes with an LDS histogram: an offline step, not timed.
constexpr int kCalThreads = 1024;

__device__ __forceinline__ uint32_t abs_key(const void* pool, int dt, int64_t i) {
  return __float_as_uint(load_elem(pool, dt, i)) & 0x7fffffffu;
}

__global__ __launch_bounds__(kCalThreads) void calibrate_kernel(const void* pool, int dt, int64_t n,
                                                                int64_t rank, float* t_out) {
  __shared__ unsigned hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int64_t s_krem;
  __shared__ int s_bin, s_binrem;
  if (rank == 0) {
    if (threadIdx.x == 0) *t_out = -INFINITY;
    return;
  }
  if (threadIdx.x == 0) { s_prefix = 0u; s_krem = rank; }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (32 - 8 * pass));
    for (int b = threadIdx.x; b < 256; b += kCalThreads) hist[b] = 0u;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int64_t i = threadIdx.x; i < n; i += kCalThreads) {
      const uint32_t k = abs_key(pool, dt, i);
      if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) wave_select_bin(hist, (int)s_krem, false, &s_bin, &s_binrem);
    __syncthreads();
    if (threadIdx.x == 0) {
      s_prefix = prefix | ((uint32_t)s_bin << shift);
      s_krem = s_binrem;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *t_out = __uint_as_float(s_prefix);
}

hipError_t launch_calibrate(const void* pool, int dt, int64_t n, int64_t rank, float* t_out, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(1), dim3(kCalThreads), 0, s, pool, dt, n, rank, t_out);
  return hipGetLastError();
}

}  // namespace as
