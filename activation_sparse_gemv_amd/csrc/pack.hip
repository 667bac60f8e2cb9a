// Compact packing of a static neuron set (GLASS summary, section 2.2 and the
// edge-deployment discussion: the static mask keeps one compact weight subset
// resident for the whole decode).  From the input-major MLP ([d, 2, d_ff] gate/up,
// [d_ff, d] down) the kept neurons' columns and rows are copied once into dense
// [d, 2, k] and [k, d] matrices; decode then runs the dense path on them, which
// also serves batches of many tokens (the same rows for every token).
#include "common.hpp"
#include "internal.hpp"

namespace as {

constexpr int kPackThreads = 256;

// One workgroup per input row i: out[i][c][j] = gu[i][c][idx[j]], c in {gate, up}.
__global__ __launch_bounds__(kPackThreads) void pack_gate_up_kernel(const uint16_t* gu, int f, const int* idx, int k,
                                                                    uint16_t* out) {
  const long i = blockIdx.x;
  const uint16_t* src = gu + i * 2L * f;
  uint16_t* dst = out + i * 2L * k;
  for (int j0 = threadIdx.x; j0 < k; j0 += 4 * kPackThreads) {
    int n[4];
    uint16_t g[4], u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) n[q] = idx[min(j0 + q * kPackThreads, k - 1)];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      g[q] = src[n[q]];
      u[q] = src[f + n[q]];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + q * kPackThreads;
      if (j < k) {
        dst[j] = g[q];
        dst[k + j] = u[q];
      }
    }
  }
}

// One workgroup per kept neuron j: out[j][:] = dn[idx[j]][:] (rows of d 16-bit
// weights; 16-byte pieces when d % 8 == 0).
__global__ __launch_bounds__(kPackThreads) void pack_down_kernel(const uint16_t* dn, int d, const int* idx,
                                                                 uint16_t* out) {
  const long j = blockIdx.x;
  const uint16_t* src = dn + (long)idx[j] * d;
  uint16_t* dst = out + j * d;
  if (d % 8 == 0) {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst);
    for (int c = threadIdx.x; c < d / 8; c += kPackThreads) d4[c] = s4[c];
  } else {
    for (int c = threadIdx.x; c < d; c += kPackThreads) dst[c] = src[c];
  }
}

hipError_t launch_pack_neuron_set(const uint16_t* gu, const uint16_t* dn, int d, int f, const int* idx, int k,
                                  uint16_t* gu_out, uint16_t* dn_out, hipStream_t s) {
  hipLaunchKernelGGL(pack_gate_up_kernel, dim3(d), dim3(kPackThreads), 0, s, gu, f, idx, k, gu_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_down_kernel, dim3(k), dim3(kPackThreads), 0, s, dn, d, idx, dn_out);
  return hipGetLastError();
}

}  // namespace as
