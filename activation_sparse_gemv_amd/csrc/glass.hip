// GLASS local signal: mean |h| of every FFN neuron over the prompt tokens.
//
// GLASS summary, section 1 and 2.2: the local importance signal comes from the
// prefill-stage activations of the prompt.  Reading: local_j = (1/P) sum_t
// |silu(x_t . Wg_j) * (x_t . Wu_j)|, the magnitude of the down-projection input.
// This is a dense prefill GEMM, run once per prompt, on the matrix cores: with
// the FFN stored neuron-major a neuron's gate (and up) row is contiguous along
// the reduction dimension, so both MFMA operands are K-contiguous: the weight
// fragment of a lane is one 16-byte load, and the prompt tile (32 columns of
// every token) is staged in LDS once per k-step for the four waves.
#include <cstdlib>
#include "common.hpp"
#include "internal.hpp"

namespace as {

typedef __bf16 g_bf16x8 __attribute__((ext_vector_type(8)));
typedef float g_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLsThreads = 256;
constexpr int kLsTokBlock = 128;          // tokens per pass (8 MFMA row tiles)
constexpr int kLsLd = 40;                 // LDS row stride (elements) of the prompt tile

__global__ __launch_bounds__(kLsThreads) void local_signal_kernel(const uint16_t* X, int P, int d,
                                                                  const uint16_t* W, long ld_neuron, long up_off,
                                                                  int d_ff, float* local) {
  __shared__ __align__(16) uint16_t xt[kLsTokBlock * kLsLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int j = (blockIdx.x * 4 + wave) * 16 + li;          // this lane's neuron (B column)
  const bool jvalid = j < d_ff;
  const uint16_t* wg = W + (long)(jvalid ? j : 0) * ld_neuron;
  const uint16_t* wu = wg + up_off;
  float asum = 0.f;
  for (int t0 = 0; t0 < P; t0 += kLsTokBlock) {
    g_f32x4 accg[8], accu[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) { accg[m] = g_f32x4{0.f, 0.f, 0.f, 0.f}; accu[m] = accg[m]; }
    for (int k0 = 0; k0 < d; k0 += 32) {
      __syncthreads();
      // prompt tile: 128 tokens x 32 columns, two 16-byte vectors per thread
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int v = tid + q * kLsThreads;               // 0..511
        const int t = v >> 2, c = (v & 3) * 8;
        u32x4 val = u32x4{0u, 0u, 0u, 0u};
        if (t0 + t < P) val = *reinterpret_cast<const u32x4*>(X + (long)(t0 + t) * d + k0 + c);
        *reinterpret_cast<u32x4*>(xt + t * kLsLd + c) = val;
      }
      __syncthreads();
      const u32x4 bg = load_w16<true>(wg + k0 + 8 * g);
      const u32x4 bu = load_w16<true>(wu + k0 + 8 * g);
      const g_bf16x8 fg = __builtin_bit_cast(g_bf16x8, bg);
      const g_bf16x8 fu = __builtin_bit_cast(g_bf16x8, bu);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(xt + (m * 16 + li) * kLsLd + 8 * g);
        const g_bf16x8 fa = __builtin_bit_cast(g_bf16x8, a);
        accg[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fg, accg[m], 0, 0, 0);
        accu[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fu, accu[m], 0, 0, 0);
      }
    }
    // lane holds D[token 4g+e of each row tile][neuron li]
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + m * 16 + 4 * g + e;
        if (t < P) asum += fabsf(silu_f32(accg[m][e]) * accu[m][e]);
      }
  }
  // combine the four lane groups (tokens 4g..4g+3 of every tile) of neuron li, in a fixed order
  const float s1 = __shfl(asum, li + 16, 64), s2 = __shfl(asum, li + 32, 64), s3 = __shfl(asum, li + 48, 64);
  if (g == 0 && jvalid) local[j] = ((asum + s1) + (s2 + s3)) / (float)P;
}

// Variant for d_model % 128 == 0 (the usual case).  At 128 tokens a weight byte
// carries 128 flops, below the matrix cores' ridge, so the kernel is bound by the
// weight stream and is written to keep it full.  The reduction runs in stages of
// 128 columns: the workgroup's 128 gate/up rows of a stage are loaded
// cooperatively, 16 lanes per row (four rows of 256 contiguous bytes per wave
// instruction, against sixteen rows of 64 bytes when each lane fetches its own
// MFMA fragment), written to a double-buffered LDS tile and read back as B
// fragments; loads run two stages ahead (three register buffers), and the prompt
// tile of the next stage is loaded into registers during the current one and
// written to the other half of a double-buffered LDS tile.  The MFMA sequence of
// every accumulator (k-steps of 32 in ascending order) is the same as in the
// kernel above, so both give the same bits.
constexpr int kLsKS = 128;                 // reduction columns per stage
constexpr int kLsLdS = kLsKS + 8;          // LDS row stride (elements) of a stage tile
constexpr int kLsTileElems = kLsTokBlock * kLsLdS;
constexpr int kLsWRows = 128;              // gate and up rows of 64 neurons

__global__ __launch_bounds__(kLsThreads, 1) void local_signal_lds_kernel(const uint16_t* X, int P, int d,
                                                                         const uint16_t* W, long ld_neuron,
                                                                         long up_off, int d_ff, float* local) {
  extern __shared__ __align__(16) uint16_t lsm[];      // x tiles [2][128][kLsLdS], w tiles [2][128][kLsLdS]
  uint16_t* xs = lsm;
  uint16_t* ws = lsm + 2 * kLsTileElems;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int j = (blockIdx.x * 4 + wave) * 16 + li;
  const bool jvalid = j < d_ff;
  const int NS = d / kLsKS;
  // cooperative weight loads: chunk c of thread tid is row (tid + 256 c) / 16, 16-byte piece (tid % 16)
  const uint16_t* wrow[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int id = tid + c * kLsThreads;
    const int r = id >> 4, piece = id & 15;
    int n = blockIdx.x * 64 + (r >> 1);
    if (n >= d_ff) n = d_ff - 1;
    wrow[c] = W + (long)n * ld_neuron + ((r & 1) ? up_off : 0) + piece * 8;
  }
  float asum = 0.f;
  for (int t0 = 0; t0 < P; t0 += kLsTokBlock) {
    g_f32x4 accg[8], accu[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) { accg[m] = g_f32x4{0.f, 0.f, 0.f, 0.f}; accu[m] = accg[m]; }
    auto load_w = [&](int st, u32x4 (&b)[8]) {
      const int k0 = (st < NS ? st : NS - 1) * kLsKS;
#pragma unroll
      for (int c = 0; c < 8; ++c) b[c] = load_w16<true>(wrow[c] + k0);
    };
    auto store_w = [&](int buf, const u32x4 (&b)[8]) {
      uint16_t* dst = ws + buf * kLsTileElems;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int id = tid + c * kLsThreads;
        *reinterpret_cast<u32x4*>(dst + (id >> 4) * kLsLdS + (id & 15) * 8) = b[c];
      }
    };
    auto load_x = [&](int st, u32x4 (&r)[8]) {
      const int k0 = (st < NS ? st : NS - 1) * kLsKS;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int v = tid + q * kLsThreads;
        const int t = v >> 4, c = (v & 15) * 8;
        const int tt = t0 + t < P ? t0 + t : P - 1;
        r[q] = *reinterpret_cast<const u32x4*>(X + (long)tt * d + k0 + c);
      }
    };
    auto store_x = [&](int buf, const u32x4 (&r)[8]) {
      uint16_t* dst = xs + buf * kLsTileElems;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int v = tid + q * kLsThreads;
        *reinterpret_cast<u32x4*>(dst + (v >> 4) * kLsLdS + (v & 15) * 8) = r[q];
      }
    };
    auto compute = [&](int buf) {
      const uint16_t* xsrc = xs + buf * kLsTileElems;
      const uint16_t* wsrc = ws + buf * kLsTileElems + (2 * (wave * 16 + li)) * kLsLdS + 8 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const g_bf16x8 fg = __builtin_bit_cast(g_bf16x8, *reinterpret_cast<const u32x4*>(wsrc + 32 * q));
        const g_bf16x8 fu = __builtin_bit_cast(g_bf16x8, *reinterpret_cast<const u32x4*>(wsrc + kLsLdS + 32 * q));
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(xsrc + (m * 16 + li) * kLsLdS + 32 * q + 8 * g);
          const g_bf16x8 fa = __builtin_bit_cast(g_bf16x8, a);
          accg[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fg, accg[m], 0, 0, 0);
          accu[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fu, accu[m], 0, 0, 0);
        }
      }
    };
    u32x4 w0[8], w1[8], w2[8], xr[8];
    __syncthreads();                       // the previous token block is done with the tiles
    // stage 0 into LDS; then the loads outstanding at the loop head in the loop's
    // own order: W(1), X(1), W(2)
    load_x(0, xr);
    __builtin_amdgcn_sched_barrier(0);
    load_w(0, w0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(1, w1);
    __builtin_amdgcn_sched_barrier(0);
    store_x(0, xr);
    store_w(0, w0);
    __builtin_amdgcn_sched_barrier(0);
    load_x(1, xr);
    __builtin_amdgcn_sched_barrier(0);
    load_w(2, w2);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // Stage st: stage st + 1 (its tile and weights, loaded during earlier stages)
    // goes to LDS, the tile of stage st + 2 and the weights of stage st + 3 are
    // fetched (unconditionally; past the end the last stage is reloaded), and
    // stage st is multiplied.  Weights load three stages ahead of their use.
    // (the scheduling barriers keep the tile loads issued before the weight loads:
    // the waits above count on that order)
    auto step = [&](int st, const u32x4 (&nxt)[8], u32x4 (&refill)[8]) {
      store_x((st + 1) & 1, xr);
      store_w((st + 1) & 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      load_x(st + 2, xr);
      __builtin_amdgcn_sched_barrier(0);
      load_w(st + 3, refill);
      __builtin_amdgcn_sched_barrier(0);
      compute(st & 1);
      __syncthreads();
    };
    int st = 0;
    for (; st + 3 <= NS; st += 3) {
      step(st, w1, w0);
      step(st + 1, w2, w1);
      step(st + 2, w0, w2);
    }
    if (st < NS) step(st, w1, w0);
    if (st + 1 < NS) step(st + 1, w2, w1);
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + m * 16 + 4 * g + e;
        if (t < P) asum += fabsf(silu_f32(accg[m][e]) * accu[m][e]);
      }
  }
  const float s1 = __shfl(asum, li + 16, 64), s2 = __shfl(asum, li + 32, 64), s3 = __shfl(asum, li + 48, 64);
  if (g == 0 && jvalid) local[j] = ((asum + s1) + (s2 + s3)) / (float)P;
}

hipError_t launch_local_signal(const uint16_t* X, int P, int d, const uint16_t* W, long ld_neuron, long up_off,
                               int d_ff, float* local, hipStream_t s) {
  const int blocks = (d_ff + 63) / 64;
  if (d % kLsKS == 0) {
    const size_t smem = size_t(4) * kLsTileElems * sizeof(uint16_t);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(local_signal_lds_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(local_signal_lds_kernel, dim3(blocks), dim3(kLsThreads), smem, s, X, P, d, W, ld_neuron,
                       up_off, d_ff, local);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(local_signal_kernel, dim3(blocks), dim3(kLsThreads), 0, s, X, P, d, W, ld_neuron, up_off, d_ff,
                     local);
  return hipGetLastError();
}

}  // namespace as
