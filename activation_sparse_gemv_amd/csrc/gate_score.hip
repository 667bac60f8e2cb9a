// Gate-score neuron selection: dense gate, single-pass threshold, up over the kept.
//
// Intra-expert summary, system implementation: the gate projection runs densely
// to score every neuron, one O(n) threshold pass masks the scores (no top-k
// sort), and only the active neurons' weights enter the up and down work.  TEAL
// slides, slides 5-6 (CATS): the score is |SiLU(x W_gate)| and W_up / W_down are
// pruned, the gate is not.
//
// FFN stored neuron-major ([d_ff, 3, d_model]: gate row, up row, down row of
// neuron j adjacent).  One wave64 takes one neuron at a time: it streams the gate
// row (d_model/512 16-byte loads per lane), reduces the dot product with x (held
// in LDS as fp32) across the wave, and only if some token keeps the neuron
// (|silu(g)| > t) streams the up row.  Many small workgroups (four waves, a few
// neurons each) keep the CUs full: the hardware refills a CU as its workgroups
// finish, which balances the uneven kept counts.  h goes out densely ([M, d_ff],
// exactly 0 for a dropped neuron): the down projection is then the row-gather GEMV
// whose slices each compact their own range of h (its nonzero rows).
#include "common.hpp"
#include "internal.hpp"

namespace as {

constexpr int kGsThreads = 256;
constexpr int kGsWaves = kGsThreads / 64;

// A row's d_model / 512 (at most NK) 16-byte loads per lane, all issued together.
template <int NK, bool NT>
__device__ __forceinline__ void gs_load(const uint16_t* w, int d, u32x4 (&v)[NK]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int c = lane * 8 + k * 512;
    v[k] = c < d ? load_w16<NT>(w + c) : u32x4{0u, 0u, 0u, 0u};
  }
}

// Dot products of a loaded row with every token's x (LDS, fp32), summed over the wave.
template <int WDT, int MT, int NK>
__device__ __forceinline__ void gs_reduce(const u32x4 (&v)[NK], const float* xs, int d, float (&acc)[MT]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int c = lane * 8 + k * 512;
    if (c < d) {
      float f[8];
      unpack8<WDT>(v[k], f);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float4 xa = *reinterpret_cast<const float4*>(xs + m * d + c);
        const float4 xb = *reinterpret_cast<const float4*>(xs + m * d + c + 4);
        const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[m] = fmaf(xv[e], f[e], acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = wave_sum(acc[m]);
}

// A wave takes neurons q = wave, wave + 4, ... of its workgroup's tile; the gate
// row of the next neuron is in flight while the current neuron's up row loads, so
// a wave waits one round trip per neuron instead of two.
template <int WDT, int MT, int NK, bool NT>
__global__ __launch_bounds__(kGsThreads) void gate_score_kernel(const GateScoreParams p) {
  extern __shared__ __align__(16) float xs[];          // [MT][d_model] fp32
  __shared__ uint32_t s_keep[kGsMaxNpb];               // bit m: token m keeps the neuron
  const int d = p.d_model, M = p.M;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j0 = blockIdx.x * p.npb;
  const int nloc = min(p.npb, p.d_ff - j0);
  u32x4 vg[NK];
  if (wave < nloc) gs_load<NK, NT>(p.W + (long)(j0 + wave) * p.ld_neuron, d, vg);
  // x to LDS, eight loads in flight per thread
  for (int i0 = threadIdx.x; i0 < MT * d; i0 += 8 * kGsThreads) {
    float v[8];
    if (p.x_dt == DT_F32) {
      const float* x = reinterpret_cast<const float*>(p.x);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kGsThreads, m = i / d, c = i % d;
        v[u] = (i < MT * d && m < M) ? x[(long)m * p.ldx + c] : 0.f;
      }
    } else {
      const uint16_t* x = reinterpret_cast<const uint16_t*>(p.x);
      uint32_t b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kGsThreads, m = i / d, c = i % d;
        b[u] = (i < MT * d && m < M) ? x[(long)m * p.ldx + c] : 0u;
      }
      const bool bf = p.x_dt == DT_BF16;
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = bf ? bf16_bits_to_f32(b[u]) : f16_bits_to_f32(b[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * kGsThreads < MT * d) xs[i0 + u * kGsThreads] = v[u];
  }
  __syncthreads();
  for (int q = wave; q < nloc; q += kGsWaves) {
    const int j = j0 + q;
    const uint16_t* wg = p.W + (long)j * p.ld_neuron;
    float g[MT];
    gs_reduce<WDT, MT, NK>(vg, xs, d, g);
    float a[MT];
    uint32_t keep = 0;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      a[m] = silu_f32(g[m]);
      keep |= (uint32_t)(m < M && (p.keep_all || fabsf(a[m]) > p.t)) << m;
    }
    u32x4 vu[NK];
    if (keep != 0) gs_load<NK, NT>(wg + p.up_off, d, vu);       // uniform: g is the wave's sum
    if (q + kGsWaves < nloc) gs_load<NK, NT>(p.W + (long)(j + kGsWaves) * p.ld_neuron, d, vg);
    float h[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) h[m] = 0.f;
    if (keep != 0) {
      float u[MT];
      gs_reduce<WDT, MT, NK>(vu, xs, d, u);
#pragma unroll
      for (int m = 0; m < MT; ++m) h[m] = ((keep >> m) & 1u) ? a[m] * u[m] : 0.f;
    }
    if (lane == 0) {
      s_keep[q] = keep;
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M) {
          p.h[m * p.ldh + j] = h[m];
          if (p.a_dbg != nullptr) p.a_dbg[m * p.ldh + j] = a[m];
        }
    }
  }
  __syncthreads();
  if (wave == 0 && (p.bits != nullptr || p.nnz != nullptr)) {
    // per-token keep masks: npb divides 64, so a tile's bits of one token land in
    // one 64-bit word (cleared by the host; several tiles share a word)
    const uint32_t kb = lane < nloc ? s_keep[lane] : 0u;
    for (int m = 0; m < M; ++m) {
      const uint64_t b = __ballot((kb >> m) & 1u);
      if (lane == 0 && b != 0) {
        if (p.bits != nullptr)
          atomicOr(reinterpret_cast<unsigned long long*>(p.bits + m * p.bits_ld + j0 / 64),
                   (unsigned long long)(b << (j0 % 64)));
        if (p.nnz != nullptr) atomicAdd(p.nnz + m, (int)__popcll(b));
      }
    }
  }
}

template <int WDT, int MT, int NK>
static hipError_t launch_gs_nk(bool nt, const GateScoreParams& p, int grid, hipStream_t s) {
  const size_t smem = size_t(MT) * p.d_model * 4;
  auto k = nt ? gate_score_kernel<WDT, MT, NK, true> : gate_score_kernel<WDT, MT, NK, false>;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(kGsThreads), smem, s, p);
  return hipGetLastError();
}

// the smallest row chunk count (512 inputs per lane row) covering d_model
template <int WDT, int MT>
static hipError_t launch_gs(bool nt, const GateScoreParams& p, int grid, hipStream_t s) {
  const int d = p.d_model;
  if (d <= 1024) return launch_gs_nk<WDT, MT, 2>(nt, p, grid, s);
  if (d <= 2048) return launch_gs_nk<WDT, MT, 4>(nt, p, grid, s);
  if (d <= 4096) return launch_gs_nk<WDT, MT, 8>(nt, p, grid, s);
  return launch_gs_nk<WDT, MT, 16>(nt, p, grid, s);
}

int gate_score_grid(int d_ff, int npb) { return (d_ff + npb - 1) / npb; }

hipError_t launch_gate_score(int wdt, int mt, bool nt, const GateScoreParams& p, hipStream_t s) {
  const int grid = gate_score_grid(p.d_ff, p.npb);
  if (p.npb < 1 || p.npb > kGsMaxNpb || 64 % p.npb != 0 || p.d_model > 512 * 16) return hipErrorInvalidValue;
  if (wdt == DT_BF16) {
    switch (mt) {
      case 1: return launch_gs<DT_BF16, 1>(nt, p, grid, s);
      case 2: return launch_gs<DT_BF16, 2>(nt, p, grid, s);
      case 4: return launch_gs<DT_BF16, 4>(nt, p, grid, s);
      case 8: return launch_gs<DT_BF16, 8>(nt, p, grid, s);
    }
  } else {
    switch (mt) {
      case 1: return launch_gs<DT_F16, 1>(nt, p, grid, s);
      case 2: return launch_gs<DT_F16, 2>(nt, p, grid, s);
      case 4: return launch_gs<DT_F16, 4>(nt, p, grid, s);
      case 8: return launch_gs<DT_F16, 8>(nt, p, grid, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace as
