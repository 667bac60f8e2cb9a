// Gate/up dot products over a list of FFN neurons stored neuron-major.
//
// GLASS summary, section 2.2 and section 5: a static top-k neuron mask is
// applied for the whole decode, so only the kept neurons' weights are used.
// With the FFN stored neuron-major ([d_ff, 3, d_model]: gate row, up row and
// down row of neuron j adjacent), a kept neuron's gate and up weights are one
// contiguous 2 * d_model burst.  One wave64 computes both dot products of a
// neuron against x (held in LDS as fp32), reduces them across the wave and
// writes h_j = silu(g_j) * u_j into a single-tile list; the down projection is
// then the row-gather GEMV over the same neurons' down rows.
#include "common.hpp"
#include "internal.hpp"

namespace as {

constexpr int kNThreads = 256;
constexpr int kChunkUnroll = 4;   // 16-byte chunks per row issued together

template <int WDT, int MT, bool NT>
__global__ __launch_bounds__(kNThreads) void neuron_gu_kernel(const NeuronGuParams p) {
  extern __shared__ __align__(16) float xs[];   // [MT][d_model]
  const int d = p.d_model;
  const int M = p.M;
  // eight elements per thread and step, all loads of a step issued together
  for (int i0 = threadIdx.x * 8; i0 < MT * d; i0 += kNThreads * 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = min(i0 + e, MT * d - 1), m = i / d, c = i % d;
      v[e] = load_elem(p.x, p.x_dt, (long)(m < M ? m : M - 1) * p.ldx + c);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (i0 + e < MT * d) xs[i0 + e] = (i0 + e) / d < M ? v[e] : 0.f;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int gwave = blockIdx.x * (kNThreads / 64) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (kNThreads / 64);
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.o_cnt != nullptr) p.o_cnt[0] = p.n_active;

  for (int q = gwave; q < p.n_active; q += nwaves) {
    const int j = p.idx != nullptr ? p.idx[q] : q;
    const uint16_t* wg = p.W + (long)j * p.ld_neuron;
    const uint16_t* wu = wg + p.up_off;
    float g[MT], u[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) { g[m] = 0.f; u[m] = 0.f; }
    for (int c0 = lane * 8; c0 < d; c0 += 64 * 8 * kChunkUnroll) {
      u32x4 vg[kChunkUnroll], vu[kChunkUnroll];
#pragma unroll
      for (int k = 0; k < kChunkUnroll; ++k) {
        const int c = c0 + k * 512;
        if (c < d) {
          vg[k] = load_w16<NT>(wg + c);
          vu[k] = load_w16<NT>(wu + c);
        } else {
          vg[k] = u32x4{0u, 0u, 0u, 0u};
          vu[k] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int k = 0; k < kChunkUnroll; ++k) {
        const int c = c0 + k * 512;
        if (c < d) {
          float fg[8], fu[8];
          unpack8<WDT>(vg[k], fg);
          unpack8<WDT>(vu[k], fu);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const float4 xa = *reinterpret_cast<const float4*>(xs + m * d + c);
            const float4 xb = *reinterpret_cast<const float4*>(xs + m * d + c + 4);
            const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              g[m] = fmaf(xv[e], fg[e], g[m]);
              u[m] = fmaf(xv[e], fu[e], u[m]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float gs = wave_sum(g[m]);
      const float us = wave_sum(u[m]);
      if (lane == 0 && m < M) {
        const float h = silu_f32(gs) * us;
        p.o_val[(long)q * M + m] = h;
        if (p.h_dbg != nullptr) p.h_dbg[m * p.ld_hdbg + q] = h;
      }
    }
    if (lane == 0 && p.o_idx != nullptr) p.o_idx[q] = j;
  }
}

// One or two tokens and d_model <= 512 * NK: x stays in registers instead of LDS
// (lane l holds the inputs l*8 + 512 k .. +8 that its weight loads meet), so the
// weight stream is not limited by LDS reads.  Rows 16-byte aligned.
template <int WDT, int MT, int NK, bool NT>
__global__ __launch_bounds__(kNThreads) void neuron_gu_reg_kernel(const NeuronGuParams p) {
  const int d = p.d_model, M = p.M;
  const int lane = threadIdx.x & 63;
  float xr[MT][NK][8];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = lane * 8 + k * 512;
      const int n = (m < M && c < d) ? 8 : 0;
      load_chunk<8>(p.x, p.x_dt, (long)(m < M ? m : 0) * p.ldx + (c < d ? c : 0), n, xr[m][k]);
    }
  const int gwave = blockIdx.x * (kNThreads / 64) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (kNThreads / 64);
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.o_cnt != nullptr) p.o_cnt[0] = p.n_active;
  for (int q = gwave; q < p.n_active; q += nwaves) {
    const int j = p.idx != nullptr ? p.idx[q] : q;
    const uint16_t* wg = p.W + (long)j * p.ld_neuron;
    const uint16_t* wu = wg + p.up_off;
    u32x4 vg[NK], vu[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = min(lane * 8 + k * 512, d - 8);
      vg[k] = load_w16<NT>(wg + c);
      vu[k] = load_w16<NT>(wu + c);
    }
    float g[MT], u[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) { g[m] = 0.f; u[m] = 0.f; }
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      if (lane * 8 + k * 512 < d) {
        float fg[8], fu[8];
        unpack8<WDT>(vg[k], fg);
        unpack8<WDT>(vu[k], fu);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            g[m] = fmaf(xr[m][k][e], fg[e], g[m]);
            u[m] = fmaf(xr[m][k][e], fu[e], u[m]);
          }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float gs = wave_sum(g[m]);
      const float us = wave_sum(u[m]);
      if (lane == 0 && m < M) {
        const float h = silu_f32(gs) * us;
        p.o_val[(long)q * M + m] = h;
        if (p.h_dbg != nullptr) p.h_dbg[m * p.ld_hdbg + q] = h;
      }
    }
    if (lane == 0 && p.o_idx != nullptr) p.o_idx[q] = j;
  }
}

template <int WDT, int MT>
static hipError_t launch_n(bool nt, const NeuronGuParams& p, hipStream_t s) {
  const int npw = p.neurons_per_wave > 0 ? p.neurons_per_wave : 2;
  int waves = (p.n_active + npw - 1) / npw;
  int blocks = (waves + 3) / 4;
  if (blocks < 1) blocks = 1;
  if constexpr (MT <= 2) {
    const int es = p.x_dt == DT_F32 ? 4 : 2;
    const bool aligned = (reinterpret_cast<uintptr_t>(p.x) & 15u) == 0 && (p.ldx * es) % 16 == 0 &&
                         p.d_model % 8 == 0;
    if (aligned && p.d_model <= 4096) {
      // 512-input chunks per lane row: the smallest count covering d_model
      auto pick = [&](auto k_nt, auto k_pl) { return nt ? k_nt : k_pl; };
      const int d = p.d_model;
      auto k = d <= 512    ? pick(neuron_gu_reg_kernel<WDT, MT, 1, true>, neuron_gu_reg_kernel<WDT, MT, 1, false>)
               : d <= 1024 ? pick(neuron_gu_reg_kernel<WDT, MT, 2, true>, neuron_gu_reg_kernel<WDT, MT, 2, false>)
               : d <= 2048 ? pick(neuron_gu_reg_kernel<WDT, MT, 4, true>, neuron_gu_reg_kernel<WDT, MT, 4, false>)
                           : pick(neuron_gu_reg_kernel<WDT, MT, 8, true>, neuron_gu_reg_kernel<WDT, MT, 8, false>);
      hipLaunchKernelGGL(k, dim3(blocks), dim3(kNThreads), 0, s, p);
      return hipGetLastError();
    }
  }
  const size_t smem = size_t(MT) * p.d_model * 4;
  auto k = nt ? neuron_gu_kernel<WDT, MT, true> : neuron_gu_kernel<WDT, MT, false>;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(blocks), dim3(kNThreads), smem, s, p);
  return hipGetLastError();
}

hipError_t launch_neuron_gu(int wdt, int mt, bool nt, const NeuronGuParams& p, hipStream_t s) {
  if (wdt == DT_BF16) {
    switch (mt) {
      case 1: return launch_n<DT_BF16, 1>(nt, p, s);
      case 2: return launch_n<DT_BF16, 2>(nt, p, s);
      case 4: return launch_n<DT_BF16, 4>(nt, p, s);
      case 8: return launch_n<DT_BF16, 8>(nt, p, s);
    }
  } else {
    switch (mt) {
      case 1: return launch_n<DT_F16, 1>(nt, p, s);
      case 2: return launch_n<DT_F16, 2>(nt, p, s);
      case 4: return launch_n<DT_F16, 4>(nt, p, s);
      case 8: return launch_n<DT_F16, 8>(nt, p, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace as
