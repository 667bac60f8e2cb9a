// The MoE layer's combined launches: two independent pieces of work of one layer
// share a launch, so the layer runs on one stream in three launches and no piece
// waits on another queue.
//
// Intra-expert summary, system implementation: the router and the shared expert
// are unchanged, the routed experts score their neurons densely (gate and up) and
// read only the kept neurons' down rows.  The pieces that do not depend on each
// other run side by side:
//   launch 1: router logits GEMV (its last workgroup routes every token)
//             | shared expert gate/up GEMV (split-K partials stored unsummed);
//   launch 2: routed experts' gate/up (needs the routing)
//             | shared expert down projection (sums the gate/up partials, SwiGLU,
//               writes Y);
//   launch 3: routed experts' down stage (exact top keep_k, gathered rows), added
//             onto Y (moe.hip).
// Workgroups of the first piece come first in the grid.  The pieces share nothing
// but the launch: each is the same workgroup routine, with the same parameters,
// as in its own kernel, so the results are the bits of the separate launches.
#pragma once
#include "gather_gemv_impl.hpp"
#include "moe_impl.hpp"

namespace as {

template <int WDT, int MT, int LPR_R, int LPR_G>
__global__ __launch_bounds__(kThreads, 2) void moe_route_gu_kernel(const GemvParams pr, const GemvParams pg) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x;
  if (b < pr.S) {   // router: one column tile, pr.S row slices
    gemv_item<WDT, MT, LPR_R, IN_ALL, OUT_ROUTER, false, true, 0>(pr, 0, b, b, pr.S, 0, pr.n_lt, smem);
    return;
  }
  const int g = b - pr.S, sl = g / pg.n_tiles;
  gemv_item<WDT, MT, LPR_G, IN_ALL, OUT_PARTS, true, true, 0>(pg, g % pg.n_tiles, sl, sl, pg.S, 0, pg.n_lt, smem);
}

// n_u touched experts at most; workgroup b < n_gu is (expert u, neuron block) =
// (b % n_u, b / n_u), the order of the expert gate/up kernel's two-dimensional grid.
template <int WDT, int MT, int NK, int LPR_D>
__global__ __launch_bounds__(kThreads, 2) void moe_gu_down_kernel(const MoeParams pm, int n_u, int n_gu,
                                                                  const GemvParams pd) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x;
  if (b < n_gu) {
    expert_gu_block<WDT, NK>(pm, b % n_u, b / n_u, reinterpret_cast<float*>(smem));
    return;
  }
  const int g = b - n_gu, sl = g / pd.n_tiles;
  gemv_item<WDT, MT, LPR_D, IN_PARTS, OUT_Y, false, true, 0>(pd, g % pd.n_tiles, sl, sl, pd.S, 0, pd.n_lt, smem);
}

template <class K>
hipError_t moe_allow_smem(K k, size_t smem) {
  if (smem <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
}

template <int WDT, int MT, int LPR_R>
hipError_t moe_route_gu_lprg(const MoeLayerCfg& c, const GemvParams& pr, const GemvParams& pg, size_t smem,
                             hipStream_t s) {
  auto k = c.lpr_g == 32 ? moe_route_gu_kernel<WDT, MT, LPR_R, 32> : moe_route_gu_kernel<WDT, MT, LPR_R, 64>;
  if (c.lpr_g != 32 && c.lpr_g != 64) return hipErrorInvalidValue;
  hipError_t e = moe_allow_smem(k, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(pr.S + pg.n_tiles * pg.S), dim3(kThreads), smem, s, pr, pg);
  return hipGetLastError();
}

template <int WDT, int MT>
hipError_t moe_route_gu_pick(const MoeLayerCfg& c, const GemvParams& pr, const GemvParams& pg, size_t smem,
                             hipStream_t s) {
  switch (c.lpr_r) {
    case 16: return moe_route_gu_lprg<WDT, MT, 16>(c, pr, pg, smem, s);
    case 32: return moe_route_gu_lprg<WDT, MT, 32>(c, pr, pg, smem, s);
    case 64: return moe_route_gu_lprg<WDT, MT, 64>(c, pr, pg, smem, s);
    default: return hipErrorInvalidValue;
  }
}

template <int WDT, int MT, int NK>
hipError_t moe_gu_down_lprd(const MoeLayerCfg& c, const MoeParams& pm, int n_u, int n_gu, const GemvParams& pd,
                            size_t smem, hipStream_t s) {
  auto k = c.lpr_d == 16 ? moe_gu_down_kernel<WDT, MT, NK, 16> : moe_gu_down_kernel<WDT, MT, NK, 64>;
  if (c.lpr_d != 16 && c.lpr_d != 64) return hipErrorInvalidValue;
  hipError_t e = moe_allow_smem(k, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(n_gu + pd.n_tiles * pd.S), dim3(kThreads), smem, s, pm, n_u, n_gu, pd);
  return hipGetLastError();
}

template <int WDT, int MT>
hipError_t moe_gu_down_pick(const MoeLayerCfg& c, const MoeParams& pm, int n_u, int n_gu, const GemvParams& pd,
                            size_t smem, hipStream_t s) {
  switch (c.nk) {
    case 0: return moe_gu_down_lprd<WDT, MT, 0>(c, pm, n_u, n_gu, pd, smem, s);
    case 1: return moe_gu_down_lprd<WDT, MT, 1>(c, pm, n_u, n_gu, pd, smem, s);
    case 2: return moe_gu_down_lprd<WDT, MT, 2>(c, pm, n_u, n_gu, pd, smem, s);
    case 4: return moe_gu_down_lprd<WDT, MT, 4>(c, pm, n_u, n_gu, pd, smem, s);
    case 8: return moe_gu_down_lprd<WDT, MT, 8>(c, pm, n_u, n_gu, pd, smem, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace as
