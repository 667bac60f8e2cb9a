// Routed MoE experts with intra-expert activation sparsity.
//
// Intra-expert summary, system implementation: the router and the shared
// expert are kept as they are; inside each routed expert the gate projection is
// run densely to score the neurons, the low-scoring neurons are masked, and the
// remaining neurons' weights are gathered for the rest of the expert.  Here the
// score of neuron n is |silu(g_n) * u_n| (gate and up dense), the keep_k best
// neurons (ties to the smaller index) reach the down projection, and only their
// down rows (one contiguous d_model row each) are read.  Gate-score mode (TEAL
// slides, slides 5-6, CATS): the score is |silu(g_n)| alone, the neurons above a
// threshold are kept, the up row is read only for them, and the down stage takes
// the nonzero h of each (token, slot) in neuron order.
//
// Kernels (one call):
//   gate/up: (touched expert, neuron block) workgroups; each derives its expert's
//            (token, slot) items itself, and one wave per neuron computes both dot
//            products for the expert's tokens (up to 4 at a time);
//   down:    (token, slot, column tile) workgroups: the exact top-k of |h| (one
//            wave, h in registers; or, for many items, chosen by the last gate/up
//            block of each expert), the kept neurons' down rows, weight w_tj; the
//            last slot to finish a (token, tile) sums the slots in slot order into
//            Y (deterministic).
#include "moe_impl.hpp"

namespace as {

// ---------------------------------------------------------------- router
// One wave per token (route_token, topk.hpp): the token's logits staged in LDS,
// exact top-k, ordered by (logit desc, index asc), softmax over the selected.
constexpr int kRouterThreads = 64;

__global__ __launch_bounds__(kRouterThreads) void router_kernel(const float* logits, int E, int top, int* ids,
                                                                float* wts) {
  __shared__ TopkSmem sm;
  __shared__ int sel[64];
  __shared__ float z[1024];       // this token's logits (E <= 1024), read once
  const long t = blockIdx.x;
  const int lane = threadIdx.x;
  for (int i = lane; i < E; i += kRouterThreads) z[i] = logits[t * E + i];
  __syncthreads();
  route_token(z, E, top, ids + t * top, wts + t * top, sel, sm);
}

hipError_t launch_router(const float* logits, int T, int E, int top, int* ids, float* wts, hipStream_t s) {
  hipLaunchKernelGGL(router_kernel, dim3(T), dim3(kRouterThreads), 0, s, logits, E, top, ids, wts);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gate/up
template <int WDT, int NK>
__global__ __launch_bounds__(kGuThreads) void expert_gu_kernel(const MoeParams p) {
  extern __shared__ __align__(16) float xs[];   // [kGuTok][d]
  expert_gu_block<WDT, NK>(p, blockIdx.x, blockIdx.y, xs);
}

// ---------------------------------------------------------------- down
constexpr int kDnThreads = 256;
constexpr int kDnWaves = kDnThreads / 64;
constexpr int kDnRed = kDnWaves * 512;     // floats of the row-slot reduction buffer, any tile width

// Column tile of the down stage: LPR lanes cover 8 * LPR columns of a row, so a wave
// takes 64 / LPR rows at once.  512 columns (LPR 64) for many (token, slot) items;
// 128 columns (LPR 16) for at most 32 items, which would otherwise leave most CUs idle
// (one token: 8 items x 16 tiles instead of 8 x 4 workgroups, each loading a quarter
// of the kept rows' bytes).  Measured on the 128-expert, d_model 2048 layer: one
// token 38.1 us (was 40.9), four tokens 68.5 (69.1); sixteen tokens keep 512 columns.
int moe_down_lpr(int items) { return items <= 32 ? 16 : 64; }

template <int WDT, int LPR>
__global__ __launch_bounds__(kDnThreads) void expert_down_kernel(const MoeParams p) {
  constexpr int TILE = LPR * 8;            // columns per workgroup
  constexpr int RG = 64 / LPR;             // rows a wave takes at once
  constexpr int NS = kDnWaves * RG;        // row slots of the workgroup
  static_assert(NS * TILE == kDnRed, "the reduction buffer holds every slot's tile");
  extern __shared__ __align__(16) unsigned char smem[];
  // keep-set capacity: keep_k, or every neuron in gate-score mode
  const int kcap = p.gate_mode ? p.d_ff : p.keep_k;
  int* keep = reinterpret_cast<int*>(smem);                        // [kcap]
  float* kval = reinterpret_cast<float*>(smem + 4 * ((kcap + 3) & ~3));
  float* red = kval + ((kcap + 3) & ~3);                           // [NS][TILE]
  float* hs = red + kDnRed;                        // [d_ff] when d_ff > 1024 (top-k mode only)
  __shared__ TopkSmem sm;
  __shared__ int s_last;
  const int item = blockIdx.x;                  // t * top + j
  const int tile = blockIdx.y;
  const int t = item / p.top, j = item % p.top;
  const int f = p.d_ff, d = p.d_model;
  int e = p.ids[item];
  const bool valid_e = e >= 0 && e < p.E;
  if (!valid_e) e = 0;
  int kk = valid_e ? p.keep_k : 0;
  // the item's keep set by wave 0 (every tile's workgroup selects the same set);
  // an item with an invalid expert keeps nothing
  int* dbg = (p.keep_dbg != nullptr && tile == 0) ? p.keep_dbg + (long)item * p.keep_k : nullptr;
  __shared__ int s_kk;
  if (p.gate_mode) {
    // gate-score mode: the item's nonzero h, in neuron order (wave 0: one ballot per
    // 64 neurons)
    if (threadIdx.x < 64) {
      const float* h = p.h + (long)item * f;
      int run = 0;
      for (int i0 = 0; valid_e && i0 < f; i0 += 64) {
        const int i = i0 + (int)threadIdx.x;
        const float v = i < f ? h[i] : 0.f;
        const uint64_t b = __ballot(v != 0.f);
        if (v != 0.f) {
          const int pos = run + lanes_below(b);
          keep[pos] = i;
          kval[pos] = v;
        }
        run += __popcll(b);
      }
      if (threadIdx.x == 0) s_kk = run;
    }
    __syncthreads();
    kk = s_kk;
  } else if (p.keep != nullptr) {
    // chosen by the gate/up stage
    for (int r = threadIdx.x; r < kk; r += kDnThreads) {
      keep[r] = p.keep[(long)item * p.keep_k + r];
      kval[r] = p.kval[(long)item * p.keep_k + r];
    }
  } else if (threadIdx.x < 64 && kk > 0) {
    const float* h = p.h + (long)item * f;
    if (f <= 1024) item_keep_small<false>(h, f, kk, keep, kval, dbg);
    else {
      // long rows: staged in LDS by this wave, radix selection over the copy
      for (int i = threadIdx.x; i < f; i += 64) hs[i] = h[i];
      __builtin_amdgcn_wave_barrier();
      wave_topk([=](int i) { return float_key(fabsf(hs[i])); }, f, kk, keep, sm);
      __builtin_amdgcn_wave_barrier();
      for (int r = threadIdx.x; r < kk; r += 64) {
        kval[r] = hs[keep[r]];
        if (dbg != nullptr) dbg[r] = keep[r];
      }
    }
  }
  if (dbg != nullptr && !valid_e)
    for (int r = threadIdx.x; r < p.keep_k; r += kDnThreads) dbg[r] = -1;
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = wave * RG + lane / LPR, cl = lane % LPR;
  const int c0 = tile * TILE + cl * 8;
  const bool cvalid = c0 < d;
  const uint16_t* Wd = p.w_down + (long)e * f * d + (cvalid ? c0 : 0);
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  // 96 kept rows per workgroup in one batch of independent loads (77 rows: one
  // round trip)
  constexpr int U = 24 / RG;
  for (int r = slot; r < kk; r += NS * U) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load_w16<true>(Wd + (long)keep[min(r + NS * u, kk - 1)] * d);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = r + NS * u;
      const float hv = rr < kk ? kval[rr] : 0.f;
      float wf[8];
      unpack8<WDT>(w[u], wf);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(hv, wf[q], acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) red[slot * TILE + cl * 8 + q] = acc[q];
  __syncthreads();
  // the row slots' sums of column c, in slot order
  auto slot_sum = [&](int c) {
    float v = red[c];
#pragma unroll
    for (int sl = 1; sl < NS; ++sl) v += red[sl * TILE + c];
    return v;
  };
  const float wt = valid_e ? p.wts[item] : 0.f;
  if (p.atomic_y) {
    // w_tj * sum over kept neurons added straight into y (fp32, written or cleared
    // before this launch); no slot partials, no counter, no combine
    if (valid_e)
      for (int c = threadIdx.x; c < TILE; c += kDnThreads) {
        const int gc = tile * TILE + c;
        if (gc < d) unsafeAtomicAdd(reinterpret_cast<float*>(p.y) + (long)t * d + gc, wt * slot_sum(c));
      }
    return;
  }
  // partial of this (token, slot): w_tj * sum over kept neurons, coherent store
  for (int c = threadIdx.x; c < TILE; c += kDnThreads) {
    const int gc = tile * TILE + c;
    if (gc < d) store_coherent(p.partials + (long)item * d + gc, wt * slot_sum(c));
  }
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = p.counters + ((long)t * p.n_tiles + tile) * kCounterStride;
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == unsigned(p.top - 1);
    if (s_last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  (void)j;
  // both columns of a thread at once: the y values and eight slots' partials of
  // each column are loaded before any is added (one round trip for eight slots)
  constexpr int kCols = (TILE + kDnThreads - 1) / kDnThreads;
  const int top = p.top;
  int gcs[kCols];
  float v[kCols], yv[kCols];
#pragma unroll
  for (int u = 0; u < kCols; ++u) {
    const int cc = threadIdx.x + u * kDnThreads;
    gcs[u] = cc < TILE ? tile * TILE + cc : d;              // d: not a column of this tile
    v[u] = 0.f;
    yv[u] = p.accumulate ? load_elem(p.y, p.y_dt, (long)t * d + (gcs[u] < d ? gcs[u] : 0)) : 0.f;
  }
  for (int q0 = 0; q0 < top; q0 += 8) {
    // unconditional loads: slots past top re-read the last slot, columns past d
    // read column 0; both are dropped below
    float tmp[kCols][8];
#pragma unroll
    for (int u = 0; u < kCols; ++u)
#pragma unroll
      for (int qq = 0; qq < 8; ++qq)
        tmp[u][qq] = load_coherent(p.partials + ((long)t * top + min(q0 + qq, top - 1)) * d +
                                   (gcs[u] < d ? gcs[u] : 0));
#pragma unroll
    for (int u = 0; u < kCols; ++u)
#pragma unroll
      for (int qq = 0; qq < 8; ++qq)
        if (q0 + qq < top && gcs[u] < d) v[u] += tmp[u][qq];      // slot order
  }
#pragma unroll
  for (int u = 0; u < kCols; ++u)
    if (gcs[u] < d) store_elem(p.y, p.y_dt, (long)t * d + gcs[u], p.accumulate ? v[u] + yv[u] : v[u]);
}

hipError_t launch_moe_down(int wdt, const MoeParams& p, hipStream_t s) {
  const int kcap = p.gate_mode ? p.d_ff : p.keep_k;
  const size_t sm2 = size_t(8) * ((kcap + 3) & ~3) + size_t(kDnRed) * 4 +
                     (p.d_ff > 1024 && !p.gate_mode ? size_t(p.d_ff) * 4 : 0);
  const int lpr = moe_down_lpr(p.T * p.top);
  if (p.n_tiles != moe_down_tiles(p.d_model, p.T * p.top)) return hipErrorInvalidValue;
  auto k2 = lpr == 16 ? (wdt == DT_BF16 ? expert_down_kernel<DT_BF16, 16> : expert_down_kernel<DT_F16, 16>)
                      : (wdt == DT_BF16 ? expert_down_kernel<DT_BF16, 64> : expert_down_kernel<DT_F16, 64>);
  if (sm2 > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k2), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       int(sm2));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k2, dim3(p.T * p.top, p.n_tiles), dim3(kDnThreads), sm2, s, p);
  return hipGetLastError();
}

hipError_t launch_moe(int wdt, const MoeParams& p, int max_unique, hipEvent_t y_ready, hipStream_t s) {
  hipError_t e;
  const int nblk = moe_gu_blocks(p);
  const size_t sm1 = moe_gu_smem(p);
  const int nk = moe_gu_nk(p);
  auto pick = [&](auto kb, auto kf) { return wdt == DT_BF16 ? kb : kf; };
  auto k1 = nk == 0   ? pick(expert_gu_kernel<DT_BF16, 0>, expert_gu_kernel<DT_F16, 0>)
            : nk == 1 ? pick(expert_gu_kernel<DT_BF16, 1>, expert_gu_kernel<DT_F16, 1>)
            : nk == 2 ? pick(expert_gu_kernel<DT_BF16, 2>, expert_gu_kernel<DT_F16, 2>)
            : nk == 4 ? pick(expert_gu_kernel<DT_BF16, 4>, expert_gu_kernel<DT_F16, 4>)
                      : pick(expert_gu_kernel<DT_BF16, 8>, expert_gu_kernel<DT_F16, 8>);
  if (sm1 > 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1), hipFuncAttributeMaxDynamicSharedMemorySize, int(sm1));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k1, dim3(max_unique, nblk), dim3(kGuThreads), sm1, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // only the down stage touches Y: the producer of Y (another stream) need not be
  // done before the grouping and the gate/up stage
  if (y_ready != nullptr && (e = hipStreamWaitEvent(s, y_ready, 0)) != hipSuccess) return e;
  return launch_moe_down(wdt, p, s);
}

int moe_down_tiles(int d_model, int items) {
  const int tile = moe_down_lpr(items) * 8;
  return (d_model + tile - 1) / tile;
}
int moe_gu_nk_of(const MoeParams& p) { return moe_gu_nk(p); }
int moe_gu_blocks_of(const MoeParams& p) { return moe_gu_blocks(p); }
size_t moe_gu_smem_of(const MoeParams& p) { return moe_gu_smem(p); }

// ---------------------------------------------------------------- one-stream layer
// The combined launches are instantiated per token tile in moe_layer_bf16_m*.hip.
#define AS_MOE_LAYER_DECL(MT)                                                                            \
  hipError_t launch_moe_route_gu_m##MT(const MoeLayerCfg&, const GemvParams&, const GemvParams&, size_t, \
                                       hipStream_t);                                                     \
  hipError_t launch_moe_gu_down_m##MT(const MoeLayerCfg&, const MoeParams&, int, int, const GemvParams&, \
                                      size_t, hipStream_t);
AS_MOE_LAYER_DECL(1)
AS_MOE_LAYER_DECL(2)
AS_MOE_LAYER_DECL(4)
AS_MOE_LAYER_DECL(8)
#undef AS_MOE_LAYER_DECL

bool moe_layer_supported(const MoeLayerCfg& c) {
  return c.wdt == DT_BF16 && (c.mt == 1 || c.mt == 2 || c.mt == 4 || c.mt == 8) &&
         (c.lpr_r == 16 || c.lpr_r == 32 || c.lpr_r == 64) && (c.lpr_g == 32 || c.lpr_g == 64) &&
         (c.lpr_d == 16 || c.lpr_d == 64) && (c.nk == 0 || c.nk == 1 || c.nk == 2 || c.nk == 4 || c.nk == 8);
}

hipError_t launch_moe_route_gu(const MoeLayerCfg& c, const GemvParams& pr, const GemvParams& pg, size_t smem,
                               hipStream_t s) {
  if (!moe_layer_supported(c)) return hipErrorInvalidValue;
  switch (c.mt) {
    case 1: return launch_moe_route_gu_m1(c, pr, pg, smem, s);
    case 2: return launch_moe_route_gu_m2(c, pr, pg, smem, s);
    case 4: return launch_moe_route_gu_m4(c, pr, pg, smem, s);
    default: return launch_moe_route_gu_m8(c, pr, pg, smem, s);
  }
}

hipError_t launch_moe_gu_down(const MoeLayerCfg& c, const MoeParams& pm, int n_u, int n_gu, const GemvParams& pd,
                              size_t smem, hipStream_t s) {
  if (!moe_layer_supported(c)) return hipErrorInvalidValue;
  switch (c.mt) {
    case 1: return launch_moe_gu_down_m1(c, pm, n_u, n_gu, pd, smem, s);
    case 2: return launch_moe_gu_down_m2(c, pm, n_u, n_gu, pd, smem, s);
    case 4: return launch_moe_gu_down_m4(c, pm, n_u, n_gu, pd, smem, s);
    default: return launch_moe_gu_down_m8(c, pm, n_u, n_gu, pd, smem, s);
  }
}

}  // namespace as
