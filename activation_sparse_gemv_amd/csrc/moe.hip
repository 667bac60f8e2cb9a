// Routed MoE experts with intra-expert activation sparsity.
//
// Intra-expert summary, system implementation: the router and the shared
// expert are kept as they are; inside each routed expert the gate projection is
// run densely to score the neurons, the low-scoring neurons are masked, and the
// remaining neurons' weights are gathered for the rest of the expert.  Here the
// score of neuron n is |silu(g_n) * u_n| (gate and up dense), the keep_k best
// neurons (ties to the smaller index) reach the down projection, and only their
// down rows (one contiguous d_model row each) are read.
//
// Kernels (one call):
//   group:   one workgroup sorts the (token, slot) assignments by expert, so the
//            weights of an expert are read once for all tokens routed to it;
//   gate/up: (touched expert, neuron block) workgroups; one wave per neuron
//            computes both dot products for up to 4 tokens at a time;
//   down:    (token, slot, column tile) workgroups: exact top-k of |h|, gathered
//            down rows, weight w_tj; the last slot to finish a (token, tile)
//            sums the slots in slot order into Y (deterministic).
#include "topk.hpp"
#include "internal.hpp"

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

// ---------------------------------------------------------------- grouping
// The (token, slot) items routed to an expert, computed by every gate/up
// workgroup for itself (at most 256 items and 1024 experts, so this is a few LDS
// passes and cheaper than a launch of its own): the touched experts in ascending
// order, the u-th of them, and its items in ascending item order (t * top + j).
// Items with an id outside [0, E) are dropped (they contribute nothing).  Returns
// the expert id, or -1 when fewer than u + 1 experts are touched.
constexpr int kGuThreads = 256;

__device__ __forceinline__ int gu_group(const MoeParams& p, int u, int* s_items, int* s_mark, int* s_scan,
                                        int* cnt_out) {
  __shared__ int s_e;
  const int tid = threadIdx.x, E = p.E, n = p.T * p.top;
  for (int e = tid; e < E; e += kGuThreads) s_mark[e] = 0;
  if (tid == 0) s_e = -1;
  __syncthreads();
  int my = -1;
  if (tid < n) {
    my = p.ids[tid];
    if (my < 0 || my >= E) my = -1;
    if (my >= 0) s_mark[my] = 1;
  }
  __syncthreads();
  // u-th touched expert: thread tid owns experts [tid * per, tid * per + per)
  const int per = (E + kGuThreads - 1) / kGuThreads;
  int c = 0;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) c += s_mark[e];
  }
  int tot;
  int off = block_excl_scan<kGuThreads>(c, s_scan, &tot);
  if (u >= off && u < off + c) {
    for (int q = 0; q < per; ++q) {
      const int e = tid * per + q;
      if (e < E && s_mark[e]) {
        if (off == u) s_e = e;
        ++off;
      }
    }
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return -1;
  const int flag = (my == e) ? 1 : 0;
  int cnt;
  const int pos = block_excl_scan<kGuThreads>(flag, s_scan, &cnt);
  if (flag) s_items[pos] = tid;
  __syncthreads();
  *cnt_out = cnt;
  return e;
}

constexpr int kGuTok = 4;   // tokens per pass

// One or two tokens of an expert: the tokens' inputs stay in registers (lane l
// holds inputs l*8 + 512 k .. +8, the columns its weight loads meet), so the
// weight stream is not limited by LDS reads.  d_model <= 512 * NK, aligned rows.
template <int WDT, int TK, int NK>
__device__ __forceinline__ void expert_neurons_reg(const MoeParams& p, const uint16_t* W, const int* items, int g0,
                                                   int ng, int n0, int n1) {
  const int d = p.d_model, f = p.d_ff;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float xr[TK][NK][8];
#pragma unroll
  for (int m = 0; m < TK; ++m) {
    const long row = (long)(items[g0 + (m < ng ? m : ng - 1)] / p.top) * p.ldx;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = lane * 8 + k * 512;
      load_chunk<8>(p.x, p.x_dt, row + (c < d ? c : 0), (m < ng && c < d) ? 8 : 0, xr[m][k]);
    }
  }
  for (int n = n0 + wave; n < n1; n += kGuThreads / 64) {
    const uint16_t* wg = W + (long)n * 2 * d;
    const uint16_t* wu = wg + d;
    u32x4 vg[NK], vu[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = min(lane * 8 + k * 512, d - 8);
      vg[k] = load_w16<true>(wg + c);
      vu[k] = load_w16<true>(wu + c);
    }
    float g[TK], uu[TK];
#pragma unroll
    for (int m = 0; m < TK; ++m) { g[m] = 0.f; uu[m] = 0.f; }
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      if (lane * 8 + k * 512 < d) {
        float fg[8], fu[8];
        unpack8<WDT>(vg[k], fg);
        unpack8<WDT>(vu[k], fu);
#pragma unroll
        for (int m = 0; m < TK; ++m)
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            g[m] = fmaf(xr[m][k][q], fg[q], g[m]);
            uu[m] = fmaf(xr[m][k][q], fu[q], uu[m]);
          }
      }
    }
#pragma unroll
    for (int m = 0; m < TK; ++m) {
      const float gs = wave_sum(g[m]);
      const float us = wave_sum(uu[m]);
      if (lane == 0 && m < ng) {
        const int it = items[g0 + m];
        const float h = silu_f32(gs) * us;
        p.h[(long)it * f + n] = h;
        if (p.h_dbg != nullptr) p.h_dbg[(long)it * f + n] = h;
      }
    }
  }
}

// NK > 0: groups of one or two tokens take the register path (d_model <= 512 NK).
template <int WDT, int NK>
__global__ __launch_bounds__(kGuThreads) void expert_gu_kernel(const MoeParams p) {
  extern __shared__ __align__(16) float xs[];   // [kGuTok][d]
  __shared__ int s_items[256];
  __shared__ int s_mark[1024];
  __shared__ int s_gscan[kGuThreads / 64 + 1];
  const int u = blockIdx.x;
  int cnt = 0;
  const int e = gu_group(p, u, s_items, s_mark, s_gscan, &cnt);
  if (e < 0) return;
  const int d = p.d_model, f = p.d_ff;
  const int st = 0, en = cnt;
  const int* items = s_items;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.y * p.neurons_per_block;
  const int n1 = min(n0 + p.neurons_per_block, f);
  const uint16_t* W = p.w_gu + (long)e * f * 2 * d;
  for (int g0 = st; g0 < en; g0 += kGuTok) {
    const int ng = min(kGuTok, en - g0);
    if constexpr (NK > 0) {
      if (ng <= 2) {
        if (ng == 1) expert_neurons_reg<WDT, 1, NK>(p, W, items, g0, ng, n0, n1);
        else expert_neurons_reg<WDT, 2, NK>(p, W, items, g0, ng, n0, n1);
        continue;
      }
    }
    __syncthreads();
    if (p.x_vec) {
      // 16-byte loads of the group's token rows, issued together, staged as fp32
      const bool f32 = p.x_dt == DT_F32, bf = p.x_dt == DT_BF16;
      const int per = f32 ? 4 : 8, nv = d / per, tot = kGuTok * nv;
      for (int j0 = threadIdx.x; j0 < tot; j0 += 4 * kGuThreads) {
        u32x4 raw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = min(j0 + q * kGuThreads, tot - 1);
          const int m = min(j / nv, ng - 1), vi = j % nv;
          const long e0 = (long)(items[g0 + m] / p.top) * p.ldx + (long)vi * per;
          raw[q] = f32 ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(p.x) + e0)
                       : *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.x) + e0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + q * kGuThreads;
          if (j < tot) {
            const int m = j / nv, vi = j % nv;
            float4* dst = reinterpret_cast<float4*>(xs + m * d + vi * per);
            const uint32_t w4[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
            const bool live = m < ng;
            if (f32) {
              dst[0] = live ? make_float4(__uint_as_float(w4[0]), __uint_as_float(w4[1]), __uint_as_float(w4[2]),
                                          __uint_as_float(w4[3]))
                            : make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
              float fv[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t hb = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
                fv[e] = live ? (bf ? bf16_bits_to_f32(hb) : f16_bits_to_f32(hb)) : 0.f;
              }
              dst[0] = make_float4(fv[0], fv[1], fv[2], fv[3]);
              dst[1] = make_float4(fv[4], fv[5], fv[6], fv[7]);
            }
          }
        }
      }
    } else {
      for (int i = threadIdx.x; i < kGuTok * d; i += kGuThreads) {
        const int m = i / d, c = i % d;
        float v = 0.f;
        if (m < ng) v = load_elem(p.x, p.x_dt, (long)(items[g0 + m] / p.top) * p.ldx + c);
        xs[i] = v;
      }
    }
    __syncthreads();
    for (int n = n0 + wave; n < n1; n += kGuThreads / 64) {
      const uint16_t* wg = W + (long)n * 2 * d;
      const uint16_t* wu = wg + d;
      float g[kGuTok], uu[kGuTok];
#pragma unroll
      for (int m = 0; m < kGuTok; ++m) { g[m] = 0.f; uu[m] = 0.f; }
      for (int c0 = lane * 8; c0 < d; c0 += 64 * 8 * 4) {
        u32x4 vg[4], vu[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int c = min(c0 + k * 512, d - 8);
          vg[k] = load_w16<true>(wg + c);
          vu[k] = load_w16<true>(wu + c);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int c = c0 + k * 512;
          if (c < d) {
            float fg[8], fu[8];
            unpack8<WDT>(vg[k], fg);
            unpack8<WDT>(vu[k], fu);
#pragma unroll
            for (int m = 0; m < kGuTok; ++m) {
              const float4 xa = *reinterpret_cast<const float4*>(xs + m * d + c);
              const float4 xb = *reinterpret_cast<const float4*>(xs + m * d + c + 4);
              const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                g[m] = fmaf(xv[q], fg[q], g[m]);
                uu[m] = fmaf(xv[q], fu[q], uu[m]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < kGuTok; ++m) {
        const float gs = wave_sum(g[m]);
        const float us = wave_sum(uu[m]);
        if (lane == 0 && m < ng) {
          const int it = items[g0 + m];
          const float h = silu_f32(gs) * us;
          p.h[(long)it * f + n] = h;
          if (p.h_dbg != nullptr) p.h_dbg[(long)it * f + n] = h;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- down
constexpr int kDnThreads = 256;
constexpr int kDnLpr = 64;                 // one wave covers 512 columns of one row
constexpr int kDnTile = kDnLpr * 8;

// Workgroup copy of n floats to LDS, eight loads in flight per thread.
__device__ __forceinline__ void copy_to_lds_f32(float* dst, const float* src, int n) {
  for (int j = threadIdx.x; j < n; j += 8 * kDnThreads) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[min(j + u * kDnThreads, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j + u * kDnThreads < n) dst[j + u * kDnThreads] = v[u];
  }
}

template <int WDT>
__global__ __launch_bounds__(kDnThreads) void expert_down_kernel(const MoeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* keep = reinterpret_cast<int*>(smem);                        // [keep_k]
  float* kval = reinterpret_cast<float*>(smem + 4 * ((p.keep_k + 3) & ~3));
  float* red = kval + ((p.keep_k + 3) & ~3);                       // [4][kDnTile]
  float* hs = red + 4 * kDnTile;                                   // [d_ff] this item's h
  __shared__ TopkSmem sm;
  __shared__ int s_last;
  const int item = blockIdx.x;                  // t * top + j
  const int tile = blockIdx.y;
  const int t = item / p.top, j = item % p.top;
  const int f = p.d_ff, d = p.d_model;
  int e = p.ids[item];
  const bool valid_e = e >= 0 && e < p.E;
  if (!valid_e) e = 0;
  const float* h = p.h + (long)item * f;
  const int kk = valid_e ? p.keep_k : 0;
  copy_to_lds_f32(hs, h, f);
  __syncthreads();
  // the exact top-k of |h| by one wave over the staged row (no workgroup barriers
  // inside the selection); the other waves wait at the barrier below
  if (threadIdx.x < 64) {
    if (f <= 64 * 16) {
      uint32_t kr[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = q * 64 + threadIdx.x;
        kr[q] = i < f ? float_key(fabsf(hs[i])) : 0u;
      }
      wave_topk_regs<16>(kr, f, kk, keep, sm);
    } else {
      wave_topk([=](int i) { return float_key(fabsf(hs[i])); }, f, kk, keep, sm);
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < kk; r += kDnThreads) kval[r] = hs[keep[r]];
  if (p.keep_dbg != nullptr && tile == 0)
    for (int r = threadIdx.x; r < p.keep_k; r += kDnThreads) p.keep_dbg[(long)item * p.keep_k + r] = kk ? keep[r] : -1;
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = tile * kDnTile + lane * 8;
  const bool cvalid = c0 < d;
  const uint16_t* Wd = p.w_down + (long)e * f * d + (cvalid ? c0 : 0);
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  // up to 24 kept rows per wave in one batch of independent loads (77 rows: one
  // round trip for the four waves)
  constexpr int U = 24;
  for (int r = wave; r < kk; r += 4 * U) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load_w16<true>(Wd + (long)keep[min(r + 4 * u, kk - 1)] * d);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = r + 4 * u;
      const float hv = rr < kk ? kval[rr] : 0.f;
      float wf[8];
      unpack8<WDT>(w[u], wf);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(hv, wf[q], acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) red[wave * kDnTile + lane * 8 + q] = acc[q];
  __syncthreads();
  const float wt = valid_e ? p.wts[item] : 0.f;
  // partial of this (token, slot): w_tj * sum over kept neurons, coherent store
  for (int c = threadIdx.x; c < kDnTile; c += kDnThreads) {
    const int gc = tile * kDnTile + c;
    if (gc < d) {
      const float v = red[c] + red[kDnTile + c] + red[2 * kDnTile + c] + red[3 * kDnTile + c];
      store_coherent(p.partials + (long)item * d + gc, wt * v);
    }
  }
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = p.counters + (long)t * p.n_tiles + tile;
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == unsigned(p.top - 1);
    if (s_last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  (void)j;
  for (int c = threadIdx.x; c < kDnTile; c += kDnThreads) {
    const int gc = tile * kDnTile + c;
    if (gc < d) {
      float tmp[32];
      const int top = p.top;
#pragma unroll
      for (int q = 0; q < 32; ++q)
        tmp[q] = q < top ? load_coherent(p.partials + ((long)t * top + q) * d + gc) : 0.f;
      float v = 0.f;
      for (int q = 0; q < top; ++q) v += tmp[q];
      if (p.accumulate) v += load_elem(p.y, p.y_dt, (long)t * d + gc);
      store_elem(p.y, p.y_dt, (long)t * d + gc, v);
    }
  }
}

hipError_t launch_moe(int wdt, const MoeParams& p, int max_unique, hipEvent_t y_ready, hipStream_t s) {
  hipError_t e;
  const int nblk = (p.d_ff + p.neurons_per_block - 1) / p.neurons_per_block;
  const size_t sm1 = size_t(kGuTok) * p.d_model * 4;
  const int d = p.d_model;
  const int nk = (!p.x_vec || d > 4096) ? 0 : d <= 512 ? 1 : d <= 1024 ? 2 : d <= 2048 ? 4 : 8;
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
  const size_t sm2 = size_t(8) * ((p.keep_k + 3) & ~3) + size_t(4) * kDnTile * 4 + size_t(p.d_ff) * 4;
  auto k2 = wdt == DT_BF16 ? expert_down_kernel<DT_BF16> : expert_down_kernel<DT_F16>;
  hipLaunchKernelGGL(k2, dim3(p.T * p.top, p.n_tiles), dim3(kDnThreads), sm2, s, p);
  return hipGetLastError();
}

int moe_down_tiles(int d_model) { return (d_model + kDnTile - 1) / kDnTile; }

}  // namespace as
