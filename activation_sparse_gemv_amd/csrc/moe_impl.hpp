// Routed-expert gate/up stage as a workgroup routine (used by the expert gate/up
// kernel and by the MoE layer's combined launches).
//
// Intra-expert summary, system implementation: inside each routed expert the gate
// and up projections are run densely to score the neurons.  One wave per neuron
// computes both dot products for the tokens routed to the expert and writes
// h = silu(g) * u per (token, slot) item.  In gate-score mode the gate dot
// products come first, and the up row is read only when some item's
// |silu(g)| passes the threshold (h = 0 for the items that drop the neuron).
#pragma once
#include "topk.hpp"
#include "internal.hpp"

namespace as {

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
  if (p.gate_mode) {
    // gate-score mode: the gate row first; the up row only if some item keeps n
    for (int n = n0 + wave; n < n1; n += kGuThreads / 64) {
      const uint16_t* wg = W + (long)n * 2 * d;
      u32x4 vg[NK];
#pragma unroll
      for (int k = 0; k < NK; ++k) vg[k] = load_w16<true>(wg + min(lane * 8 + k * 512, d - 8));
      float g[TK];
#pragma unroll
      for (int m = 0; m < TK; ++m) g[m] = 0.f;
#pragma unroll
      for (int k = 0; k < NK; ++k)
        if (lane * 8 + k * 512 < d) {
          float fg[8];
          unpack8<WDT>(vg[k], fg);
#pragma unroll
          for (int m = 0; m < TK; ++m)
#pragma unroll
            for (int q = 0; q < 8; ++q) g[m] = fmaf(xr[m][k][q], fg[q], g[m]);
        }
      float a[TK];
      uint32_t keep = 0;
#pragma unroll
      for (int m = 0; m < TK; ++m) {
        a[m] = silu_f32(wave_sum(g[m]));
        keep |= (uint32_t)(m < ng && fabsf(a[m]) > p.gate_t) << m;
      }
      float uu[TK];
#pragma unroll
      for (int m = 0; m < TK; ++m) uu[m] = 0.f;
      if (keep != 0) {                                   // uniform across the wave
        u32x4 vu[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) vu[k] = load_w16<true>(wg + d + min(lane * 8 + k * 512, d - 8));
#pragma unroll
        for (int k = 0; k < NK; ++k)
          if (lane * 8 + k * 512 < d) {
            float fu[8];
            unpack8<WDT>(vu[k], fu);
#pragma unroll
            for (int m = 0; m < TK; ++m)
#pragma unroll
              for (int q = 0; q < 8; ++q) uu[m] = fmaf(xr[m][k][q], fu[q], uu[m]);
          }
#pragma unroll
        for (int m = 0; m < TK; ++m) uu[m] = wave_sum(uu[m]);
      }
#pragma unroll
      for (int m = 0; m < TK; ++m)
        if (lane == 0 && m < ng) {
          const int it = items[g0 + m];
          const float h = ((keep >> m) & 1u) ? a[m] * uu[m] : 0.f;
          store_coherent(p.h + (long)it * f + n, h);
          if (p.h_dbg != nullptr) p.h_dbg[(long)it * f + n] = h;
          if (p.a_dbg != nullptr) p.a_dbg[(long)it * f + n] = a[m];
        }
    }
    return;
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
        store_coherent(p.h + (long)it * f + n, h);
        if (p.h_dbg != nullptr) p.h_dbg[(long)it * f + n] = h;
      }
    }
  }
}

// NK > 0: groups of one or two tokens take the register path (d_model <= 512 NK).
// Keep set of one (token, slot) item by one wave: the item's h (d_ff <= 64 * KPL)
// read straight into registers (coherent loads when other workgroups of the same
// launch wrote it), the exact top-k of |h| (ties to the smaller index;
// intra-expert summary, method section: the lowest-scoring neurons are skipped),
// the kept indices and their h written in ascending index order.
template <int KPL, bool COH>
__device__ __forceinline__ void item_keep_regs(const float* h, int f, int k, int* keep, float* kval, int* dbg) {
  const int lane = threadIdx.x & 63;
  float v[KPL];
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    const int i = min(q * 64 + lane, f - 1);
    v[q] = COH ? load_coherent(h + i) : h[i];
  }
  uint32_t key[KPL];
#pragma unroll
  for (int q = 0; q < KPL; ++q) key[q] = float_key(fabsf(v[q]));     // lanes past f: ignored
  wave_topk_regs_emit<KPL>(key, f, k, [&](int pos, int q, int i) {
    keep[pos] = i;
    kval[pos] = v[q];
    if (dbg != nullptr) dbg[pos] = i;
  });
}

template <bool COH>
__device__ __forceinline__ void item_keep_small(const float* h, int f, int k, int* keep, float* kval, int* dbg) {
  if (f <= 256) item_keep_regs<4, COH>(h, f, k, keep, kval, dbg);
  else if (f <= 512) item_keep_regs<8, COH>(h, f, k, keep, kval, dbg);
  else if (f <= 768) item_keep_regs<12, COH>(h, f, k, keep, kval, dbg);
  else item_keep_regs<16, COH>(h, f, k, keep, kval, dbg);
}

// Workgroup (u, nb): the u-th touched expert's neurons [nb * neurons_per_block, ...).
// xs: [kGuTok][d_model] fp32 of dynamic LDS.
template <int WDT, int NK>
__device__ __forceinline__ void expert_gu_block(const MoeParams& p, int u, int nb, float* xs) {
  __shared__ int s_items[256];
  __shared__ int s_mark[1024];
  __shared__ int s_gscan[kGuThreads / 64 + 1];
  int cnt = 0;
  const int e = gu_group(p, u, s_items, s_mark, s_gscan, &cnt);
  if (e < 0) return;
  const int d = p.d_model, f = p.d_ff;
  const int st = 0, en = cnt;
  const int* items = s_items;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = nb * p.neurons_per_block;
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
    if (p.gate_mode) {
      // gate-score mode over the staged tokens: gate dot products first, the up
      // row only if some item keeps the neuron
      for (int n = n0 + wave; n < n1; n += kGuThreads / 64) {
        const uint16_t* wg = W + (long)n * 2 * d;
        float g[kGuTok], uu[kGuTok];
#pragma unroll
        for (int m = 0; m < kGuTok; ++m) { g[m] = 0.f; uu[m] = 0.f; }
        auto dots = [&](const uint16_t* wr, float (&acc)[kGuTok]) {
          for (int c0 = lane * 8; c0 < d; c0 += 64 * 8 * 4) {
            u32x4 vw[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) vw[k] = load_w16<true>(wr + min(c0 + k * 512, d - 8));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int c = c0 + k * 512;
              if (c < d) {
                float fw[8];
                unpack8<WDT>(vw[k], fw);
#pragma unroll
                for (int m = 0; m < kGuTok; ++m) {
                  const float4 xa = *reinterpret_cast<const float4*>(xs + m * d + c);
                  const float4 xb = *reinterpret_cast<const float4*>(xs + m * d + c + 4);
                  const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                  for (int q = 0; q < 8; ++q) acc[m] = fmaf(xv[q], fw[q], acc[m]);
                }
              }
            }
          }
#pragma unroll
          for (int m = 0; m < kGuTok; ++m) acc[m] = wave_sum(acc[m]);
        };
        dots(wg, g);
        float a[kGuTok];
        uint32_t keep = 0;
#pragma unroll
        for (int m = 0; m < kGuTok; ++m) {
          a[m] = silu_f32(g[m]);
          keep |= (uint32_t)(m < ng && fabsf(a[m]) > p.gate_t) << m;
        }
        if (keep != 0) dots(wg + d, uu);                 // uniform across the wave
#pragma unroll
        for (int m = 0; m < kGuTok; ++m)
          if (lane == 0 && m < ng) {
            const int it = items[g0 + m];
            const float h = ((keep >> m) & 1u) ? a[m] * uu[m] : 0.f;
            store_coherent(p.h + (long)it * f + n, h);
            if (p.h_dbg != nullptr) p.h_dbg[(long)it * f + n] = h;
            if (p.a_dbg != nullptr) p.a_dbg[(long)it * f + n] = a[m];
          }
      }
      continue;
    }
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
          store_coherent(p.h + (long)it * f + n, h);
          if (p.h_dbg != nullptr) p.h_dbg[(long)it * f + n] = h;
        }
      }
    }
  }
  if (p.keep == nullptr) return;
  // The last neuron block of the expert to finish chooses every item's keep set:
  // the h stores above are device-coherent and complete before the counter
  // increment (the protocol of the split-K combine).
  __shared__ int s_last;
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned nblk = (unsigned)((f + p.neurons_per_block - 1) / p.neurons_per_block);
    const unsigned prev = __hip_atomic_fetch_add(p.gu_cnt + (long)u * kCounterStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == nblk - 1;
    if (s_last) __hip_atomic_store(p.gu_cnt + (long)u * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last || p.keep_k <= 0) return;
  for (int m = wave; m < en; m += kGuThreads / 64) {
    const int it = items[m];
    const long o = (long)it * p.keep_k;
    item_keep_small<true>(p.h + (long)it * f, f, p.keep_k, p.keep + o, p.kval + o,
                          p.keep_dbg != nullptr ? p.keep_dbg + o : nullptr);
  }
}

// Launch shape of the gate/up stage: inputs held in registers for one or two tokens
// when rows are aligned (NK 512-input chunks per lane, 0 = LDS staging only),
// neuron blocks per expert, and the LDS staging of kGuTok token rows.
inline int moe_gu_nk(const MoeParams& p) {
  const int d = p.d_model;
  return (!p.x_vec || d > 4096) ? 0 : d <= 512 ? 1 : d <= 1024 ? 2 : d <= 2048 ? 4 : 8;
}
inline int moe_gu_blocks(const MoeParams& p) { return (p.d_ff + p.neurons_per_block - 1) / p.neurons_per_block; }
inline size_t moe_gu_smem(const MoeParams& p) { return size_t(kGuTok) * p.d_model * 4; }

}  // namespace as
