// Exact top-k selection with index tie-break, as a workgroup-level device routine.
//
// GLASS summary, section 2.2 (selection): the k neurons with the highest score
// form the mask.  Intra-expert summary, method section: the lowest-scoring
// neurons of a routed expert are skipped.  Both need an exact order statistic:
// here every score is mapped to an order-preserving 32-bit key, an MSB-first
// radix select over four 8-bit digits (LDS histogram) finds the k-th largest key
// T and how many keys equal to T must be taken, and a final pass in index order
// keeps every key above T plus the first such keys equal to T, so ties go to the
// smaller index.  Output: an ascending index list and a 64-bit-word bitmask.
#pragma once
#include "common.hpp"

namespace as {

// Order-preserving key of a float: larger value -> larger key; -0.0 == +0.0;
// NaN maps to 0, below every number (-inf maps to 0x007fffff).
__device__ __forceinline__ uint32_t float_key(float f) {
  if (f != f) return 0u;
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkSmem {
  unsigned hist[256];
  int wave_cnt[32];
  uint32_t prefix;
  int krem;
  int sel_bin, sel_krem;
  int run_eq, run_sel;
};

// Select the k largest of n keys (key(i) for i < n), ties to the smaller index.
// NT threads (multiple of 64, <= 1024).  Writes idx[0..k) ascending (if idx) and
// ceil(n/64) mask words (if mask).  Every thread of the workgroup must call it.
template <int NT, class KeyFn>
__device__ void block_topk(KeyFn key, int n, int k, uint64_t* mask, int* idx, TopkSmem& sm) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (k > n) k = n;
  uint32_t T = 0u;
  int take_eq = 0;
  bool all = k >= n, none = k <= 0;
  if (!all && !none) {
    if (tid == 0) { sm.prefix = 0u; sm.krem = k; }
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (32 - 8 * pass));
      for (int b = tid; b < 256; b += NT) sm.hist[b] = 0u;
      __syncthreads();
      const uint32_t prefix = sm.prefix;
      for (int i = tid; i < n; i += NT) {
        const uint32_t kk = key(i);
        if ((kk & hi_mask) == prefix) atomicAdd(&sm.hist[(kk >> shift) & 0xffu], 1u);
      }
      __syncthreads();
      if (w == 0) wave_select_bin(sm.hist, sm.krem, true, &sm.sel_bin, &sm.sel_krem);
      __syncthreads();
      if (tid == 0) {
        sm.prefix = prefix | ((uint32_t)sm.sel_bin << shift);
        sm.krem = sm.sel_krem;
      }
      __syncthreads();
    }
    T = sm.prefix;
    take_eq = sm.krem;
  }
  if (tid == 0) { sm.run_eq = 0; sm.run_sel = 0; }
  __syncthreads();
  for (int base = 0; base < n; base += NT) {
    const int i = base + tid;
    bool sel = false, eq = false;
    if (i < n) {
      if (all) sel = true;
      else if (!none) {
        const uint32_t kk = key(i);
        sel = kk > T;
        eq = kk == T;
      }
    }
    // rank of this key among the keys equal to T, in index order
    const uint64_t eqb = __ballot(eq);
    if (lane == 0) sm.wave_cnt[w] = __popcll(eqb);
    __syncthreads();
    int eq_before = sm.run_eq;
    for (int v = 0; v < w; ++v) eq_before += sm.wave_cnt[v];
    eq_before += lanes_below(eqb);
    if (eq && eq_before < take_eq) sel = true;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int v = 0; v < NW; ++v) tot += sm.wave_cnt[v];
      sm.run_eq += tot;
    }
    const uint64_t sb = __ballot(sel);
    if (mask != nullptr && lane == 0 && (base + w * 64) < n) mask[(base + w * 64) >> 6] = sb;
    __syncthreads();
    if (lane == 0) sm.wave_cnt[w] = __popcll(sb);
    __syncthreads();
    int pos = sm.run_sel;
    for (int v = 0; v < w; ++v) pos += sm.wave_cnt[v];
    pos += lanes_below(sb);
    if (sel && idx != nullptr) idx[pos] = i;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int v = 0; v < NW; ++v) tot += sm.wave_cnt[v];
      sm.run_sel += tot;
    }
    __syncthreads();
  }
}

// The same selection by a single wave, without workgroup barriers (only the
// calling wave may use `sm`; a wave's LDS operations complete in order).  For
// small n, where the barriers of the workgroup version dominate: the router's
// logits, one expert's neurons.  Writes idx[0..k) ascending.
template <class KeyFn>
__device__ void wave_topk(KeyFn key, int n, int k, int* idx, TopkSmem& sm) {
  const int lane = threadIdx.x & 63;
  if (k > n) k = n;
  if (k <= 0) return;
  const bool all = k >= n;
  uint32_t T = 0u;
  int take_eq = 0;
  if (!all) {
    uint32_t prefix = 0u;
    int krem = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (32 - 8 * pass));
      for (int b = lane; b < 256; b += 64) sm.hist[b] = 0u;
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < n; i += 64) {
        const uint32_t kk = key(i);
        if ((kk & hi_mask) == prefix) atomicAdd(&sm.hist[(kk >> shift) & 0xffu], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      wave_select_bin(sm.hist, krem, true, &sm.sel_bin, &sm.sel_krem);
      __builtin_amdgcn_wave_barrier();
      prefix |= (uint32_t)sm.sel_bin << shift;
      krem = sm.sel_krem;
      __builtin_amdgcn_wave_barrier();
    }
    T = prefix;
    take_eq = krem;
  }
  int run_eq = 0, run_sel = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    bool sel = false, eq = false;
    if (i < n) {
      if (all) sel = true;
      else {
        const uint32_t kk = key(i);
        sel = kk > T;
        eq = kk == T;
      }
    }
    const uint64_t eqb = __ballot(eq);
    if (eq && run_eq + lanes_below(eqb) < take_eq) sel = true;
    run_eq += __popcll(eqb);
    const uint64_t sb = __ballot(sel);
    if (sel && idx != nullptr) idx[run_sel + lanes_below(sb)] = i;
    run_sel += __popcll(sb);
  }
}

// The same selection by one wave with the keys in registers: key[q] is the key of
// index q * 64 + lane (n <= 64 * KPL; lanes past n hold anything).  Each radix pass
// issues the lane's histogram atomics back to back (no LDS reads of the keys), and
// the final pass walks the 64-index chunks in order with ballots.  Writes idx[0..k)
// ascending.  Called by the 64 threads of one wave.
template <int KPL>
__device__ void wave_topk_regs(const uint32_t (&key)[KPL], int n, int k, int* idx, TopkSmem& sm) {
  const int lane = threadIdx.x & 63;
  if (k > n) k = n;
  if (k <= 0) return;
  const bool all = k >= n;
  uint32_t T = 0u;
  int take_eq = 0;
  if (!all) {
    uint32_t prefix = 0u;
    int krem = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (32 - 8 * pass));
      for (int b = lane; b < 256; b += 64) sm.hist[b] = 0u;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < KPL; ++q)
        if (q * 64 + lane < n && (key[q] & hi_mask) == prefix) atomicAdd(&sm.hist[(key[q] >> shift) & 0xffu], 1u);
      __builtin_amdgcn_wave_barrier();
      wave_select_bin(sm.hist, krem, true, &sm.sel_bin, &sm.sel_krem);
      __builtin_amdgcn_wave_barrier();
      prefix |= (uint32_t)sm.sel_bin << shift;
      krem = sm.sel_krem;
      __builtin_amdgcn_wave_barrier();
    }
    T = prefix;
    take_eq = krem;
  }
  int run_eq = 0, run_sel = 0;
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    if (q * 64 >= n) break;
    const int i = q * 64 + lane;
    bool sel = false, eq = false;
    if (i < n) {
      if (all) sel = true;
      else {
        sel = key[q] > T;
        eq = key[q] == T;
      }
    }
    const uint64_t eqb = __ballot(eq);
    if (eq && run_eq + lanes_below(eqb) < take_eq) sel = true;
    run_eq += __popcll(eqb);
    const uint64_t sb = __ballot(sel);
    if (sel && idx != nullptr) idx[run_sel + lanes_below(sb)] = i;
    run_sel += __popcll(sb);
  }
}

// Routing of one token by one wave (intra-expert summary, system implementation:
// the router picks the top experts by logit and weights them by a softmax over
// the picked logits): z = the token's E logits (LDS), the exact top-`top` by
// logit (ties to the smaller expert), written in (logit desc, index asc) order to
// ids[0..top) with weights softmax over the selected logits, shifted by their
// maximum.  sel: [64] LDS scratch; E <= 1024, top <= 64.
__device__ __forceinline__ void route_token(const float* z, int E, int top, int* ids, float* wts, int* sel,
                                            TopkSmem& sm) {
  const int lane = threadIdx.x & 63;
  if (E <= 64 * 4) {
    uint32_t kr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) kr[q] = q * 64 + lane < E ? float_key(z[q * 64 + lane]) : 0u;
    wave_topk_regs<4>(kr, E, top, sel, sm);
  } else {
    wave_topk([=](int i) { return float_key(z[i]); }, E, top, sel, sm);
  }
  __builtin_amdgcn_wave_barrier();
  // lane a < top holds selection a; its rank in (logit desc, index asc) order
  int me = 0, rank = 0;
  uint32_t km = 0u;
  if (lane < top) {
    me = sel[lane];
    km = float_key(z[me]);
    for (int b = 0; b < top; ++b) {
      const int ob = sel[b];
      const uint32_t kb = float_key(z[ob]);
      rank += (kb > km) || (kb == km && ob < me);
    }
  }
  float m = lane < top ? z[me] : -INFINITY;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float ev = lane < top ? expf(z[me] - m) : 0.f;
  const float sum = wave_sum(ev);
  if (lane < top) {
    ids[rank] = me;
    wts[rank] = ev / sum;
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace as
