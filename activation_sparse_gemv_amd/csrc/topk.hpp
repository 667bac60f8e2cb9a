// Exact top-k selection with index tie-break, as a workgroup-level device routine.
//
// GLASS summary, section 2.2 (selection): the k neurons with the highest score
// form the mask.  Intra-expert summary, method section: the lowest-scoring
// neurons of a routed expert are skipped.  Both need an exact order statistic:
// here every score is mapped to an order-preserving 32-bit key, the k-th largest
// key T is found (an MSB-first radix select over four 8-bit digits with an LDS
// histogram for the workgroup and long-row forms; a bracketed count search over
// keys held in registers for one wave and at most 1024 keys), and a final pass in
// index order keeps every key above T plus the first keys equal to T, so ties go
// to the smaller index.  Output: an ascending index list (and, for the workgroup
// form, a 64-bit-word bitmask).
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
  uint32_t prefix;
  int krem;
  int sel_bin, sel_krem;
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
  // Emission.  The kept keys equal to T are the first take_eq of them in index
  // order, i.e. those at or below the index i_cut of the take_eq-th; thread t owns
  // the run [t R, t R + R) of R = ceil(n / NT) consecutive indices, and two
  // workgroup scans over the runs find i_cut and each run's first output slot.
  // The mask words come from ballots over 64 consecutive indices.
  __shared__ int s_scan[NW + 1];
  __shared__ int s_cut;
  const int R = (n + NT - 1) / NT;
  const int ra = min(tid * R, n), rb = min(ra + R, n);
  int i_cut = -1;
  if (!all && !none) {
    int ce = 0;
    for (int i = ra; i < rb; ++i) ce += (int)(key(i) == T);
    int tot;
    const int before = block_excl_scan<NT>(ce, s_scan, &tot);
    if (before < take_eq && take_eq <= before + ce) {
      int c = before;
      for (int i = ra; i < rb; ++i)
        if (key(i) == T && ++c == take_eq) {
          s_cut = i;
          break;
        }
    }
    __syncthreads();
    i_cut = s_cut;
  }
  auto selected = [&](int i) -> bool {
    if (all) return true;
    if (none) return false;
    const uint32_t kk = key(i);
    return kk > T || (kk == T && i <= i_cut);
  };
  if (idx != nullptr) {
    int cs = 0;
    for (int i = ra; i < rb; ++i) cs += (int)selected(i);
    int tot;
    int pos = block_excl_scan<NT>(cs, s_scan, &tot);
    for (int i = ra; i < rb; ++i)
      if (selected(i)) idx[pos++] = i;
  }
  if (mask != nullptr)
    for (int i0 = w * 64; i0 < n; i0 += NT) {
      const int i = i0 + lane;
      const uint64_t sb = __ballot(i < n && selected(i));
      if (lane == 0) mask[i0 >> 6] = sb;
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
// index q * 64 + lane (n <= 64 * KPL; lanes past n hold anything).  The k-th
// largest key T is bracketed: at least k keys are >= a, fewer than k are >= b.
// Each step counts the keys >= a candidate c in (a, b) (one ballot per 64 keys, no
// LDS or memory) and moves a or b to c.  Candidates alternate between a guess
// interpolated from the two counts and the midpoint, so the search takes at most
// twice the steps of bisection over 32 bits and, on smooth score distributions,
// far fewer.  When exactly k keys are >= a candidate, T is the smallest of them
// and the kept keys are those >= T; otherwise (ties at T) the final pass walks the
// 64-index chunks in order with ballots (keys above T, then the first keys equal
// to T).  Either pass calls emit(pos, q, i) for the pos-th
// selected index i = q * 64 + lane, in ascending order of i.  Called by the 64
// threads of one wave (a single wave issues one instruction per four cycles, so
// the steps are kept short and branch-free).
template <int KPL, class Emit>
__device__ void wave_topk_regs_emit(const uint32_t (&key_in)[KPL], int n, int k, Emit emit) {
  const int lane = threadIdx.x & 63;
  if (k > n) k = n;
  if (k <= 0) return;
  const bool all = k >= n;
  // lanes past n take key 0, which no candidate of the search counts (all are >= 1)
  // and no count of keys above T includes, so the counting loops need no bounds
  uint32_t key[KPL];
#pragma unroll
  for (int q = 0; q < KPL; ++q) key[q] = q * 64 + lane < n ? key_in[q] : 0u;
  uint32_t T = 0u;
  int take_eq = 0;
  if (!all) {
    uint32_t mx = 0u;
#pragma unroll
    for (int q = 0; q < KPL; ++q) mx = key[q] > mx ? key[q] : mx;
    // the largest key is at most that of +inf (0xff800000), so b does not wrap
    uint32_t a = 0u, b = wave_max_u32(mx) + 1u;
    int ca = n, cb = 0;                         // keys >= a, keys >= b
    bool exact = false;
    for (int it = 0; it < 72; ++it) {           // bisection every other step: w <= 1 before 72
      const uint32_t w = b - a;
      if (w <= 1u) break;
      uint32_t off;
      if (it & 1) {
        off = w >> 1;
      } else {
        const float fr = __fdividef((float)(ca - k), (float)(ca - cb));
        off = (uint32_t)((float)w * fr);
        off = off < 1u ? 1u : (off > w - 1u ? w - 1u : off);
      }
      const uint32_t c = a + off;
      // per-lane counts (VALU only), then one wave sum (exact: at most 1024 in fp32)
      int lc = 0;
#pragma unroll
      for (int q = 0; q < KPL; ++q) lc += key[q] >= c ? 1 : 0;
      const int cnt = (int)wave_sum((float)lc);
      if (cnt >= k) {
        a = c;
        ca = cnt;
        if (cnt == k) {
          exact = true;
          break;
        }
      } else {
        b = c;
        cb = cnt;
      }
    }
    if (exact) {
      uint32_t m = 0xffffffffu;
#pragma unroll
      for (int q = 0; q < KPL; ++q) m = (key[q] >= a && key[q] < m) ? key[q] : m;
      T = wave_min_u32(m);
    } else {
      T = a;                                    // b = a + 1: a is the k-th largest key
    }
    int gt = 0;
#pragma unroll
    for (int q = 0; q < KPL; ++q) gt += __popcll(__ballot(key[q] > T));
    take_eq = k - gt;
    // an exact count (k keys >= T) keeps every key equal to T: a plain threshold
    if (exact) {
      int run = 0;
#pragma unroll
      for (int q = 0; q < KPL; ++q) {
        const bool sel = key[q] >= T;                // lanes past n hold 0 < T
        const uint64_t sb = __ballot(sel);
        if (sel) emit(run + lanes_below(sb), q, q * 64 + lane);
        run += __popcll(sb);
      }
      return;
    }
  }
  int run_eq = 0, run_sel = 0;
#pragma unroll
  for (int q = 0; q < KPL; ++q) {
    const bool valid = q * 64 + lane < n;
    bool sel = valid && (all || key[q] > T);
    const bool eq = valid && !all && key[q] == T;
    const uint64_t eqb = __ballot(eq);
    if (eq && run_eq + lanes_below(eqb) < take_eq) sel = true;
    run_eq += __popcll(eqb);
    const uint64_t sb = __ballot(sel);
    if (sel) emit(run_sel + lanes_below(sb), q, q * 64 + lane);
    run_sel += __popcll(sb);
  }
}

// The selection above writing idx[0..k) (ascending indices).  `sm` is not used.
template <int KPL>
__device__ __forceinline__ void wave_topk_regs(const uint32_t (&key)[KPL], int n, int k, int* idx, TopkSmem& sm) {
  (void)sm;
  wave_topk_regs_emit<KPL>(key, n, k, [&](int pos, int, int i) {
    if (idx != nullptr) idx[pos] = i;
  });
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
  if (E <= 64 * 2) {
    uint32_t kr[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) kr[q] = float_key(z[min(q * 64 + lane, E - 1)]);
    wave_topk_regs<2>(kr, E, top, sel, sm);
  } else if (E <= 64 * 4) {
    uint32_t kr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) kr[q] = float_key(z[min(q * 64 + lane, E - 1)]);
    wave_topk_regs<4>(kr, E, top, sel, sm);
  } else {
    uint32_t kr[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) kr[q] = float_key(z[min(q * 64 + lane, E - 1)]);
    wave_topk_regs<16>(kr, E, top, sel, sm);
  }
  __builtin_amdgcn_wave_barrier();
  // lane a < top holds selection a; its rank in (logit desc, index asc) order
  int me = 0, rank = 0;
  uint32_t km = 0u;
  if (lane < top) {
    me = sel[lane];
    km = float_key(z[me]);
  }
  // the other selections' (index, key) from their lanes by readlane (no LDS)
  for (int b = 0; b < top; ++b) {
    const int ob = __builtin_amdgcn_readlane(me, b);
    const uint32_t kb = (uint32_t)__builtin_amdgcn_readlane((int)km, b);
    rank += (kb > km) || (kb == km && ob < me);
  }
  float m = lane < top ? z[me] : -INFINITY;
  m = wave_max(m);
  const float ev = lane < top ? expf(z[me] - m) : 0.f;
  const float sum = wave_sum(ev);
  if (lane < top) {
    ids[rank] = me;
    wts[rank] = ev / sum;
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace as
