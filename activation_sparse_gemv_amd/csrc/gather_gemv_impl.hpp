// Row-gather GEMV for activation-sparse decode on gfx950.
//
// TEAL slides, slide 11 (Hardware-Aware Acceleration): the mask is generated
// inside the sparse kernel and only the weight rows of surviving inputs are
// loaded; the mask itself is never stored.  Here W is input-major ([K, N]
// row-major), so the weights of one surviving input neuron are one contiguous
// row and every load below is a coalesced 16-byte-per-lane burst.
//
// Work decomposition (one launch):
//   * every workgroup rebuilds the compacted list of surviving rows from the
//     8 KB input vector (wave64 ballots + a workgroup scan), keeping only the
//     slice of the list it owns: slices split the list evenly, so work is
//     balanced whatever the mask looks like;
//   * the grid is n_tiles column tiles x S slices; a workgroup streams its
//     slice of rows for its tile's columns and accumulates in fp32 registers;
//   * the S partial tiles are combined by the last workgroup to finish a tile
//     (device-coherent partial stores and a per-tile counter), always in slice
//     order so the result is bitwise reproducible, and that workgroup runs the
//     epilogue: store y, or the SwiGLU step h = silu(g) * u, the |h| > t_h mask
//     and a per-tile compacted list that feeds the down projection.  On request
//     (atomic_y) a y-storing launch skips that combine instead: every slice adds
//     its tile into an fp32 y with atomic adds, in no fixed order.
#pragma once
#include <atomic>
#include "common.hpp"
#include "internal.hpp"
#include "topk.hpp"

namespace as {

constexpr int kThreads = 256;
// Rows whose weight loads a lane keeps in flight per main-loop step: one token
// has room for sixteen (the loop is bound by loads in flight per CU: measured on
// the 4096 x 2 x 14336 gather, 8 rows per lane left it ~15% below the rate that
// 16 rows reach); several tokens keep eight (their accumulators take the room).
// Phase timeline, compiled into libactsparse_timeline.so only (AS_PHASE_TIMELINE):
// thread 0 of each workgroup writes the device's 100 MHz constant clock into slot
// `slot` of its 16 words at phase boundaries.  Slots: 0 entry, 1 prologue done,
// 2 main loop done (thread 0's wave), 3 slot reduction done, 4 partial tile stored
// and complete, 5 tile counter returned, 6 output written (last workgroup of a
// tile), 7 rows gathered (a count, not a time), 8 input of the prologue arrived, 9
// prologue scan (IN_THRESH) or SwiGLU staging (IN_PARTS) done, 10 h exports done,
// 11 split points (IN_THRESH), 12 row list written by thread 0's wave, 13 barrier
// after the row list passed.
#ifdef AS_PHASE_TIMELINE
#define AS_PHASE(p, slot)                                                                    \
  do {                                                                                       \
    if ((p).phase_tl != nullptr && threadIdx.x == 0)                                         \
      (p).phase_tl[(long)blockIdx.x * 16 + (slot)] = __builtin_amdgcn_s_memrealtime();       \
  } while (0)
#define AS_PHASE_VAL(p, slot, v)                                                             \
  do {                                                                                       \
    if ((p).phase_tl != nullptr && threadIdx.x == 0) (p).phase_tl[(long)blockIdx.x * 16 + (slot)] = (v); \
  } while (0)
// orders a stamp after the arrival of `v` (the empty asm reads its register)
#define AS_PHASE_AFTER(v) asm volatile("" ::"v"(v))
#else
#define AS_PHASE(p, slot) do {} while (0)
#define AS_PHASE_VAL(p, slot, v) do {} while (0)
#define AS_PHASE_AFTER(v) do {} while (0)
#endif

template <int MT>
struct Unroll {
  static constexpr int value = MT == 1 ? 16 : 8;
};

template <int LPR>
struct TileShape {
  static constexpr int RPW = 64 / LPR;     // rows per wave instruction
  static constexpr int NSLOT = 4 * RPW;    // row slots per workgroup
  static constexpr int TN = LPR * 8;       // tile width in columns
};

__host__ __device__ inline size_t align16(size_t b) { return (b + 15) & ~size_t(15); }


// Verification exports of the per-token input masks (bits and nnz by workgroup 0;
// the ascending index list, M == 1 only, by the workgroups of column tile 0).
// With the input normalised in the prologue (norm_x), the bits are those of the
// normalised values: each value is scaled by the same fp32 factor the prologue
// applied (inv_scale), so the comparison sees exactly the value that was masked.
template <int MT>
__device__ __forceinline__ void thresh_exports(const GemvParams& p, const int* s_idx, int* s_scan, int tid, int tile, int lo,
                               int cnt, bool first, float inv_scale) {
  (void)s_scan;
  const int K = p.K;
  const float t = p.t;
  const int M = p.M;
  if ((p.x_bits != nullptr || p.x_nnz != nullptr) && first) {
    // one 64-bit word of one token per wave and step: lane b tests input 64 w + b
    // (coalesced loads, eight words in flight per wave), ballot, count
    __shared__ int s_nnz[MT];
    if (tid < MT) s_nnz[tid] = 0;
    __syncthreads();
    const int nw = (K + 63) / 64, lane = tid & 63, wave = tid >> 6;
    constexpr int NWV = kThreads / 64;
    for (int j0 = wave; j0 < M * nw; j0 += 8 * NWV) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = min(j0 + u * NWV, M * nw - 1);
        const int m = j / nw, i = min((j % nw) * 64 + lane, K - 1);
        v[u] = load_elem(p.x, p.x_dt, (long)m * p.ldx + i);
        if (p.norm_x) v[u] *= inv_scale;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * NWV;
        if (j < M * nw) {
          const int m = j / nw, w = j % nw;
          const uint64_t bits = __ballot(w * 64 + lane < K && fabsf(v[u]) > t);
          if (lane == 0) {
            if (p.x_bits != nullptr) p.x_bits[m * p.x_bits_ld + w] = bits;
            atomicAdd(&s_nnz[m], __popcll(bits));
          }
        }
      }
    }
    __syncthreads();
    if (p.x_nnz != nullptr && tid < M) p.x_nnz[tid] = s_nnz[tid];
  }
  if (p.x_idx != nullptr && tile == 0) {
    __syncthreads();
    for (int r = tid; r < cnt; r += kThreads) p.x_idx[lo + r] = s_idx[r];
  }
}

// Plain global -> LDS copy by the whole workgroup with eight loads in flight per
// thread (the stores to LDS would otherwise wait on each load in turn).
template <class T>
__device__ __forceinline__ void copy_to_lds(T* dst, const T* src, int n) {
  // indices past n re-read element n - 1 (the loads stay unconditional and
  // issue together); only the stores are predicated
  for (int j = threadIdx.x; j < n; j += 8 * kThreads) {
    T v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[min(j + u * kThreads, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j + u * kThreads < n) dst[j + u * kThreads] = v[u];
  }
}

// Two such copies with all of their loads in flight together; COH reads the
// sources device-coherently (data written by other workgroups of the same launch).
template <bool COH, class T>
__device__ __forceinline__ T load_maybe_coherent(const T* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool COH, class T, class U>
__device__ __forceinline__ void copy2_to_lds(T* d1, const T* s1, int n1, U* d2, const U* s2, int n2) {
  const int n = n1 > n2 ? n1 : n2;
  for (int j = threadIdx.x; j < n; j += 8 * kThreads) {
    T a[8];
    U b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int jj = j + u * kThreads;
      a[u] = n1 > 0 ? load_maybe_coherent<COH>(s1 + min(jj, n1 - 1)) : T(0);
      b[u] = n2 > 0 ? load_maybe_coherent<COH>(s2 + min(jj, n2 - 1)) : U(0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int jj = j + u * kThreads;
      if (jj < n1) d1[jj] = a[u];
      if (jj < n2) d2[jj] = b[u];
    }
  }
}

// ---------------------------------------------------------------- MFMA main loop
// Batches of 9..16 tokens: the per-row FMA count outgrows the VALU, so the
// contraction runs on the matrix cores (v_mfma_f32_16x16x32_bf16).  MFMA wants
// the reduction (row) index contiguous per lane, while input-major rows are
// contiguous along the output columns.  Each chunk of CR rows (32 KB of bf16
// weights whatever the tile width) is therefore split into 8x8 blocks, one per
// thread: the thread loads 8 rows of 8 consecutive columns (16 bytes each),
// transposes the block in registers and writes each column's 8 rows as one
// 16-byte vector into a K-major LDS chunk (column pitch CR + 8 elements, so the
// 16 columns of a fragment read fall on distinct banks); a B fragment is then a
// single 16-byte LDS read.  Two chunks are in flight per workgroup: the loads of
// chunk c + 2 are issued as soon as chunk c has been written to LDS, into the
// register buffer chunk c came from.
// Activations are fp32 in LDS; each is split into bf16 hi + bf16 lo (x - hi),
// two MFMAs per fragment, which keeps fp32 inputs (h, normalised x) to ~2^-16
// relative precision while bf16 inputs stay exact.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int TN>
struct MfmaShape {
  static constexpr int CR = 32 * (512 / TN);          // rows per staged chunk
  static constexpr int LDK = CR + 8;                   // K-major LDS column pitch (elements)
  static constexpr int KS = CR / 32;                   // MFMA k-steps per chunk
  static constexpr int NRG = CR / 8;                   // 8-row groups per chunk
  static constexpr int VPT = 8;                        // one 8x8 block (8 row vectors) per thread
  static constexpr size_t kBytes = size_t(TN) * LDK * 2;
};

template <int LPR, bool GU, bool NT>
__device__ __forceinline__ void mfma_main_loop(const GemvParams& p, const int* s_idx, const float* s_val, uint16_t* s_w, int cap,
                               int cnt, int tile, float* s_out /* [16][TN], aliases s_w */) {
  constexpr int TN = LPR * 8, TB = TN / 2;
  using MS = MfmaShape<TN>;
  constexpr int CR = MS::CR, LDK = MS::LDK, KS = MS::KS, VPT = MS::VPT, NRG = MS::NRG;
  constexpr int NB = TN / 16;              // 16-column blocks in the tile
  constexpr int NBW = NB / 4;              // blocks per wave
  static_assert(NRG * (TN / 8) == kThreads, "one 8x8 block per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  f32x4_t acc[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // this thread's block: chunk rows 8 * rg .. 8 * rg + 7, tile columns vcol .. vcol + 7
  // (consecutive threads take consecutive row groups, so a wave's LDS writes spread
  // over the banks; each of its loads covers NRG rows)
  const int rg = tid % NRG, vcol = (tid / NRG) * 8;
  long vsrc;
  {
    long gc;
    bool ok;
    if constexpr (GU) {
      const int n = tile * TB + (vcol % TB);
      ok = n < p.N;
      gc = vcol < TB ? (long)n : p.gu_off + n;
    } else {
      const int n = tile * TN + vcol;
      ok = n < p.N;
      gc = n;
    }
    vsrc = ok ? gc : 0;
  }
  const int nch = (cnt + CR - 1) / CR;
  // rows past the end of the list repeat its last row (their activations are 0)
  auto fetch = [&](int ch, u32x4 (&buf)[VPT]) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int row = s_idx[min(ch * CR + rg * 8 + q, cnt - 1)];
      buf[q] = load_w16<NT>(p.W + (long)row * p.ldw + vsrc);
    }
  };
  // refill: issue the loads of chunk ch + 2 into buf once chunk ch is in LDS
  auto step = [&](int ch, u32x4 (&buf)[VPT], bool refill) {
    __syncthreads();                       // every wave is done reading the previous chunk
    // transpose the 8x8 block while writing it: word m of row q holds columns 2m
    // (low half) and 2m + 1 (high half); word n of column c's vector holds rows
    // 2n (low half) and 2n + 1 (high half)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u32x4 lo, hi;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const unsigned a = buf[2 * n][m], b = buf[2 * n + 1][m];
        lo[n] = (a & 0xffffu) | (b << 16);
        hi[n] = (a >> 16) | (b & 0xffff0000u);
      }
      *reinterpret_cast<u32x4*>(s_w + (vcol + 2 * m) * LDK + rg * 8) = lo;
      *reinterpret_cast<u32x4*>(s_w + (vcol + 2 * m + 1) * LDK + rg * 8) = hi;
    }
    __syncthreads();
    if (refill) fetch(ch + 2, buf);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // A fragment: token li, rows 8g .. 8g+7 of this k-step, split into hi + lo
      const int r0 = ch * CR + ks * 32 + 8 * g;
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(s_val + li * cap + r0);
      const f32x4_t xa = src[0], xb = src[1];
      bf16x8_t ahi, alo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = r0 + e < cnt ? (e < 4 ? xa[e] : xb[e - 4]) : 0.f;
        const uint16_t hb = f32_to_bf16_bits(x);
        const float hf = bf16_bits_to_f32(hb);
        const uint16_t lb = f32_to_bf16_bits(x - hf);
        ahi[e] = __builtin_bit_cast(__bf16, hb);
        alo[e] = __builtin_bit_cast(__bf16, lb);
      }
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        // B fragment: column col, rows 8g .. 8g+7 of this k-step, one 16-byte read
        const int col = (wave * NBW + b) * 16 + li;
        const bf16x8_t bw = *reinterpret_cast<const bf16x8_t*>(s_w + col * LDK + ks * 32 + 8 * g);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bw, acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bw, acc[b], 0, 0, 0);
      }
    }
  };
  // The steady-state loop refills unconditionally, so the two buffers' loads are
  // always outstanding in the same order and the wait before a buffer's LDS write
  // leaves the other buffer's loads in flight; the last two or three chunks are
  // peeled off.
  u32x4 ba[VPT], bb[VPT];
  if (nch == 1) {
    fetch(0, ba);
    step(0, ba, false);
  } else if (nch >= 2) {
    fetch(0, ba);
    fetch(1, bb);
    int ch = 0;
    for (; ch + 3 < nch; ch += 2) {
      step(ch, ba, true);
      step(ch + 1, bb, true);
    }
    if (nch - ch == 3) {
      step(ch, ba, true);
      step(ch + 1, bb, false);
      step(ch + 2, ba, false);
    } else {
      step(ch, ba, false);
      step(ch + 1, bb, false);
    }
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const int col = (wave * NBW + b) * 16 + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) s_out[(4 * g + e) * TN + col] = acc[b][e];
  }
  __syncthreads();
}

// ---------------------------------------------------------------- input compaction
// Both return the number of rows kept (entries [lo, lo + count) of the compacted
// list, *lo_out = lo), with s_idx / s_val filled; the caller synchronises.
// Entries are in ascending input order; with `split`, the workgroup keeps entries
// [sl * nnz / S, (sl + 1) * nnz / S), so slices are equal whatever the mask.

// Each thread owns a chunk of consecutive inputs of [i0, i1): 8 * NV of them
// loaded as 16-byte vectors issued together (NV > 0, 16-byte aligned rows), or
// ceil(len / threads) element by element (NV == 0).  A row is kept if any token
// keeps it; a workgroup scan of the per-thread counts places the chunks.  One
// token's values stay in registers; for several tokens every kept row's values
// are gathered afterwards in one pass of independent loads.
template <int MT, int NV, bool WDT_SCALED = false>
__device__ __forceinline__ int compact_chunks(const GemvParams& p, int i0, int i1, bool split, int sl, int S,
                                              int* s_idx, float* s_val, int cap, int* s_scan, int* lo_out,
                                              bool export_xn, float* inv_out,
                                              const unsigned char* head_on = nullptr) {
  const int tid = threadIdx.x;
  const int M = p.M;
  const float t = p.t;
  const int L = max(0, i1 - i0);
  constexpr int CEV = NV > 0 ? 8 * NV : 1;
  const int CE = NV > 0 ? CEV : (L + kThreads - 1) / kThreads;
  const int c0 = min(i0 + tid * CE, i1), n = max(0, min(CE, i1 - c0));
  uint64_t ubits = 0;       // NV > 0: bit e for input c0 + e
  float v0[CEV];            // MT == 1, NV > 0: the chunk's values
  int c = 0;
  if constexpr (NV > 0 && MT == 1) {
    // int8 rows: the chunk's row scales load together with its inputs
    float4 sc[WDT_SCALED ? CEV / 4 : 1];
    if constexpr (WDT_SCALED) {
      if (n == CEV) {
        const float4* q = reinterpret_cast<const float4*>(p.row_scale + c0);
#pragma unroll
        for (int k = 0; k < CEV / 4; ++k) sc[k] = q[k];
      }
    }
    load_chunk<CEV>(p.x, p.x_dt, c0, n, v0);
    if (p.norm_x && split) {
      // RMS of the whole input (the chunks of all threads cover it): per-thread sum
      // of squares, wave sums, the four wave partials added in wave order
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < CEV; ++e) ss = fmaf(v0[e], v0[e], ss);
      ss = wave_sum(ss);
      float* s_part = reinterpret_cast<float*>(s_scan);
      if ((tid & 63) == 0) s_part[tid >> 6] = ss;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) tot += s_part[w];
      __syncthreads();   // s_scan is reused by the scan below
      const float inv = 1.0f / sqrtf(tot / (float)(i1 - i0) + p.norm_eps);
      *inv_out = inv;
#pragma unroll
      for (int e = 0; e < CEV; ++e) v0[e] *= inv;
      if (export_xn && p.xn_out != nullptr) {
        // constant trip count: v0 stays in registers
#pragma unroll
        for (int e = 0; e < CEV; ++e)
          if (e < n) p.xn_out[c0 + e] = v0[e];
      }
    }
    const bool keep_all = p.keep_all != 0;
#pragma unroll
    for (int e = 0; e < CEV; ++e) ubits |= (uint64_t)(e < n && (keep_all || fabsf(v0[e]) > t)) << e;
    if (p.head_dim > 0) {
      // only rows of the listed heads
      uint64_t hb = 0;
#pragma unroll
      for (int e = 0; e < CEV; ++e) hb |= (uint64_t)(e < n && head_on[(c0 + e) / p.head_dim]) << e;
      ubits &= hb;
    }
    c = __popcll(ubits);
    if constexpr (WDT_SCALED) {
      // int8 rows: the kept value is x_i * row_scale[i] (the mask stays on x)
      if (n == CEV) {
#pragma unroll
        for (int k = 0; k < CEV / 4; ++k) {
          v0[4 * k] *= sc[k].x; v0[4 * k + 1] *= sc[k].y; v0[4 * k + 2] *= sc[k].z; v0[4 * k + 3] *= sc[k].w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < CEV; ++e)
          if (e < n) v0[e] *= p.row_scale[c0 + e];
      }
    }
    AS_PHASE_AFTER(c);
    AS_PHASE(p, 8);
  } else if constexpr (NV > 0) {
    if (n == CEV && p.x_dt != DT_F32) {
      // the chunks of up to 8 tokens are loaded before any is used
      constexpr int NVV = CEV / 8;
      constexpr int G = MT < 8 ? MT : 8;
      const bool bf = p.x_dt == DT_BF16;
#pragma unroll
      for (int m0 = 0; m0 < MT; m0 += G) {
        if (m0 < M) {
          u32x4 raw[G][NVV];
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const int m = m0 + j;
            const u32x4* q = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.x) +
                                                            (long)(m < M ? m : M - 1) * p.ldx + c0);
#pragma unroll
            for (int k = 0; k < NVV; ++k) raw[j][k] = q[k];
          }
#pragma unroll
          for (int j = 0; j < G; ++j) {
            uint64_t b = 0;
#pragma unroll
            for (int k = 0; k < NVV; ++k) {
              const uint32_t w4[4] = {raw[j][k].x, raw[j][k].y, raw[j][k].z, raw[j][k].w};
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t hb = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
                const float v = bf ? bf16_bits_to_f32(hb) : f16_bits_to_f32(hb);
                b |= (uint64_t)(fabsf(v) > t) << (8 * k + e);
              }
            }
            if (m0 + j < M) ubits |= b;
          }
        }
      }
    } else if (n == CEV) {
      // fp32 rows: groups of 4 tokens
      constexpr int NF = CEV / 4;
      constexpr int G = MT < 4 ? MT : 4;
#pragma unroll
      for (int m0 = 0; m0 < MT; m0 += G) {
        if (m0 < M) {
          float4 raw[G][NF];
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const int m = m0 + j;
            const float4* q = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.x) +
                                                              (long)(m < M ? m : M - 1) * p.ldx + c0);
#pragma unroll
            for (int k = 0; k < NF; ++k) raw[j][k] = q[k];
          }
#pragma unroll
          for (int j = 0; j < G; ++j) {
            uint64_t b = 0;
#pragma unroll
            for (int k = 0; k < NF; ++k) {
              b |= (uint64_t)(fabsf(raw[j][k].x) > t) << (4 * k);
              b |= (uint64_t)(fabsf(raw[j][k].y) > t) << (4 * k + 1);
              b |= (uint64_t)(fabsf(raw[j][k].z) > t) << (4 * k + 2);
              b |= (uint64_t)(fabsf(raw[j][k].w) > t) << (4 * k + 3);
            }
            if (m0 + j < M) ubits |= b;
          }
        }
      }
    } else {
      for (int e = 0; e < n; ++e) {
        float xv[MT];
        load_tokens<MT>(p.x, p.x_dt, p.ldx, c0 + e, M, xv);
        bool a = false;
#pragma unroll
        for (int m = 0; m < MT; ++m) a |= fabsf(xv[m]) > t;
        ubits |= (uint64_t)a << e;
      }
    }
    c = __popcll(ubits);
  } else {
    for (int e = 0; e < n; ++e) {
      float xv[MT];
      load_tokens<MT>(p.x, p.x_dt, p.ldx, c0 + e, M, xv);
      bool a = false;
#pragma unroll
      for (int m = 0; m < MT; ++m) a |= fabsf(xv[m]) > t;
      c += a;
    }
  }
  int nnz;
  const int off = block_excl_scan<kThreads>(c, s_scan, &nnz);
  AS_PHASE(p, 9);
  const int lo = split ? split_point(sl, nnz, S) : 0;
  const int hi = split ? split_point(sl + 1, nnz, S) : nnz;
  *lo_out = lo;
  AS_PHASE_AFTER(hi);
  AS_PHASE(p, 11);
  if (off < hi && off + c > lo) {
    if constexpr (NV > 0) {
      // each kept input's place is its rank among the thread's kept inputs (a
      // popcount of the lower bits), so the writes carry no chain of dependent adds
      const int base = off - lo;
      const unsigned span = (unsigned)(hi - lo);
#pragma unroll
      for (int e = 0; e < CEV; ++e) {
        int r;
        if constexpr (CEV <= 32) r = base + __popc((uint32_t)ubits & ((1u << e) - 1u));
        else r = base + __popcll(ubits & ((uint64_t(1) << e) - 1u));
        if (((ubits >> e) & 1u) && (unsigned)r < span) {
          s_idx[r] = c0 + e;
          if constexpr (MT == 1) s_val[r] = v0[e];
        }
      }
    } else {
      int r = off;
      for (int e = 0; e < n && r < hi; ++e) {
        float xv[MT];
        load_tokens<MT>(p.x, p.x_dt, p.ldx, c0 + e, M, xv);
        bool a = false;
#pragma unroll
        for (int m = 0; m < MT; ++m) a |= fabsf(xv[m]) > t;
        if (a) {
          if (r >= lo) {
            s_idx[r - lo] = c0 + e;
            if constexpr (MT == 1) s_val[r - lo] = xv[0];
          }
          ++r;
        }
      }
    }
  }
  AS_PHASE(p, 12);
  __syncthreads();
  AS_PHASE(p, 13);
  const int cnt = hi - lo;
  if constexpr (MT == 1) return cnt;
  for (int r = tid; r < cnt; r += kThreads) {
    float xv[MT];
    load_tokens<MT>(p.x, p.x_dt, p.ldx, s_idx[r], M, xv);
#pragma unroll
    for (int m = 0; m < MT; ++m) s_val[m * cap + r] = fabsf(xv[m]) > t ? xv[m] : 0.f;
  }
  return cnt;
}

// Compaction of a range [i0, i0 + L) whose values sit in LDS (stage: [MT][L]
// fp32).  The range is cut into units of 64 rows and wave w takes a contiguous run
// of units, lane l row l of each unit: the union mask over tokens (|v| > t for any
// token, or every row with keep_all) is a ballot per unit, so a wave counts its
// kept rows without a loop over bits; one barrier exchanges the four wave totals,
// then each wave writes its kept rows in ascending order (a token's value is 0
// where its own |v| <= t).  Returns the number of kept rows; synchronises before
// returning.
template <int MT>
__device__ __forceinline__ int compact_stage(const float* stage, int L, int i0, float t, bool keep_all, int* s_idx,
                                             float* s_val, int cap, int* s_scan) {
  constexpr int NW = kThreads / 64;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int units = (L + 63) / 64;
  const int u0 = split_point(w, units, NW), u1 = split_point(w + 1, units, NW);
  auto keep = [&](int e) {
    if (e >= L) return false;
    bool a = keep_all;
#pragma unroll
    for (int m = 0; m < MT; ++m) a |= fabsf(stage[m * L + e]) > t;
    return a;
  };
  int cnt = 0;
  for (int u = u0; u < u1; ++u) cnt += __popcll(__ballot(keep(u * 64 + lane)));
  if (lane == 0) s_scan[w] = cnt;
  __syncthreads();
  int r = 0, nnz = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int c = s_scan[k];
    r += k < w ? c : 0;
    nnz += c;
  }
  for (int u = u0; u < u1; ++u) {
    const int e = u * 64 + lane;
    const bool a = keep(e);
    const uint64_t bits = __ballot(a);
    if (a) {
      const int pos = r + lanes_below(bits);
      s_idx[pos] = i0 + e;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float xv = stage[m * L + e];
        s_val[m * cap + pos] = (keep_all || fabsf(xv) > t) ? xv : 0.f;
      }
    }
    r += __popcll(bits);
  }
  __syncthreads();
  return nnz;
}

// Several tokens, a range [i0, i1) of at most 2 * kThreads inputs: each thread owns
// two consecutive inputs and loads every token's value of them into registers (no
// LDS staging), forms their union mask (|v| > t for any token), and after a
// workgroup scan writes the kept rows in input order, a token's value being 0 where
// its own |v| <= t.  The same rows and values as the staged version below.
template <int MT>
__device__ __forceinline__ int compact_range_regs(const GemvParams& p, int i0, int i1, int* s_idx, float* s_val,
                                                  int cap, int* s_scan) {
  const int tid = threadIdx.x, M = p.M;
  const float t = p.t;
  const int L = max(0, i1 - i0);
  const int c0 = 2 * tid;
  float xv[2][MT];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const long row = L > 0 ? (long)i0 + min(c0 + e, L - 1) : 0;    // past L: a row in range, dropped
    load_tokens<MT>(p.x, p.x_dt, p.ldx, row, M, xv[e]);
  }
  bool a[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    bool any = false;
#pragma unroll
    for (int m = 0; m < MT; ++m) any |= m < M && fabsf(xv[e][m]) > t;
    a[e] = c0 + e < L && any;
  }
  int nnz;
  int r = block_excl_scan<kThreads>((int)a[0] + (int)a[1], s_scan, &nnz);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (a[e]) {
      s_idx[r] = i0 + c0 + e;
#pragma unroll
      for (int m = 0; m < MT; ++m) s_val[m * cap + r] = (m < M && fabsf(xv[e][m]) > t) ? xv[e][m] : 0.f;
      ++r;
    }
  }
  __syncthreads();
  return nnz;
}

// Several tokens, one slice's own range [i0, i1): every token's values of the
// range are staged in LDS (stage: [MT][len] fp32) with one round trip of
// independent loads (16-byte vectors when NV > 0, i.e. aligned rows), then each
// thread takes a contiguous chunk of the range for the union mask, a workgroup
// scan places the chunks, and the kept rows' values are copied from the stage.
template <int MT, int NV>
__device__ __forceinline__ int compact_range_staged(const GemvParams& p, int i0, int i1, int* s_idx, float* s_val,
                                                    int cap, float* stage, int* s_scan) {
  const int tid = threadIdx.x, M = p.M;
  const float t = p.t;
  const int L = max(0, i1 - i0);
  if constexpr (NV > 0) {
    // vectors of 8 (16-bit) or 4 (fp32) inputs; L is a multiple of 64 except at the end
    const bool f32 = p.x_dt == DT_F32, bf = p.x_dt == DT_BF16;
    const int per = f32 ? 4 : 8;
    const int nvec = (L + per - 1) / per;               // per token
    const int tot = nvec * MT;
    for (int j0 = tid; j0 < tot; j0 += 8 * kThreads) {
      u32x4 raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = min(j0 + u * kThreads, tot - 1);
        const int m = j / nvec, vi = j % nvec;
        const int mm = m < M ? m : M - 1;
        const long e = (long)mm * p.ldx + i0 + (long)vi * per;
        raw[u] = f32 ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(p.x) + e)
                     : *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.x) + e);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * kThreads;
        if (j < tot) {
          const int m = j / nvec, vi = j % nvec;
          // L is a multiple of 8 (whole vectors), so each vector is one or two
          // 16-byte LDS stores
          f32x4_t* dst = reinterpret_cast<f32x4_t*>(stage + m * L + vi * per);
          const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
          const bool live = m < M;
          if (f32) {
            dst[0] = live ? f32x4_t{__uint_as_float(w4[0]), __uint_as_float(w4[1]), __uint_as_float(w4[2]),
                                    __uint_as_float(w4[3])}
                          : f32x4_t{0.f, 0.f, 0.f, 0.f};
          } else {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t hb = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
              f[e] = live ? (bf ? bf16_bits_to_f32(hb) : f16_bits_to_f32(hb)) : 0.f;
            }
            dst[0] = f32x4_t{f[0], f[1], f[2], f[3]};
            dst[1] = f32x4_t{f[4], f[5], f[6], f[7]};
          }
        }
      }
    }
  } else {
    for (int j = tid; j < L * MT; j += kThreads) {
      const int m = j / L, i = j % L;
      stage[j] = m < M ? load_elem(p.x, p.x_dt, (long)m * p.ldx + i0 + i) : 0.f;
    }
  }
  __syncthreads();
  return compact_stage<MT>(stage, L, i0, t, false, s_idx, s_val, cap, s_scan);
}

// Sum of the gate and up partials of four consecutive rows (offset `off` of slice
// 0) over the S1 gate/up slices, in slice order from 0: batches of up to kB slices
// are loaded together (one round trip per batch).
__device__ __forceinline__ void sum_parts4(const float* P, int off, int S1, int slice_ld, int up, f32x4_t& g,
                                           f32x4_t& u) {
  constexpr int kB = 8;
  g = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S1; s0 += kB) {
    f32x4_t tg[kB], tu[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      // the slice count is uniform: a batch past the last slice issues no loads
      if (s0 + k < S1) {
        const float* ps = P + (s0 + k) * slice_ld + off;
        tg[k] = *reinterpret_cast<const f32x4_t*>(ps);
        tu[k] = *reinterpret_cast<const f32x4_t*>(ps + up);
      } else {
        tg[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        tu[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (s0 + k < S1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g[e] += tg[k][e];
          u[e] += tu[k][e];
        }
      }
  }
}

// One token, a range of at most 4 * kThreads rows, no h exports: thread j owns rows
// 4j..4j+3 and keeps their h values in registers; a workgroup scan of the per-thread
// kept counts places the rows, which go from registers straight to the row list (no
// LDS staging, no second pass).  The same rows, order and values as the staged path.
__device__ __forceinline__ int compact_parts_regs(const GemvParams& p, int i0, int L, int* s_idx, float* s_val,
                                                  int* s_scan) {
  const int tid = threadIdx.x;
  const int nq = L / 4;
  const bool live = tid < nq;
  f32x4_t h = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    f32x4_t g, u;
    sum_parts4(reinterpret_cast<const float*>(p.x), i0 + 4 * tid, p.x_parts, (int)p.ldx, (int)p.x_up, g, u);
    AS_PHASE_AFTER(g[0]);
    AS_PHASE_AFTER(u[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = silu_f32(g[e]) * u[e];
  }
  AS_PHASE(p, 8);
  const bool keep_all = p.keep_all != 0;
  unsigned kb = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) kb |= (unsigned)(live && (keep_all || fabsf(h[e]) > p.t)) << e;
  AS_PHASE(p, 9);
  AS_PHASE(p, 10);
  int nnz;
  int r = block_excl_scan<kThreads>(__popc(kb), s_scan, &nnz);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if ((kb >> e) & 1u) {
      s_idx[r] = i0 + 4 * tid + e;
      s_val[r] = h[e];
      ++r;
    }
  __syncthreads();
  return nnz;
}

// The input of a down projection is h = silu(g) * u of a paired gate/up launch
// that stored its split-K partials without summing them (OUT_PARTS).  Slice sl
// owns the 64-aligned range [i0, i1) of h: for each token and each group of four
// rows, the gate and up partials of every gate/up slice are summed in slice order
// starting from 0 (sum_parts4), which is exactly the sum the gate/up launch's own
// combine would form; h goes to the stage ([MT][L] fp32), then the range is masked
// and compacted.  With `exports`, h and its mask bits are also written out (one
// workgroup per range does this).  One token without exports takes the register
// path above.
template <int MT>
__device__ __forceinline__ int compact_parts(const GemvParams& p, int i0, int i1, int* s_idx, float* s_val, int cap,
                                             float* stage, int* s_scan, bool exports) {
  const int tid = threadIdx.x, M = p.M;
  const float t = p.t;
  const int L = max(0, i1 - i0);            // a multiple of 64 (K is)
  const int nq = L / 4;                     // groups of four rows per token
  const bool exporting = exports && (p.h != nullptr || p.h_bits != nullptr || p.h_nnz != nullptr);
  if constexpr (MT == 1) {
    if (!exporting && nq <= kThreads) return compact_parts_regs(p, i0, L, s_idx, s_val, s_scan);
  }
  const int tot = nq * MT;
  const float* P = reinterpret_cast<const float*>(p.x);
  // 32-bit offsets: the partials buffer holds fewer than 2^31 floats
  const int tok_ld = (int)p.ldx, slice_ld = M * tok_ld, up = (int)p.x_up;
  for (int j = tid; j < tot; j += kThreads) {
    const int m = j / nq, q = j % nq;
    f32x4_t g, u;
    sum_parts4(P, (m < M ? m : M - 1) * tok_ld + i0 + 4 * q, p.x_parts, slice_ld, up, g, u);
    if (j == tid) {
      AS_PHASE_AFTER(g[0]);
      AS_PHASE_AFTER(u[3]);
      AS_PHASE(p, 8);
    }
    f32x4_t h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = m < M ? silu_f32(g[e]) * u[e] : 0.f;
    *reinterpret_cast<f32x4_t*>(stage + m * L + 4 * q) = h;
  }
  __syncthreads();
  AS_PHASE(p, 9);
  if (exporting) {
    if (p.h != nullptr)
      for (int j = tid; j < M * L; j += kThreads) p.h[(j / L) * p.ldh + i0 + j % L] = stage[j];
    if (p.h_bits != nullptr || p.h_nnz != nullptr) {
      // one wave per 64-row word (words never straddle tokens: L is a multiple of 64);
      // the count is accumulated with integer atomics (exact in any order)
      const int lane = tid & 63;
      for (int b = (tid >> 6) * 64; b < M * L; b += kThreads) {
        const uint64_t bits = __ballot(fabsf(stage[b + lane]) > t);
        if (lane == 0) {
          if (p.h_bits != nullptr) p.h_bits[(b / L) * p.h_bits_ld + (i0 + b % L) / 64] = bits;
          if (p.h_nnz != nullptr && bits) atomicAdd(p.h_nnz + b / L, (int)__popcll(bits));
        }
      }
    }
  }
  AS_PHASE(p, 10);
  return compact_stage<MT>(stage, L, i0, t, p.keep_all != 0, s_idx, s_val, cap, s_scan);
}

// One work item: column tile `tile`, row slice `sl` of S (p.S) equal parts of the
// compacted row list (IN_PARTS: the range [rr0, rr1) of h when rr1 >= 0); its
// partial tile is slot `part` of `n_parts` combined by the last item of the tile to
// finish.  IN_LISTS reads list tiles [lt0, lt0 + n_lt).  Used by the GEMV kernel
// below (one item per workgroup) and by the one-stream MoE layer's launches.
template <int WDT, int MT, int LPR, int IN, int OUT, bool GU, bool NT, int NV>
__device__ __forceinline__ void gemv_item(const GemvParams& p, int tile, int sl, int part, int n_parts, int lt0, int n_lt,
                          unsigned char* smem, int rr0 = 0, int rr1 = -1) {
  using TS = TileShape<LPR>;
  constexpr int RPW = TS::RPW, NSLOT = TS::NSLOT, TN = TS::TN, TB = TN / 2;
  const int cap = p.cap;
  // LDS: row list | activations [MT][cap] | slot reduction (VALU loop) | list-tile
  // prefix sums | staging region (the input range during an IN_RANGE / IN_PARTS
  // prologue, then the MFMA weight chunk, whose buffer also holds the MFMA output
  // tile).
  constexpr bool kMfma = MT == 16;
  int* s_idx = reinterpret_cast<int*>(smem);
  float* s_val = reinterpret_cast<float*>(smem + align16(size_t(cap) * 4));
  unsigned char* after_val = smem + align16(size_t(cap) * 4) + align16(size_t(cap) * MT * 4);
  const size_t red_bytes = kMfma ? 0 : align16(size_t(NSLOT > MT ? NSLOT : MT) * TN * 4);
  int* s_pref = reinterpret_cast<int*>(after_val + red_bytes);
  uint16_t* s_w = reinterpret_cast<uint16_t*>(reinterpret_cast<unsigned char*>(s_pref) +
                                              (IN == IN_LISTS ? align16(size_t(p.n_lt + 1) * 4) : 0));
  float* s_red = kMfma ? reinterpret_cast<float*>(s_w) : reinterpret_cast<float*>(after_val);
  (void)n_lt;
  __shared__ int s_scan[kThreads / 64 + 1];
  __shared__ int s_flag;
  __shared__ unsigned char s_head_on[MT == 1 ? 1024 : 1];

  const int tid = threadIdx.x;
  const int S = p.S;
  const int M = p.M;
  AS_PHASE(p, 0);

  // ------------------------------------------------------------ prologue
  int cnt = 0;
  if constexpr (IN == IN_THRESH || IN == IN_RANGE) {
    // IN_THRESH: the whole input, split into S equal parts of the compacted list.
    // IN_RANGE: slice sl owns the inputs of its 64-aligned range and keeps all of them.
    const bool split = IN == IN_THRESH;
    if constexpr (MT == 1) {
      if (p.head_dim > 0) {
        // head mask: the listed heads' flags in LDS before the range is masked
        for (int h = tid; h < p.n_heads; h += kThreads) s_head_on[h] = 0;
        __syncthreads();
        for (int q = tid; q < p.n_heads_keep; q += kThreads) {
          const int h = p.heads[q];
          if (h >= 0 && h < p.n_heads) s_head_on[h] = 1;
        }
        __syncthreads();
      }
    }
    int r0 = 0, r1 = p.K;
    if (!split) {
      const int units = (p.K + 63) / 64;
      r0 = min(p.K, split_point(sl, units, S) * 64);
      r1 = min(p.K, split_point(sl + 1, units, S) * 64);
    }
    int lo = 0;
    float inv_scale = 1.0f;     // the normalisation factor (norm_x), the same in every thread
    if constexpr (IN == IN_RANGE && MT > 1)
      cnt = r1 - r0 <= 2 * kThreads
                ? compact_range_regs<MT>(p, r0, r1, s_idx, s_val, cap, s_scan)
                : compact_range_staged<MT, NV>(p, r0, r1, s_idx, s_val, cap, reinterpret_cast<float*>(s_w), s_scan);
    else
      cnt = compact_chunks<MT, NV, WDT == DT_I8>(p, r0, r1, split, sl, S, s_idx, s_val, cap, s_scan, &lo,
                                                 tile == 0 && sl == 0, &inv_scale, s_head_on);
    if (split && (p.x_bits != nullptr || p.x_nnz != nullptr || p.x_idx != nullptr))
      thresh_exports<MT>(p, s_idx, s_scan, tid, tile, lo, cnt, tile == 0 && sl == 0, inv_scale);
  } else if constexpr (IN == IN_PARTS) {
    // the range of h: explicit (one-launch MLP) or slice sl of S 64-aligned parts
    const int units = (p.K + 63) / 64;
    const int r0 = rr1 >= 0 ? rr0 : min(p.K, split_point(sl, units, S) * 64);
    const int r1 = rr1 >= 0 ? rr1 : min(p.K, split_point(sl + 1, units, S) * 64);
    cnt = compact_parts<MT>(p, r0, r1, s_idx, s_val, cap, reinterpret_cast<float*>(s_w), s_scan, tile == 0);
  } else if constexpr (IN == IN_LISTS) {
    // Tile counts: up to kLB batches of 256 tiles are loaded together (one round
    // trip), then scanned batch by batch into the prefix table s_pref.
    constexpr int kLB = MT >= 8 ? 2 : MT >= 4 ? 4 : 8;   // batch per thread (registers)
    int run = 0;
    for (int base0 = 0; base0 < n_lt; base0 += kLB * kThreads) {
      int v[kLB];
#pragma unroll
      for (int k = 0; k < kLB; ++k) {
        const int q = base0 + k * kThreads + tid;
        v[k] = q < n_lt ? p.list_cnt[lt0 + q] : 0;
      }
#pragma unroll
      for (int k = 0; k < kLB; ++k) {
        if (base0 + k * kThreads >= n_lt) break;         // uniform
        const int q = base0 + k * kThreads + tid;
        int tot;
        const int off = block_excl_scan<kThreads>(v[k], s_scan, &tot);
        if (q < n_lt) s_pref[q] = run + off;
        run += tot;
      }
    }
    if (tid == 0) s_pref[n_lt] = run;
    __syncthreads();
    const int nnz = run;
    const int lo = split_point(sl, nnz, S), hi = split_point(sl + 1, nnz, S);
    cnt = hi - lo;
    // Entries: a batch of up to kLB entries per thread is located in the prefix
    // table first (binary searches in LDS), then all its loads issue together.
    for (int r0 = tid; r0 < cnt; r0 += kLB * kThreads) {
      long e[kLB];
#pragma unroll
      for (int k = 0; k < kLB; ++k) {
        const int r = r0 + k * kThreads;
        const int g = lo + min(r, cnt - 1);
        int a = 0, b = n_lt;            // largest q with s_pref[q] <= g
        while (b - a > 1) {
          const int mid = (a + b) >> 1;
          if (s_pref[mid] <= g) a = mid; else b = mid;
        }
        e[k] = (long)(lt0 + a) * p.lt_stride + (g - s_pref[a]);
      }
      int idx[kLB];
      float xv[kLB][MT];
#pragma unroll
      for (int k = 0; k < kLB; ++k) {
        idx[k] = p.list_idx[e[k]];
#pragma unroll
        for (int m = 0; m < MT; ++m) xv[k][m] = p.list_val[e[k] * M + (m < M ? m : M - 1)];
      }
#pragma unroll
      for (int k = 0; k < kLB; ++k) {
        const int r = r0 + k * kThreads;
        if (r < cnt) {
          s_idx[r] = idx[k];
#pragma unroll
          for (int m = 0; m < MT; ++m) s_val[m * cap + r] = m < M ? xv[k][m] : 0.f;
        }
      }
    }
  } else {  // IN_ALL: every row, no mask (dense baseline); with a head list, every row of the listed heads
    int K = p.K;
    const int* hl = nullptr;
    if constexpr (MT == 1) {
      if (p.head_dim > 0) {
        // the listed heads (entries outside [0, n_heads) ignored, repeats once) in
        // ascending order, kept in the reduction buffer (unused until the main loop
        // ends); the slices then take equal shares of those heads' rows
        int* s_hl = reinterpret_cast<int*>(s_red);
        for (int h = tid; h < p.n_heads; h += kThreads) s_head_on[h] = 0;
        __syncthreads();
        for (int q = tid; q < p.n_heads_keep; q += kThreads) {
          const int h = p.heads[q];
          if (h >= 0 && h < p.n_heads) s_head_on[h] = 1;
        }
        __syncthreads();
        int c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int h = 4 * tid + e;
          c += (h < p.n_heads && s_head_on[h]) ? 1 : 0;
        }
        int tot;
        int off = block_excl_scan<kThreads>(c, s_scan, &tot);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int h = 4 * tid + e;
          if (h < p.n_heads && s_head_on[h]) s_hl[off++] = h;
        }
        __syncthreads();
        K = tot * p.head_dim;
        hl = s_hl;
      }
    }
    const int lo = split_point(sl, K, S), hi = split_point(sl + 1, K, S);
    cnt = hi - lo;
    for (int r = tid; r < cnt; r += kThreads) {
      const int g = lo + r;
      const int row = hl != nullptr ? hl[g / p.head_dim] * p.head_dim + g % p.head_dim : g;
      s_idx[r] = row;
      float xv[MT];
      load_tokens<MT>(p.x, p.x_dt, p.ldx, row, M, xv);
      if constexpr (WDT == DT_I8) {
        const float sc = p.row_scale[row];
#pragma unroll
        for (int m = 0; m < MT; ++m) xv[m] *= sc;
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) s_val[m * cap + r] = xv[m];
    }
  }
  __syncthreads();
  AS_PHASE(p, 1);
  AS_PHASE_VAL(p, 7, (unsigned long long)cnt);

  constexpr int CPT = (TN + kThreads - 1) / kThreads;   // tile columns per thread
  float res[MT][CPT];
  if constexpr (MT == 16) {
    static_assert(WDT == DT_BF16, "the MFMA path takes bf16 weights");
    mfma_main_loop<LPR, GU, NT>(p, s_idx, s_val, s_w, cap, cnt, tile, s_red);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = tid + q * kThreads;
        res[m][q] = c < TN ? s_red[m * TN + c] : 0.f;
      }
  } else {
  // ------------------------------------------------------------ main loop
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPR, l = lane % LPR;
  const int slot = wave * RPW + sub;
  long wcol;
  bool valid;
  if constexpr (GU) {
    const int nb = tile * TB + (l % (LPR / 2)) * 8;
    valid = nb < p.N;
    wcol = (l < LPR / 2) ? nb : p.gu_off + nb;
  } else {
    const int c0 = tile * TN + l * 8;
    valid = c0 < p.N;
    wcol = c0;
  }
  // Lanes past a ragged column edge read column 0 of the same rows (their sums are
  // discarded), and rows past the end of the slice repeat its last row with x = 0,
  // so every load below is unconditional and all kUnroll loads issue back to back.
  constexpr int kUnroll = Unroll<MT>::value;
  const uint16_t* Wc = p.W + (valid ? wcol : 0);
  const long ldw = p.ldw;

  float acc[MT][8];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;

  if constexpr (WDT == DT_I8) {
    // int8 rows: 8-byte pieces (eight columns per lane, as for 16-bit weights), twice
    // as many rows in flight for the same bytes; the row scale is in s_val
    constexpr int kU8 = 2 * kUnroll;
    const int8_t* W8 = reinterpret_cast<const int8_t*>(p.W) + (valid ? wcol : 0);
    for (int r = slot; r < cnt; r += NSLOT * kU8) {
      int row[kU8];
#pragma unroll
      for (int u = 0; u < kU8; ++u) row[u] = s_idx[min(r + u * NSLOT, cnt - 1)];
      u32x2 w[kU8];
#pragma unroll
      for (int u = 0; u < kU8; ++u) w[u] = load_w8<NT>(W8 + (long)row[u] * ldw);
#pragma unroll
      for (int u = 0; u < kU8; ++u) {
        const int rr = r + u * NSLOT;
        float wf[8];
        unpack8_i8(w[u], wf);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float xv = rr < cnt ? s_val[m * cap + rr] : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[m][j] = fmaf(xv, wf[j], acc[m][j]);
        }
      }
    }
  } else
  for (int r = slot; r < cnt; r += NSLOT * kUnroll) {
    int row[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) row[u] = s_idx[min(r + u * NSLOT, cnt - 1)];
    u32x4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = load_w16<NT>(Wc + (long)row[u] * ldw);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int rr = r + u * NSLOT;
      float wf[8];
      unpack8<WDT>(w[u], wf);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float xv = rr < cnt ? s_val[m * cap + rr] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[m][j] = fmaf(xv, wf[j], acc[m][j]);
      }
    }
  }

  AS_PHASE(p, 2);
  // ------------------------------------------------------------ slot reduction
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) s_red[slot * TN + l * 8 + j] = acc[m][j];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kThreads;
      float v = 0.f;
      if (c < TN)
#pragma unroll
        for (int s2 = 0; s2 < NSLOT; ++s2) v += s_red[s2 * TN + c];
      res[m][q] = v;
    }
  }

  }

  AS_PHASE(p, 3);
  // tile-local column c -> (validity, partial/output column)
  auto col_of = [&](int c, bool& ok) -> long {
    if constexpr (GU) {
      const int n = tile * TB + (c % TB);
      ok = n < p.N;
      return c < TB ? (long)n : (long)p.N + n;
    } else {
      const int n = tile * TN + c;
      ok = n < p.N;
      return n;
    }
  };

  // ------------------------------------------------------------ unsummed partials
  if constexpr (OUT == OUT_PARTS) {
    // the next launch sums the slices (its kernel boundary makes these stores visible)
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kThreads;
      bool ok;
      const long pc = col_of(c, ok);
      if (c < TN && ok)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < M) store_coherent(p.partials + ((long)part * M + m) * p.part_ld + pc, res[m][q]);
    }
    // one workgroup clears the y that the next launch adds into
    if (p.zero_y != nullptr && tile == 0 && part == 0)
      for (long i = tid; i < p.zero_n; i += kThreads) p.zero_y[i] = 0.f;
#ifdef AS_PHASE_TIMELINE
    if (p.phase_tl != nullptr && tid == 0) wait_vmem();
#endif
    AS_PHASE(p, 4);
    return;
  }

  // ------------------------------------------------------------ split-K combine
  if constexpr (OUT == OUT_Y) {
    if (n_parts > 1 && p.atomic_y) {
      // every slice adds its partial tile into y (fp32, cleared by the host or the
      // previous launch unless accumulating); slice 0 adds the residual
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = tid + q * kThreads;
        bool ok;
        const long gc = col_of(c, ok);
        if (c < TN && ok)
#pragma unroll
          for (int m = 0; m < MT; ++m)
            if (m < M) {
              float v = res[m][q];
              if (part == 0 && p.res != nullptr) v += load_elem(p.res, p.res_dt, m * p.ldres + gc);
              unsafeAtomicAdd(reinterpret_cast<float*>(p.y) + m * p.ldy + gc, v);
            }
      }
      return;
    }
  }
  if constexpr (OUT == OUT_Y || OUT == OUT_SWIGLU) {
    if (n_parts > 1 && p.defer_sum) {
      // the next launch sums the slices in slice order (its kernel boundary makes
      // these stores visible): no counter, and no one workgroup loading every
      // slice's tile
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = tid + q * kThreads;
        bool ok;
        const long pc = col_of(c, ok);
        if (c < TN && ok)
#pragma unroll
          for (int m = 0; m < MT; ++m)
            if (m < M) p.partials[((long)part * M + m) * p.part_ld + pc] = res[m][q];
      }
      return;
    }
  }
  if (n_parts > 1) {
    // Partials are written through to the device-coherent level (relaxed agent-scope
    // atomic stores) and the wave waits for their completion before the counter
    // increment; the last workgroup reads them back with coherent loads.  No
    // L2 writeback/invalidate fence is needed on any workgroup.
    //
    // Memory-ordering argument.  Under the HIP/C++ model alone this is not enough:
    // relaxed atomics order nothing, and the portable form is a release on the
    // counter increment and an acquire on the last workgroup's side.  At agent scope
    // on this chip those fences become a writeback of the XCD's whole L2 and an
    // invalidate of it, microseconds on every workgroup.  The protocol relies
    // instead on what the AMDGPU memory model (LLVM AMDGPUUsage, gfx942/gfx950
    // memory model) gives these operations on this target:
    //  (1) an agent-scope atomic store/load is a global store/load with the cache
    //      policy bits that make it coherent across the XCDs (no stale line in a
    //      non-coherent per-XCD L2 can satisfy or absorb it);
    //  (2) wait_vmem() (s_waitcnt vmcnt(0)) returns only after those stores are
    //      acknowledged, i.e. performed at that coherent level;
    //  (3) the __syncthreads() then orders every wave's completed stores before
    //      thread 0's counter fetch-add, itself an agent-scope atomic performed at
    //      the same level;
    //  (4) the last workgroup issues its loads only after the fetch-add's returned
    //      value is known (s_flag through LDS and a barrier), and those loads are
    //      agent-scope atomic loads, so they read the coherent level.
    // Every value written before (2) is therefore visible to the loads in (4).
    // The bitwise run-twice tests and the integer-valued exact tests exercise it.
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kThreads;
      bool ok;
      const long pc = col_of(c, ok);
      if (c < TN && ok)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < M) store_coherent(p.partials + ((long)part * M + m) * p.part_ld + pc, res[m][q]);
    }
    wait_vmem();
    __syncthreads();
    AS_PHASE(p, 4);
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(p.counters + (long)tile * kCounterStride, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_flag = (prev == unsigned(n_parts - 1));
    }
    __syncthreads();
    AS_PHASE(p, 5);
    if (!s_flag) return;
    if (tid == 0) __hip_atomic_store(p.counters + (long)tile * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Batches of slices are loaded together for every token (one round trip per
    // batch, at most 128 values in flight per thread), then summed in slice order.
    constexpr int kBudget = 128 / (MT * CPT);
    constexpr int kBatch = kBudget < 1 ? 1 : (kBudget > 16 ? 16 : kBudget);
    // 32-bit element offsets (the partials buffer holds fewer than 2^31 floats);
    // columns past the tile edge read column 0 and are dropped, so every load is
    // unconditional.
    int pcs[CPT];
    bool oks[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kThreads;
      bool ok;
      const long pc = col_of(c, ok);
      oks[q] = c < TN && ok;
      pcs[q] = oks[q] ? (int)pc : 0;
    }
    const int slice_stride = M * (int)p.part_ld;
    float v[MT][CPT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < CPT; ++q) v[m][q] = 0.f;
    for (int s0 = 0; s0 < n_parts; s0 += kBatch) {
      float tmp[MT][CPT][kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float* ps = p.partials + min(s0 + k, n_parts - 1) * slice_stride;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float* pm = ps + (m < M ? m : M - 1) * (int)p.part_ld;
#pragma unroll
          for (int q = 0; q < CPT; ++q) tmp[m][q][k] = load_coherent(pm + pcs[q]);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < CPT; ++q)
#pragma unroll
          for (int k = 0; k < kBatch; ++k)
            if (s0 + k < n_parts && oks[q]) v[m][q] += tmp[m][q][k];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < CPT; ++q) res[m][q] = m < M ? v[m][q] : 0.f;
  }

  // ------------------------------------------------------------ epilogues
  if constexpr (OUT == OUT_Y) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kThreads;
      bool ok;
      const long gc = col_of(c, ok);
      if (c < TN && ok)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < M) {
            float v = res[m][q];
            if (p.accumulate) v += load_elem(p.y, p.y_dt, m * p.ldy + gc);
            if (p.res != nullptr) v += load_elem(p.res, p.res_dt, m * p.ldres + gc);
            store_elem(p.y, p.y_dt, m * p.ldy + gc, v);
          }
    }
#ifdef AS_PHASE_TIMELINE
    if (p.phase_tl != nullptr && tid == 0) wait_vmem();
#endif
    AS_PHASE(p, 6);
  } else if constexpr (OUT == OUT_ROUTER) {
    // the logits of every token (the grid has this one column tile): stored, staged
    // in LDS, and each token routed by one wave
    __shared__ TopkSmem r_sm[kThreads / 64];
    __shared__ int r_sel[kThreads / 64][64];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kThreads;
      if (c < TN)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          s_red[m * TN + c] = res[m][q];
          if (m < M && c < p.N) store_elem(p.y, p.y_dt, m * p.ldy + c, res[m][q]);
        }
    }
    __syncthreads();
    const int wave = tid >> 6;
    for (int m = wave; m < M; m += kThreads / 64)
      route_token(s_red + m * TN, p.N, p.route_top, p.route_ids + m * p.route_top, p.route_wts + m * p.route_top,
                  r_sel[wave], r_sm[wave]);
  } else if constexpr (OUT == OUT_SWIGLU) {
    static_assert(GU, "the SwiGLU epilogue needs paired gate/up columns");
    // the one workgroup finishing tile 0 clears the y that the next launch adds into
    if (p.zero_y != nullptr && tile == 0)
      for (long i = tid; i < p.zero_n; i += kThreads) p.zero_y[i] = 0.f;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = tid + q * kThreads;
      if (c < TN)
#pragma unroll
        for (int m = 0; m < MT; ++m) s_red[m * TN + c] = res[m][q];
    }
    __syncthreads();
    const int n = tile * TB + tid;
    const bool nvalid = tid < TB && n < p.N;
    float hv[MT];
    bool any = false;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      hv[m] = 0.f;
      if (nvalid && m < M) {
        const float g = s_red[m * TN + tid], u = s_red[m * TN + TB + tid];
        hv[m] = silu_f32(g) * u;
        any |= fabsf(hv[m]) > p.t_h;
        p.h[m * p.ldh + n] = hv[m];
      }
    }
    if ((p.h_bits != nullptr || p.h_nnz != nullptr) && tid < TB) {
      for (int m = 0; m < M; ++m) {
        const uint64_t bits = __ballot(nvalid && fabsf(hv[m]) > p.t_h);
        if ((tid & 63) == 0 && tile * TB + tid < p.N) {
          if (p.h_bits != nullptr) p.h_bits[m * p.h_bits_ld + (tile * TB + tid) / 64] = bits;
          // the mask's count: integer adds, exact in any order (cleared by the host)
          if (p.h_nnz != nullptr && bits) atomicAdd(p.h_nnz + m, (int)__popcll(bits));
        }
      }
    }
    if (p.o_cnt != nullptr) {
      const int flag = (nvalid && any) ? 1 : 0;
      int tot;
      const int pos = block_excl_scan<kThreads>(flag, s_scan, &tot);
      if (flag) {
        const long e = (long)tile * TB + pos;
        store_coherent_i32(p.o_idx + e, n);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < M) store_coherent(p.o_val + e * M + m, fabsf(hv[m]) > p.t_h ? hv[m] : 0.f);
      }
      if (tid == 0) store_coherent_i32(p.o_cnt + tile, tot);
    }
  }
}

// At least two waves per SIMD (two workgroups per CU): the register budget of the
// widest instantiations (16 tokens) must stay within 256 per lane.
template <int WDT, int MT, int LPR, int IN, int OUT, bool GU, bool NT, int NV>
__global__ __launch_bounds__(kThreads, 2) void gather_gemv_kernel(const GemvParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tile = blockIdx.x % p.n_tiles, sl = blockIdx.x / p.n_tiles;
  gemv_item<WDT, MT, LPR, IN, OUT, GU, NT, NV>(p, tile, sl, sl, p.S, 0, p.n_lt, smem);
}

// ---------------------------------------------------------------- dispatch
template <int WDT, int MT, int LPR, int IN, int OUT, bool GU, bool NT, int NV>
hipError_t launch_one(const GemvParams& p, size_t smem, hipStream_t s) {
  auto k = gather_gemv_kernel<WDT, MT, LPR, IN, OUT, GU, NT, NV>;
  if (smem > 64 * 1024) {
    // raised per instantiation only when a launch asks for more than before
    static std::atomic<size_t> allowed{64 * 1024};
    if (smem > allowed.load(std::memory_order_acquire)) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
      if (e != hipSuccess) return e;
      size_t cur = allowed.load(std::memory_order_relaxed);
      while (cur < smem && !allowed.compare_exchange_weak(cur, smem, std::memory_order_acq_rel)) {
      }
    }
  }
  hipLaunchKernelGGL(k, dim3(p.n_tiles * p.S), dim3(kThreads), smem, s, p);
  return hipGetLastError();
}

template <int WDT, int MT, int LPR, int IN, int OUT, bool GU, bool NT>
hipError_t pick_nv(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  // 16-byte chunk prologue: 2 vectors per thread, or 8 for one token
  if constexpr (IN == IN_THRESH || IN == IN_RANGE) {
    if (c.nv == 2) return launch_one<WDT, MT, LPR, IN, OUT, GU, NT, 2>(p, smem, s);
    if constexpr (MT == 1) {
      if (c.nv == 8) return launch_one<WDT, MT, LPR, IN, OUT, GU, NT, 8>(p, smem, s);
    }
  }
  return launch_one<WDT, MT, LPR, IN, OUT, GU, NT, 0>(p, smem, s);
}

template <int WDT, int MT, int LPR, int IN, int OUT, bool GU>
hipError_t pick_nt(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  return c.nt ? pick_nv<WDT, MT, LPR, IN, OUT, GU, true>(c, p, smem, s)
              : pick_nv<WDT, MT, LPR, IN, OUT, GU, false>(c, p, smem, s);
}

template <int WDT, int MT, int LPR>
hipError_t pick_mode(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  if (c.gu) {
    if (c.out == OUT_PARTS) {
      if constexpr (MT <= 8) {
        if (c.in == IN_THRESH) return pick_nt<WDT, MT, LPR, IN_THRESH, OUT_PARTS, true>(c, p, smem, s);
        if (c.in == IN_RANGE) return pick_nt<WDT, MT, LPR, IN_RANGE, OUT_PARTS, true>(c, p, smem, s);
        if (c.in == IN_ALL) return pick_nt<WDT, MT, LPR, IN_ALL, OUT_PARTS, true>(c, p, smem, s);
      }
      return hipErrorInvalidValue;
    }
    if (c.out != OUT_SWIGLU) return hipErrorInvalidValue;
    if (c.in == IN_THRESH) return pick_nt<WDT, MT, LPR, IN_THRESH, OUT_SWIGLU, true>(c, p, smem, s);
    if (c.in == IN_RANGE) return pick_nt<WDT, MT, LPR, IN_RANGE, OUT_SWIGLU, true>(c, p, smem, s);
    if (c.in == IN_ALL) return pick_nt<WDT, MT, LPR, IN_ALL, OUT_SWIGLU, true>(c, p, smem, s);
    return hipErrorInvalidValue;
  }
  if (c.out == OUT_ROUTER) {
    if constexpr (MT <= 8) {
      if (c.in == IN_ALL) return pick_nt<WDT, MT, LPR, IN_ALL, OUT_ROUTER, false>(c, p, smem, s);
    }
    return hipErrorInvalidValue;
  }
  if (c.out != OUT_Y) return hipErrorInvalidValue;
  if (c.in == IN_THRESH) return pick_nt<WDT, MT, LPR, IN_THRESH, OUT_Y, false>(c, p, smem, s);
  if (c.in == IN_RANGE) return pick_nt<WDT, MT, LPR, IN_RANGE, OUT_Y, false>(c, p, smem, s);
  if (c.in == IN_LISTS) return pick_nt<WDT, MT, LPR, IN_LISTS, OUT_Y, false>(c, p, smem, s);
  if (c.in == IN_PARTS) {
    if constexpr (MT <= 8) return pick_nt<WDT, MT, LPR, IN_PARTS, OUT_Y, false>(c, p, smem, s);
    return hipErrorInvalidValue;
  }
  return pick_nt<WDT, MT, LPR, IN_ALL, OUT_Y, false>(c, p, smem, s);
}

// int8 weights: one token, the threshold prologue (16-byte chunks) or every row.
template <int LPR>
hipError_t pick_i8_mode(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  if (c.gu || c.out != OUT_Y) return hipErrorInvalidValue;
  if (c.in == IN_THRESH) {
    if (c.nv == 2) return c.nt ? launch_one<DT_I8, 1, LPR, IN_THRESH, OUT_Y, false, true, 2>(p, smem, s)
                               : launch_one<DT_I8, 1, LPR, IN_THRESH, OUT_Y, false, false, 2>(p, smem, s);
    if (c.nv == 8) return c.nt ? launch_one<DT_I8, 1, LPR, IN_THRESH, OUT_Y, false, true, 8>(p, smem, s)
                               : launch_one<DT_I8, 1, LPR, IN_THRESH, OUT_Y, false, false, 8>(p, smem, s);
    return hipErrorInvalidValue;
  }
  if (c.in == IN_RANGE) {
    if (c.nv == 2) return c.nt ? launch_one<DT_I8, 1, LPR, IN_RANGE, OUT_Y, false, true, 2>(p, smem, s)
                               : launch_one<DT_I8, 1, LPR, IN_RANGE, OUT_Y, false, false, 2>(p, smem, s);
    if (c.nv == 8) return c.nt ? launch_one<DT_I8, 1, LPR, IN_RANGE, OUT_Y, false, true, 8>(p, smem, s)
                               : launch_one<DT_I8, 1, LPR, IN_RANGE, OUT_Y, false, false, 8>(p, smem, s);
    return hipErrorInvalidValue;
  }
  if (c.in == IN_ALL) return c.nt ? launch_one<DT_I8, 1, LPR, IN_ALL, OUT_Y, false, true, 0>(p, smem, s)
                                  : launch_one<DT_I8, 1, LPR, IN_ALL, OUT_Y, false, false, 0>(p, smem, s);
  return hipErrorInvalidValue;
}

template <int WDT, int MT>
hipError_t pick_lpr(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s) {
  switch (c.lpr) {
    case 16: return pick_mode<WDT, MT, 16>(c, p, smem, s);
    case 32: return pick_mode<WDT, MT, 32>(c, p, smem, s);
    case 64: return pick_mode<WDT, MT, 64>(c, p, smem, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace as
