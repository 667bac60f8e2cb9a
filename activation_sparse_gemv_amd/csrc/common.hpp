// Device helpers shared by the gfx950 kernels: dtype conversion, 16-byte weight
// loads, wave64 / workgroup scans, and the internal launch interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace as {

enum { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2, DT_I8 = 3 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
  return (float)h;
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                                                  // RNE
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Element i of a vector stored in dtype dt, as fp32 (exact for f16/bf16).
__device__ __forceinline__ float load_elem(const void* p, int dt, long i) {
  if (dt == DT_F32) return reinterpret_cast<const float*>(p)[i];
  uint32_t b = reinterpret_cast<const uint16_t*>(p)[i];
  return dt == DT_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

__device__ __forceinline__ void store_elem(void* p, int dt, long i, float v) {
  if (dt == DT_F32) reinterpret_cast<float*>(p)[i] = v;
  else if (dt == DT_BF16) reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
  else reinterpret_cast<uint16_t*>(p)[i] = f32_to_f16_bits(v);
}

// 16-byte weight load (8 x 16-bit), nontemporal when NT is set: the rows are
// streamed once per call, so they should not displace x, h and the partials.
// NT is a compile-time choice: a runtime select between the two forms gets merged
// into one plain load by the optimizer, which drops the nontemporal hint.
template <bool NT>
__device__ __forceinline__ u32x4 load_w16(const uint16_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  if constexpr (NT) return __builtin_nontemporal_load(q);
  else return *q;
}

// Eight int8 weights (one 8-byte piece of a row), plain or nontemporal.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ u32x2 load_w8(const int8_t* p) {
  const u32x2* q = reinterpret_cast<const u32x2*>(p);
  if constexpr (NT) return __builtin_nontemporal_load(q);
  else return *q;
}

// Eight int8 weights (four per dword, lowest byte first) to fp32: the sign bit is
// flipped so each byte reads as an unsigned value biased by 128 (one byte-to-float
// conversion and one subtraction per weight, both exact).
__device__ __forceinline__ void unpack8_i8(const u32x2 v, float w[8]) {
  const uint32_t a = v.x ^ 0x80808080u, b = v.y ^ 0x80808080u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[k] = (float)((a >> (8 * k)) & 0xffu) - 128.f;
    w[4 + k] = (float)((b >> (8 * k)) & 0xffu) - 128.f;
  }
}

// Unpack 8 weights (two per dword, low half first) to fp32.
template <int WDT>
__device__ __forceinline__ void unpack8(const u32x4 v, float w[8]) {
  if constexpr (WDT == DT_BF16) {
    w[0] = __uint_as_float(v.x << 16); w[1] = __uint_as_float(v.x & 0xffff0000u);
    w[2] = __uint_as_float(v.y << 16); w[3] = __uint_as_float(v.y & 0xffff0000u);
    w[4] = __uint_as_float(v.z << 16); w[5] = __uint_as_float(v.z & 0xffff0000u);
    w[6] = __uint_as_float(v.w << 16); w[7] = __uint_as_float(v.w & 0xffff0000u);
  } else {
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[2 * k] = f16_bits_to_f32(q[k] & 0xffffu);
      w[2 * k + 1] = f16_bits_to_f32(q[k] >> 16);
    }
  }
}

// CE consecutive elements of a vector (dtype dt) starting at element `off`, as fp32.
// n == CE: vector loads (the caller guarantees 16-byte alignment); otherwise the
// first n elements are loaded one by one and the rest are zero.
template <int CE>
__device__ __forceinline__ void load_chunk(const void* x, int dt, long off, int n, float v[CE]) {
  static_assert(CE % 8 == 0, "chunk of whole 16-byte vectors");
  if (n == CE) {
    if (dt == DT_F32) {
      const float4* q = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
      float4 f[CE / 4];
#pragma unroll
      for (int k = 0; k < CE / 4; ++k) f[k] = q[k];
#pragma unroll
      for (int k = 0; k < CE / 4; ++k) {
        v[4 * k] = f[k].x; v[4 * k + 1] = f[k].y; v[4 * k + 2] = f[k].z; v[4 * k + 3] = f[k].w;
      }
    } else {
      const u32x4* q = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + off);
      u32x4 raw[CE / 8];
#pragma unroll
      for (int k = 0; k < CE / 8; ++k) raw[k] = q[k];
#pragma unroll
      for (int k = 0; k < CE / 8; ++k) {
        if (dt == DT_BF16) unpack8<DT_BF16>(raw[k], v + 8 * k);
        else unpack8<DT_F16>(raw[k], v + 8 * k);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < CE; ++e) v[e] = e < n ? load_elem(x, dt, off + e) : 0.f;
  }
}

// Values at input index i of tokens 0..MT-1 (token rows at or past M re-read row
// M - 1 and read as 0).  The dtype test sits outside the loads, so all MT loads
// issue back to back instead of one round trip per token.
template <int MT>
__device__ __forceinline__ void load_tokens(const void* x, int dt, long ldx, long i, int M, float (&v)[MT]) {
  if (dt == DT_F32) {
    const float* q = reinterpret_cast<const float*>(x) + i;
#pragma unroll
    for (int m = 0; m < MT; ++m) v[m] = q[(long)(m < M ? m : M - 1) * ldx];
  } else {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(x) + i;
    uint32_t b[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) b[m] = q[(long)(m < M ? m : M - 1) * ldx];
    if (dt == DT_BF16) {
#pragma unroll
      for (int m = 0; m < MT; ++m) v[m] = bf16_bits_to_f32(b[m]);
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m) v[m] = f16_bits_to_f32(b[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
    if (m >= M) v[m] = 0.f;
}

// floor(a * b / c) in 32-bit unsigned arithmetic, for a * b < 2^32 (split points of
// at most 2^24 items into parts): a 64-bit division is a long scalar sequence here.
__device__ __forceinline__ int split_point(int a, int b, int c) {
  return (int)((unsigned)a * (unsigned)b / (unsigned)c);
}

// Wait until every vector-memory operation this wave issued has completed.
__device__ __forceinline__ void wait_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt/lgkmcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Device-coherent (agent scope) store / load: written through to, or read from,
// the level shared by every XCD, so no L2 writeback or invalidate is needed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent_i32(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_coherent_i32(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_coherent_u32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- wave64 helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` in lanes below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave reductions without LDS: DPP moves within each row of 16 lanes (quad lane
// swaps xor 1 and xor 2, then rotations by 4 and 8 lanes), after which every lane
// holds its row's result; the four row results are read out with readlane and
// combined as (row0 op row1) op (row2 op row3).  The result is the same in every
// lane.  Called with the whole wave active.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float dppf(float v, int ctrl_sel) {
  switch (ctrl_sel) {
    case 0: return __int_as_float(dpp_mov<0xB1>(__float_as_int(v)));    // quad_perm [1, 0, 3, 2]
    case 1: return __int_as_float(dpp_mov<0x4E>(__float_as_int(v)));    // quad_perm [2, 3, 0, 1]
    case 2: return __int_as_float(dpp_mov<0x124>(__float_as_int(v)));   // row_ror:4
    default: return __int_as_float(dpp_mov<0x128>(__float_as_int(v)));  // row_ror:8
  }
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 0; s < 4; ++s) v += dppf(v, s);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 0; s < 4; ++s) v = fmaxf(v, dppf(v, s));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t x = (uint32_t)__float_as_int(dppf(__int_as_float((int)v), s));
    v = x > v ? x : v;
  }
  uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16) {
    const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)v, l);
    r = x > r ? x : r;
  }
  return r;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t x = (uint32_t)__float_as_int(dppf(__int_as_float((int)v), s));
    v = x < v ? x : v;
  }
  uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16) {
    const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)v, l);
    r = x < r ? x : r;
  }
  return r;
}

// Inclusive prefix sum over the 64 lanes by DPP: shifts right by 1, 2, 4 and 8
// lanes within each row of 16 (lanes without a source add 0), then the last lane
// of row 0 is broadcast into rows 1 and 3 and the last lane of row 1 into rows 2
// and 3.  Called with the whole wave active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
  return v;
}

// Radix-select step, run by one full wave: given a 256-bin histogram, find the
// bin holding the krem-th key counted from the top (from_top) or from the bottom,
// and the rank of that key inside the bin.  Lane l owns bins 4l..4l+3; the
// counts above (below) a lane come from a wave suffix (prefix) scan, so the
// search is a few shuffles instead of a 256-step serial walk.
__device__ __forceinline__ void wave_select_bin(const unsigned* hist, int krem, bool from_top, int* bin_out,
                                                int* krem_out) {
  const int l = lane_id();
  int c[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) c[q] = (int)hist[4 * l + q];
  const int local = c[0] + c[1] + c[2] + c[3];
  // inclusive scan in the direction of the walk
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = from_top ? __shfl_down(incl, o, 64) : __shfl_up(incl, o, 64);
    if (from_top ? (l + o < 64) : (l >= o)) incl += t;
  }
  int run = incl - local;             // keys in bins strictly before this lane's bins (walk order)
  int found = -1, rem = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int qq = from_top ? 3 - q : q;
    const int b = 4 * l + qq;
    if (found < 0 && run < krem && krem <= run + c[qq]) { found = b; rem = krem - run; }
    run += c[qq];
  }
  if (found >= 0) { *bin_out = found; *krem_out = rem; }
}

// Exclusive scan over a workgroup of NT threads (NT a multiple of 64, <= 1024).
// `sm` needs NT/64 + 1 ints.  Returns the exclusive prefix; *total = the sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* sm, int* total) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  int inc = wave_incl_scan(v);
  if (l == 63) sm[w] = inc;
  __syncthreads();
  // every wave adds up the wave totals itself (no serial step by one thread)
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = sm[i];
    base += i < w ? c : 0;
    tot += c;
  }
  *total = tot;
  __syncthreads();   // sm may be reused as soon as this returns
  return base + inc - v;
}

}  // namespace as
