// Top-k neuron masks: value mode and the GLASS rank blend.
//
// GLASS summary, section 2.2: the local (prompt) and global (prior) importance
// signals are turned into ranks R^(l), R^(g); the neuron score is
// (1 - lambda) R^(l) + lambda R^(g) and the k best neurons form the static mask.
// Ranks are ordinal (largest value -> n, equal values -> the smaller index ranks
// higher), so they form a permutation; lambda is carried in 16-bit fixed point,
// which makes the blend an exact integer computation:
//   S_j = (65536 - lq) R^(l)_j + lq R^(g)_j,   lq = round(lambda * 65536).
#include "topk.hpp"
#include "internal.hpp"

namespace as {

constexpr int kTopkThreads = 1024;

// One workgroup per row; rows up to kValueLdsMax keys are staged in LDS once
// (eight loads in flight per thread), longer rows are read from memory by every
// pass of the selection.
constexpr int kValueLdsMax = 16384;

template <bool SLDS>
__global__ __launch_bounds__(kTopkThreads) void topk_value_kernel(const float* score, int n, int k, uint64_t* mask,
                                                                  int* idx) {
  __shared__ TopkSmem sm;
  extern __shared__ __align__(16) uint32_t kl[];
  const long r = blockIdx.x;
  const float* s = score + r * n;
  uint64_t* mk = mask ? mask + r * ((n + 63) / 64) : nullptr;
  int* ix = idx ? idx + r * (long)k : nullptr;
  if constexpr (SLDS) {
    constexpr int kB = 8;
    for (int i0 = threadIdx.x; i0 < n; i0 += kB * kTopkThreads) {
      float v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) v[u] = i0 + u * kTopkThreads < n ? s[i0 + u * kTopkThreads] : 0.f;
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (i0 + u * kTopkThreads < n) kl[i0 + u * kTopkThreads] = float_key(v[u]);
    }
    __syncthreads();
    block_topk<kTopkThreads>([=](int i) { return kl[i]; }, n, k, mk, ix, sm);
  } else {
    block_topk<kTopkThreads>([=](int i) { return float_key(s[i]); }, n, k, mk, ix, sm);
  }
}

// Ordinal ranks: rank_j - 1 = #{i : v_i < v_j or (v_i == v_j and i > j)}, the
// number of entries before j in the order (key ascending, index descending).
// (1) chunk_sort_kernel: every chunk of 256 consecutive entries is sorted in that
//     order (each entry's place in its chunk by counting over the chunk in LDS,
//     four threads per entry) into the workspace as (key, index) pairs;
// (2) rank_search_kernel: for each j and each sorted chunk, the entries of the
//     chunk that come before j form a prefix of it, found by a binary search
//     (nine steps); a workgroup takes 256 values of j against a batch of up to
//     kRankBatch chunks staged in LDS and adds its counts into cnt (cleared by
//     the blend kernel after use).
// Both launches spread over the chip: n/256 workgroups per signal for (1) and
// (n/256) * ceil(n/256/kRankBatch) for (2).
constexpr int kRankChunk = 256;
constexpr int kRankBatch = 16;

__device__ __forceinline__ bool rank_before(uint32_t ke, uint32_t ie, uint32_t kj, uint32_t j) {
  return ke < kj || (ke == kj && ie > j);
}

// Four threads per entry, each counting over a quarter of the chunk.
constexpr int kSortParts = 4;

__global__ __launch_bounds__(kRankChunk * kSortParts) void chunk_sort_kernel(const float* score, const float* prior,
                                                                             int n, uint32_t* skey, uint32_t* sidx) {
  __shared__ __align__(16) uint32_t k_s[kRankChunk];
  __shared__ int s_part[kSortParts][kRankChunk];
  const int t = threadIdx.x & (kRankChunk - 1), part = threadIdx.x / kRankChunk, c = blockIdx.x;
  const int r = blockIdx.y >> 1, sig = blockIdx.y & 1;
  const float* v = (sig == 0 ? score : prior) + (long)r * n;
  const int i0 = c * kRankChunk, len = min(kRankChunk, n - i0);
  if (part == 0) k_s[t] = t < len ? float_key(v[i0 + t]) : 0u;
  __syncthreads();
  const uint32_t kt = k_s[t];
  // entries u of [u0, u1) that come before t: smaller key, or equal key and larger index
  constexpr int kQ = kRankChunk / kSortParts;
  const int u0 = part * kQ, u1 = min(u0 + kQ, len);
  int pos = 0;
  if (u1 - u0 == kQ) {
#pragma unroll 4
    for (int u = u0; u < u1; u += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(k_s + u);
      pos += (int)(q.x < kt || (q.x == kt && u > t)) + (int)(q.y < kt || (q.y == kt && u + 1 > t)) +
             (int)(q.z < kt || (q.z == kt && u + 2 > t)) + (int)(q.w < kt || (q.w == kt && u + 3 > t));
    }
  } else {
    for (int u = u0; u < u1; ++u) {
      const uint32_t ku = k_s[u];
      pos += (int)(ku < kt || (ku == kt && u > t));
    }
  }
  s_part[part][t] = pos;
  __syncthreads();
  if (part != 0 || t >= len) return;
  pos = s_part[0][t] + s_part[1][t] + s_part[2][t] + s_part[3][t];
  const long o = ((long)r * 2 + sig) * n + i0 + pos;
  skey[o] = kt;
  sidx[o] = (uint32_t)(i0 + t);
}

__global__ __launch_bounds__(kRankChunk) void rank_search_kernel(const float* score, const float* prior, int n,
                                                                 const uint32_t* skey, const uint32_t* sidx,
                                                                 unsigned* cnt) {
  __shared__ uint2 bp[kRankBatch * kRankChunk];        // (key, index) of the batch's sorted chunks
  const int t = threadIdx.x;
  const int r = blockIdx.z >> 1, sig = blockIdx.z & 1;
  const long row = ((long)r * 2 + sig) * n;
  const int nch = (n + kRankChunk - 1) / kRankChunk;
  const int c0 = blockIdx.y * kRankBatch, c1 = min(c0 + kRankBatch, nch);
  const int e0 = c0 * kRankChunk, e1 = min(c1 * kRankChunk, n);
  {
    // the batch's sorted pairs, every load of a thread issued before the first is used
    uint32_t lk[kRankBatch], li[kRankBatch];
#pragma unroll
    for (int u = 0; u < kRankBatch; ++u) {
      const int e = e0 + t + u * kRankChunk;
      lk[u] = e < e1 ? skey[row + e] : 0u;
      li[u] = e < e1 ? sidx[row + e] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kRankBatch; ++u)
      if (e0 + t + u * kRankChunk < e1) bp[t + u * kRankChunk] = make_uint2(lk[u], li[u]);
  }
  const float* v = (sig == 0 ? score : prior) + (long)r * n;
  const int j = blockIdx.x * kRankChunk + t;
  const uint32_t kj = j < n ? float_key(v[j]) : 0u;
  __syncthreads();
  if (j >= n) return;
  // the batch's binary searches side by side: kRankBatch independent LDS reads per step
  int pos[kRankBatch], len[kRankBatch];
#pragma unroll
  for (int c = 0; c < kRankBatch; ++c) {
    pos[c] = 0;
    len[c] = c0 + c < c1 ? min(kRankChunk, n - (c0 + c) * kRankChunk) : 0;
  }
#pragma unroll
  for (int step = kRankChunk; step > 0; step >>= 1) {
#pragma unroll
    for (int c = 0; c < kRankBatch; ++c) {
      const int q = pos[c] + step;
      if (q <= len[c]) {
        const uint2 e = bp[c * kRankChunk + q - 1];
        if (rank_before(e.x, e.y, kj, (uint32_t)j)) pos[c] = q;
      }
    }
  }
  unsigned tot = 0u;
#pragma unroll
  for (int c = 0; c < kRankBatch; ++c) tot += (unsigned)pos[c];
  atomicAdd(cnt + row + j, tot);
}

// Blended score S_j = (65536 - lq) R^(l)_j + lq R^(g)_j (ranks = counts + 1; fits
// 32 bits for n <= 65535), staged in LDS when it fits (SLDS) or in the workspace,
// then the exact top-k over it.  The counts are cleared for the next call.
template <bool SLDS>
__global__ __launch_bounds__(kTopkThreads) void topk_blend_kernel(unsigned* cnt, int n, int k, uint32_t lq,
                                                                  uint64_t* mask, int* idx, uint32_t* s_glob) {
  __shared__ TopkSmem sm;
  extern __shared__ __align__(16) uint32_t s_lds[];
  const long r = blockIdx.x;
  unsigned* cl = cnt + r * 2 * (long)n;
  unsigned* cg = cl + n;
  uint32_t* S = SLDS ? s_lds : s_glob + r * n;
  const uint32_t* Sg = s_glob + r * n;
  const uint32_t wl = 65536u - lq;
  constexpr int kB = 8;                                // loads in flight per thread
  for (int j0 = threadIdx.x; j0 < n; j0 += kB * kTopkThreads) {
    uint32_t a[kB], b[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int j = j0 + u * kTopkThreads;
      a[u] = j < n ? cl[j] : 0u;
      b[u] = j < n ? cg[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int j = j0 + u * kTopkThreads;
      if (j < n) {
        S[j] = wl * (a[u] + 1u) + lq * (b[u] + 1u);
        cl[j] = 0u;
        cg[j] = 0u;
      }
    }
  }
  __syncthreads();
  uint64_t* mk = mask ? mask + r * ((n + 63) / 64) : nullptr;
  int* ix = idx ? idx + r * (long)k : nullptr;
  if constexpr (SLDS) block_topk<kTopkThreads>([=](int i) { return s_lds[i]; }, n, k, mk, ix, sm);
  else block_topk<kTopkThreads>([=](int i) { return Sg[i]; }, n, k, mk, ix, sm);
}


constexpr int kBlendLdsMax = 32768;   // blended scores staged in LDS up to this n

// counts [rows][2][n], blended scores [rows][n], then the sorted chunks' keys and
// indices [rows][2][n] each
size_t topk_blend_ws_bytes(int rows, int n) {
  return (size_t(rows) * 2 * n * 3 + size_t(rows) * n) * sizeof(unsigned);
}

hipError_t launch_topk_value(const float* score, int rows, int n, int k, uint64_t* mask, int* idx, hipStream_t s) {
  if (n <= kValueLdsMax) {
    const size_t smem = size_t(n) * 4;
    if (smem > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_value_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_value_kernel<true>, dim3(rows), dim3(kTopkThreads), smem, s, score, n, k, mask, idx);
  } else {
    hipLaunchKernelGGL(topk_value_kernel<false>, dim3(rows), dim3(kTopkThreads), 0, s, score, n, k, mask, idx);
  }
  return hipGetLastError();
}

hipError_t launch_topk_blend(const float* score, const float* prior, int rows, int n, int k, uint32_t lq,
                             uint64_t* mask, int* idx, unsigned* ws, hipStream_t s) {
  unsigned* cnt = ws;                                // [rows][2][n], zero between calls
  uint32_t* s_glob = ws + size_t(rows) * 2 * n;
  uint32_t* skey = s_glob + size_t(rows) * n;
  uint32_t* sidx = skey + size_t(rows) * 2 * n;
  hipError_t e;
  const int nch = (n + kRankChunk - 1) / kRankChunk;
  hipLaunchKernelGGL(chunk_sort_kernel, dim3(nch, rows * 2), dim3(kRankChunk * kSortParts), 0, s, score, prior, n,
                     skey, sidx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(rank_search_kernel, dim3(nch, (nch + kRankBatch - 1) / kRankBatch, rows * 2),
                     dim3(kRankChunk), 0, s, score, prior, n, skey, sidx, cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (n <= kBlendLdsMax) {
    const size_t smem = size_t(n) * 4;
    if (smem > 64 * 1024) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_blend_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_blend_kernel<true>, dim3(rows), dim3(kTopkThreads), smem, s, cnt, n, k, lq, mask, idx,
                       s_glob);
  } else {
    hipLaunchKernelGGL(topk_blend_kernel<false>, dim3(rows), dim3(kTopkThreads), 0, s, cnt, n, k, lq, mask, idx,
                       s_glob);
  }
  return hipGetLastError();
}

}  // namespace as
