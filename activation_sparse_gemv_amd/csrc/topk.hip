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

__global__ __launch_bounds__(kTopkThreads) void topk_value_kernel(const float* score, int n, int k, uint64_t* mask,
                                                                  int* idx) {
  __shared__ TopkSmem sm;
  const long r = blockIdx.x;
  const float* s = score + r * n;
  block_topk<kTopkThreads>([=](int i) { return float_key(s[i]); }, n, k,
                           mask ? mask + r * ((n + 63) / 64) : nullptr, idx ? idx + r * (long)k : nullptr, sm);
}

// Ordinal ranks by counting: rank_j - 1 = #{i : v_i < v_j or (v_i == v_j and
// i > j)}, accumulated over chunks of i into cnt[r][sig][j] (atomically; the blend
// kernel clears it), where sig 0 ranks score[r] and sig 1 ranks prior[r].
// The chunk's keys sit in LDS and are read four at a time; each thread ranks
// kRankJ consecutive values, so one LDS read feeds 16 comparisons.  A wave's
// values span a window of 256 indices: chunk keys below the window are strictly
// smaller-index (ties do not count), keys past it are larger-index (ties count),
// and only keys inside the window take the exact index comparison.
constexpr int kRankThreads = 256;
constexpr int kRankJ = 4;

__global__ __launch_bounds__(kRankThreads) void rank_count_kernel(const float* score, const float* prior, int n,
                                                                  int chunks, unsigned* part) {
  extern __shared__ __align__(16) uint32_t keys[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int chunk = blockIdx.y;
  const int r = blockIdx.z >> 1, sig = blockIdx.z & 1;
  const float* v = (sig == 0 ? score : prior) + (long)r * n;
  const int i0 = split_point(chunk, n, chunks), i1 = split_point(chunk + 1, n, chunks);
  const int len = i1 - i0;
  for (int t = tid; t < len; t += kRankThreads) keys[t] = float_key(v[i0 + t]);
  __syncthreads();
  const int j0 = (blockIdx.x * kRankThreads + tid) * kRankJ;
  uint32_t kj[kRankJ];
  unsigned c[kRankJ];
#pragma unroll
  for (int q = 0; q < kRankJ; ++q) {
    kj[q] = j0 + q < n ? float_key(v[j0 + q]) : 0u;
    c[q] = 0u;
  }
  // chunk-local bounds of the wave's index window [jw0, jw0 + 64 * kRankJ)
  const int jw0 = j0 - lane * kRankJ;
  const int len4 = len & ~3;
  const int wa = min(max(jw0 - i0, 0), len), wb = min(max(jw0 + 64 * kRankJ - i0, 0), len);
  const int sa = min(wa & ~3, len4);                 // [0, sa): every key is below the window
  const int sb = max(min((wb + 3) & ~3, len4), sa);  // [sb, len4): every key is past it
  for (int t = 0; t < sa; t += 4) {
    const uint4 q4 = *reinterpret_cast<const uint4*>(keys + t);
#pragma unroll
    for (int q = 0; q < kRankJ; ++q)
      c[q] += (unsigned)(q4.x < kj[q]) + (unsigned)(q4.y < kj[q]) + (unsigned)(q4.z < kj[q]) + (unsigned)(q4.w < kj[q]);
  }
  for (int t = sb; t < len4; t += 4) {
    const uint4 q4 = *reinterpret_cast<const uint4*>(keys + t);
#pragma unroll
    for (int q = 0; q < kRankJ; ++q)
      c[q] += (unsigned)(q4.x <= kj[q]) + (unsigned)(q4.y <= kj[q]) + (unsigned)(q4.z <= kj[q]) +
              (unsigned)(q4.w <= kj[q]);
  }
  auto exact = [&](int t) {
    const uint32_t ki = keys[t];
    const int i = i0 + t;
#pragma unroll
    for (int q = 0; q < kRankJ; ++q) c[q] += (unsigned)((ki < kj[q]) | ((ki == kj[q]) & (i > j0 + q)));
  };
  for (int t = sa; t < sb; ++t) exact(t);
  for (int t = max(sb, len4); t < len; ++t) exact(t);
  unsigned* out = part + ((long)r * 2 + sig) * n;
#pragma unroll
  for (int q = 0; q < kRankJ; ++q)
    if (j0 + q < n && c[q]) atomicAdd(out + j0 + q, c[q]);
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
  for (int j = threadIdx.x; j < n; j += kTopkThreads) {
    S[j] = wl * (cl[j] + 1u) + lq * (cg[j] + 1u);
    cl[j] = 0u;
    cg[j] = 0u;
  }
  __syncthreads();
  uint64_t* mk = mask ? mask + r * ((n + 63) / 64) : nullptr;
  int* ix = idx ? idx + r * (long)k : nullptr;
  if constexpr (SLDS) block_topk<kTopkThreads>([=](int i) { return s_lds[i]; }, n, k, mk, ix, sm);
  else block_topk<kTopkThreads>([=](int i) { return Sg[i]; }, n, k, mk, ix, sm);
}

constexpr int kBlendLdsMax = 32768;   // blended scores staged in LDS up to this n

// Chunks of the counting grid: about 512 workgroups in all, chunks of >= 64 keys.
int rank_chunks(int rows, int n) {
  const long jb = (n + kRankThreads * kRankJ - 1) / (kRankThreads * kRankJ);
  long c = (512 + jb * 2 * rows - 1) / (jb * 2 * rows);
  if (c > 64) c = 64;
  if (c > n / 64) c = n / 64;
  return c < 1 ? 1 : (int)c;
}

size_t topk_blend_ws_bytes(int rows, int n) {
  return (size_t(rows) * 2 * n + size_t(rows) * n) * sizeof(unsigned);
}

hipError_t launch_topk_value(const float* score, int rows, int n, int k, uint64_t* mask, int* idx, hipStream_t s) {
  hipLaunchKernelGGL(topk_value_kernel, dim3(rows), dim3(kTopkThreads), 0, s, score, n, k, mask, idx);
  return hipGetLastError();
}

hipError_t launch_topk_blend(const float* score, const float* prior, int rows, int n, int k, uint32_t lq,
                             uint64_t* mask, int* idx, unsigned* ws, hipStream_t s) {
  unsigned* cnt = ws;                                // [rows][2][n], zero between calls
  uint32_t* s_glob = ws + size_t(rows) * 2 * n;
  hipError_t e;
  const int chunks = rank_chunks(rows, n);
  const int maxlen = (n + chunks - 1) / chunks;
  const size_t smem1 = (size_t(maxlen) * 4 + 15) & ~size_t(15);
  const dim3 grid((n + kRankThreads * kRankJ - 1) / (kRankThreads * kRankJ), chunks, rows * 2);
  hipLaunchKernelGGL(rank_count_kernel, grid, dim3(kRankThreads), smem1, s, score, prior, n, chunks, cnt);
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
