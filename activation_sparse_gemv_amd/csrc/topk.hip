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

// cnt[r][sig][j] += #{i in chunk : v_i < v_j or (v_i == v_j and i > j)}, where
// sig 0 ranks score[r] and sig 1 ranks prior[r].  Keys are tiled through LDS.
constexpr int kRankThreads = 256;
constexpr int kRankTile = 1024;

__global__ __launch_bounds__(kRankThreads) void rank_count_kernel(const float* score, const float* prior, int n,
                                                                  int chunks, unsigned* cnt) {
  __shared__ uint32_t tile[kRankTile];
  const int j = blockIdx.x * kRankThreads + threadIdx.x;
  const int chunk = blockIdx.y;
  const int r = blockIdx.z >> 1, sig = blockIdx.z & 1;
  const float* v = (sig == 0 ? score : prior) + (long)r * n;
  const uint32_t kj = j < n ? float_key(v[j]) : 0u;
  const int i0 = (int)((long)chunk * n / chunks), i1 = (int)((long)(chunk + 1) * n / chunks);
  unsigned c = 0;
  for (int base = i0; base < i1; base += kRankTile) {
    const int len = min(kRankTile, i1 - base);
    __syncthreads();
    for (int t = threadIdx.x; t < len; t += kRankThreads) tile[t] = float_key(v[base + t]);
    __syncthreads();
    if (j < n) {
      for (int t = 0; t < len; ++t) {
        const uint32_t ki = tile[t];
        const int i = base + t;
        c += (ki < kj) | ((ki == kj) & (i > j));
      }
    }
  }
  if (j < n && c) atomicAdd(cnt + ((long)r * 2 + sig) * n + j, c);
}

__global__ __launch_bounds__(kTopkThreads) void topk_blend_kernel(const unsigned* cnt, int n, int k, uint32_t lq,
                                                                  uint64_t* mask, int* idx) {
  __shared__ TopkSmem sm;
  const long r = blockIdx.x;
  const unsigned* cl = cnt + r * 2 * n;
  const unsigned* cg = cl + n;
  const uint32_t wl = 65536u - lq;
  block_topk<kTopkThreads>([=](int i) { return wl * (cl[i] + 1u) + lq * (cg[i] + 1u); }, n, k,
                           mask ? mask + r * ((n + 63) / 64) : nullptr, idx ? idx + r * (long)k : nullptr, sm);
}

hipError_t launch_topk_value(const float* score, int rows, int n, int k, uint64_t* mask, int* idx, hipStream_t s) {
  hipLaunchKernelGGL(topk_value_kernel, dim3(rows), dim3(kTopkThreads), 0, s, score, n, k, mask, idx);
  return hipGetLastError();
}

hipError_t launch_topk_blend(const float* score, const float* prior, int rows, int n, int k, uint32_t lq,
                             uint64_t* mask, int* idx, unsigned* cnt, hipStream_t s) {
  hipError_t e = launch_fill_zero(cnt, size_t(rows) * 2 * n * sizeof(unsigned), s);
  if (e != hipSuccess) return e;
  int chunks = (n + 2047) / 2048;
  if (chunks < 1) chunks = 1;
  if (chunks > 16) chunks = 16;
  dim3 grid((n + kRankThreads - 1) / kRankThreads, chunks, rows * 2);
  hipLaunchKernelGGL(rank_count_kernel, grid, dim3(kRankThreads), 0, s, score, prior, n, chunks, cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_blend_kernel, dim3(rows), dim3(kTopkThreads), 0, s, cnt, n, k, lq, mask, idx);
  return hipGetLastError();
}

}  // namespace as
