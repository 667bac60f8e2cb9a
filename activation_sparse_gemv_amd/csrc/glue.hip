// Decoder-block glue around the sparse projections: RMSNorm and dense GQA decode
// attention.  TEAL slides, method slide: the inputs of the attention and MLP
// projections are sparsified while the attention core itself stays dense.
// Readings taken (the pages describe no block): pre-norm RMSNorm with unit gain,
// no rotary embedding, query head h reads key/value head h / (n_q / n_kv), and
// the keys are the cached context plus the current token's own key.
#include "common.hpp"
#include "internal.hpp"

namespace as {

// ---------------------------------------------------------------- RMSNorm
constexpr int kNormThreads = 256;

// y[r] = x[r] / sqrt(mean(x[r]^2) + eps) in fp32; copy[r] = x[r] (fp32) if given.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const void* x, int x_dt, int d, float eps, float* y,
                                                               float* copy) {
  __shared__ float s_part[kNormThreads / 64];
  const long r = blockIdx.x;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += kNormThreads) {
    const float v = load_elem(x, x_dt, r * d + i);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < kNormThreads / 64; ++w) tot += s_part[w];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += kNormThreads) {
    const float v = load_elem(x, x_dt, r * d + i);
    y[r * d + i] = v * inv;
    if (copy != nullptr) copy[r * d + i] = v;
  }
}

hipError_t launch_rmsnorm(const void* x, int x_dt, int rows, int d, float eps, float* y, float* copy, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(kNormThreads), 0, s, x, x_dt, d, eps, y, copy);
  return hipGetLastError();
}

// ---------------------------------------------------------------- attention
// One decode token.  Workgroup (kv head g, key chunk c) scores its chunk of
// keys against the n_q / n_kv query heads of the group, keeps the chunk's
// running max and exp-sum, and its unnormalised partial output; the last chunk
// of a kv head to finish merges the chunks in chunk order (deterministic).
// Loads are 16-byte: four lanes share one 256-byte key row for the scores, and
// sixteen lanes one value row for the output.
constexpr int kAttThreads = 256;
constexpr int kMaxGroup = 8;      // query heads per kv head
constexpr int kAttHd = 128;       // head dimension of the vectorised path
constexpr int kMaxChunks = 64;

__device__ __forceinline__ void kv_row8(const uint16_t* cache, const float* fresh, bool from_cache, long off,
                                        float v[8]) {
  if (from_cache) {
    unpack8<DT_BF16>(*reinterpret_cast<const u32x4*>(cache + off), v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fresh[off + e];
  }
}

__global__ __launch_bounds__(kAttThreads) void attention_kernel(const AttnParams p) {
  extern __shared__ __align__(16) float sm[];
  constexpr int hd = kAttHd;
  const int grp = p.n_q / p.n_kv;
  const int g = blockIdx.x, c = blockIdx.y, C = gridDim.y;
  const int n_keys = p.n_ctx + 1;
  const int j0 = (int)((long)c * n_keys / C), j1 = (int)((long)(c + 1) * n_keys / C);
  const int nk = j1 - j0;
  float* qs = sm;                          // [grp][hd]  (pre-scaled)
  float* sc = qs + grp * hd;               // [grp][nk]
  float* red = sc + grp * ((nk + 3) & ~3); // [16][grp][hd] output partials per key group
  __shared__ float s_m[kMaxGroup], s_l[kMaxGroup];
  __shared__ float s_ml[kMaxChunks * kMaxGroup * 2];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float scale = 1.0f / sqrtf((float)hd);
  for (int i = tid; i < grp * hd; i += kAttThreads) {
    const int qh = g * grp + i / hd, dd = i % hd;
    qs[i] = p.q[(long)qh * hd + dd] * scale;
  }
  __syncthreads();
  // scores: four lanes per key, 32 dimensions (four 16-byte loads) each
  {
    const int part = tid & 3, d0 = part * 32;
    for (int jj = tid >> 2; jj < nk; jj += kAttThreads / 4) {
      const int j = j0 + jj;
      const bool fromc = j < p.n_ctx;
      const long off = fromc ? ((long)j * p.n_kv + g) * hd + d0 : (long)g * hd + d0;
      float acc[kMaxGroup];
#pragma unroll
      for (int a = 0; a < kMaxGroup; ++a) acc[a] = 0.f;
#pragma unroll
      for (int v8 = 0; v8 < 4; ++v8) {
        float kv[8];
        kv_row8(p.k_cache, p.k_new, fromc, off + v8 * 8, kv);
#pragma unroll
        for (int a = 0; a < kMaxGroup; ++a)
          if (a < grp)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[a] = fmaf(qs[a * hd + d0 + v8 * 8 + e], kv[e], acc[a]);
      }
#pragma unroll
      for (int a = 0; a < kMaxGroup; ++a) {
        float v = acc[a];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        if (part == 0 && a < grp) sc[a * nk + jj] = v;
      }
    }
  }
  __syncthreads();
  // chunk softmax statistics per query head (one wave per head)
  for (int a = wave; a < grp; a += kAttThreads / 64) {
    float m = -INFINITY;
    for (int t = lane; t < nk; t += 64) m = fmaxf(m, sc[a * nk + t]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float l = 0.f;
    for (int t = lane; t < nk; t += 64) {
      const float e = expf(sc[a * nk + t] - m);
      sc[a * nk + t] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { s_m[a] = m; s_l[a] = l; }
  }
  __syncthreads();
  // unnormalised partial outputs: thread = (key group kg of 16, 8 dims dg of 16)
  {
    const int dg = tid & 15, kg = tid >> 4;
    float acc[kMaxGroup][8];
#pragma unroll
    for (int a = 0; a < kMaxGroup; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[a][e] = 0.f;
    for (int jj = kg; jj < nk; jj += 16) {
      const int j = j0 + jj;
      const bool fromc = j < p.n_ctx;
      const long off = fromc ? ((long)j * p.n_kv + g) * hd + dg * 8 : (long)g * hd + dg * 8;
      float vv[8];
      kv_row8(p.v_cache, p.v_new, fromc, off, vv);
#pragma unroll
      for (int a = 0; a < kMaxGroup; ++a)
        if (a < grp) {
          const float pa = sc[a * nk + jj];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[a][e] = fmaf(pa, vv[e], acc[a][e]);
        }
    }
#pragma unroll
    for (int a = 0; a < kMaxGroup; ++a)
      if (a < grp)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[(kg * grp + a) * hd + dg * 8 + e] = acc[a][e];
  }
  __syncthreads();
  for (int i = tid; i < grp * hd; i += kAttThreads) {
    const int a = i / hd, dd = i % hd;
    float o = 0.f;
    for (int kg = 0; kg < 16; ++kg) o += red[(kg * grp + a) * hd + dd];
    const long base = ((long)g * C + c) * grp + a;          // partial record index
    store_coherent(p.part_o + base * hd + dd, o);
    if (dd == 0) {
      store_coherent(p.part_ml + base * 2, s_m[a]);
      store_coherent(p.part_ml + base * 2 + 1, s_l[a]);
    }
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.counters + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == unsigned(C - 1);
    if (s_last) __hip_atomic_store(p.counters + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  // merge: O = sum_c exp(m_c - M) o_c / sum_c exp(m_c - M) l_c.  The partial outputs
  // of 32 chunks of every output of this thread are loaded together, issued before
  // the chunk statistics are waited for; the weights exp(m_c - M) and the sums L
  // depend on (chunk, head) only and are formed once in LDS.  Chunks are merged in
  // chunk order.
  constexpr int kOut = kMaxGroup * kAttHd / kAttThreads;
  const int n_out = (grp * hd + kAttThreads - 1) / kAttThreads;      // in use (uniform)
  float ov[kOut][32];
  auto load_ov = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kOut; ++u) {
      if (u < n_out) {
        const int i = min(tid + u * kAttThreads, grp * hd - 1), a = i / hd, dd = i % hd;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const int cc = min(c0 + k, C - 1);
          ov[u][k] = load_coherent(p.part_o + (((long)g * C + cc) * grp + a) * hd + dd);
        }
      }
    }
  };
  load_ov(0);
  for (int i = tid; i < C * grp * 2; i += kAttThreads) s_ml[i] = load_coherent(p.part_ml + (long)g * C * grp * 2 + i);
  __syncthreads();
  __shared__ float s_M[kMaxGroup], s_L[kMaxGroup];
  __shared__ float s_w[kMaxChunks * kMaxGroup];                     // [C][grp] merge weights
  if (tid < grp) {
    float M = -INFINITY;
    for (int cc = 0; cc < C; ++cc) M = fmaxf(M, s_ml[(cc * grp + tid) * 2]);
    s_M[tid] = M;
  }
  __syncthreads();
  for (int i = tid; i < C * grp; i += kAttThreads) s_w[i] = expf(s_ml[i * 2] - s_M[i % grp]);
  __syncthreads();
  if (tid < grp) {
    float L = 0.f;
    for (int cc = 0; cc < C; ++cc) L = fmaf(s_w[cc * grp + tid], s_ml[(cc * grp + tid) * 2 + 1], L);
    s_L[tid] = L;
  }
  __syncthreads();
  float O[kOut];
#pragma unroll
  for (int u = 0; u < kOut; ++u) O[u] = 0.f;
  for (int c0 = 0; c0 < C; c0 += 32) {
    if (c0 > 0) load_ov(c0);
#pragma unroll
    for (int u = 0; u < kOut; ++u) {
      if (u < n_out) {
        const int a = min(tid + u * kAttThreads, grp * hd - 1) / hd;
#pragma unroll
        for (int k = 0; k < 32; ++k)
          if (c0 + k < C) O[u] = fmaf(s_w[(c0 + k) * grp + a], ov[u][k], O[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kOut; ++u) {
    const int i = tid + u * kAttThreads;
    if (u < n_out && i < grp * hd) {
      const int a = i / hd;
      p.o[(long)(g * grp + a) * hd + i % hd] = O[u] / s_L[a];
    }
  }
}

hipError_t launch_attention(const AttnParams& p, int chunks, hipStream_t s) {
  const int grp = p.n_q / p.n_kv;
  const int n_keys = p.n_ctx + 1;
  const int max_chunk = (n_keys + chunks - 1) / chunks;
  const size_t smem = size_t(grp) * kAttHd * 4 + size_t(grp) * ((max_chunk + 3) & ~3) * 4 +
                      size_t(16) * grp * kAttHd * 4;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attention_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attention_kernel, dim3(p.n_kv, chunks), dim3(kAttThreads), smem, s, p);
  return hipGetLastError();
}

int attention_max_group() { return kMaxGroup; }
int attention_head_dim() { return kAttHd; }
int attention_max_chunks() { return kMaxChunks; }

}  // namespace as
