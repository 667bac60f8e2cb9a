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
constexpr int kAttThreads = 256;
constexpr int kMaxGroup = 8;      // query heads per kv head
constexpr int kMaxHd = 256;

__global__ __launch_bounds__(kAttThreads) void attention_kernel(const AttnParams p) {
  extern __shared__ __align__(16) float sm[];
  const int hd = p.head_dim, grp = p.n_q / p.n_kv;
  const int g = blockIdx.x, c = blockIdx.y, C = gridDim.y;
  const int n_keys = p.n_ctx + 1;
  const int j0 = (int)((long)c * n_keys / C), j1 = (int)((long)(c + 1) * n_keys / C);
  const int nk = j1 - j0;
  float* qs = sm;                          // [grp][hd]  (pre-scaled)
  float* sc = qs + grp * hd;               // [grp][chunk]
  __shared__ float s_m[kMaxGroup], s_l[kMaxGroup];
  __shared__ int s_last;
  const float scale = 1.0f / sqrtf((float)hd);
  for (int i = threadIdx.x; i < grp * hd; i += kAttThreads) {
    const int qh = g * grp + i / hd, dd = i % hd;
    qs[i] = p.q[(long)qh * hd + dd] * scale;
  }
  __syncthreads();
  // scores: wave w takes keys j0 + w, j0 + w + 4, ...; lanes split the head dim
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = j0 + wave; j < j1; j += kAttThreads / 64) {
    float part[kMaxGroup];
#pragma unroll
    for (int a = 0; a < kMaxGroup; ++a) part[a] = 0.f;
    for (int dd = lane; dd < hd; dd += 64) {
      const float kv = j < p.n_ctx ? bf16_bits_to_f32(p.k_cache[((long)j * p.n_kv + g) * hd + dd])
                                   : p.k_new[(long)g * hd + dd];
#pragma unroll
      for (int a = 0; a < kMaxGroup; ++a)
        if (a < grp) part[a] = fmaf(qs[a * hd + dd], kv, part[a]);
    }
#pragma unroll
    for (int a = 0; a < kMaxGroup; ++a) {
      if (a < grp) {
        const float s = wave_sum(part[a]);
        if (lane == 0) sc[a * nk + (j - j0)] = s;
      }
    }
  }
  __syncthreads();
  // chunk softmax statistics per query head (one wave per head, looping)
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
  // unnormalised partial outputs: thread -> (head a, dim dd)
  for (int i = threadIdx.x; i < grp * hd; i += kAttThreads) {
    const int a = i / hd, dd = i % hd;
    float o = 0.f;
    for (int t = 0; t < nk; ++t) {
      const int j = j0 + t;
      const float vv = j < p.n_ctx ? bf16_bits_to_f32(p.v_cache[((long)j * p.n_kv + g) * hd + dd])
                                   : p.v_new[(long)g * hd + dd];
      o = fmaf(sc[a * nk + t], vv, o);
    }
    const long base = ((long)g * C + c) * grp + a;          // partial record index
    store_coherent(p.part_o + base * hd + dd, o);
    if (dd == 0) {
      store_coherent(p.part_ml + base * 2, s_m[a]);
      store_coherent(p.part_ml + base * 2 + 1, s_l[a]);
    }
  }
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.counters + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == unsigned(C - 1);
    if (s_last) __hip_atomic_store(p.counters + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  // merge: O = sum_c exp(m_c - M) o_c / sum_c exp(m_c - M) l_c
  for (int i = threadIdx.x; i < grp * hd; i += kAttThreads) {
    const int a = i / hd, dd = i % hd;
    float M = -INFINITY;
    for (int cc = 0; cc < C; ++cc) M = fmaxf(M, load_coherent(p.part_ml + (((long)g * C + cc) * grp + a) * 2));
    float L = 0.f, O = 0.f;
    for (int cc = 0; cc < C; ++cc) {
      const long base = ((long)g * C + cc) * grp + a;
      const float w = expf(load_coherent(p.part_ml + base * 2) - M);
      L = fmaf(w, load_coherent(p.part_ml + base * 2 + 1), L);
      O = fmaf(w, load_coherent(p.part_o + base * hd + dd), O);
    }
    p.o[(long)(g * grp + a) * hd + dd] = O / L;
  }
}

hipError_t launch_attention(const AttnParams& p, int chunks, hipStream_t s) {
  const int grp = p.n_q / p.n_kv;
  const int n_keys = p.n_ctx + 1;
  const int max_chunk = (n_keys + chunks - 1) / chunks;
  const size_t smem = size_t(grp) * p.head_dim * 4 + size_t(grp) * max_chunk * 4;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attention_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attention_kernel, dim3(p.n_kv, chunks), dim3(kAttThreads), smem, s, p);
  return hipGetLastError();
}

int attention_max_group() { return kMaxGroup; }
int attention_max_head_dim() { return kMaxHd; }

}  // namespace as
