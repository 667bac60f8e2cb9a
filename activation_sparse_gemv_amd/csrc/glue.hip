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
// One decode token.  Workgroup (kv head g, key chunk c) takes at most kMaxKeys
// keys: the group's query heads, then every K row and then every V row of its
// chunk (16 lanes per 256-byte row, 16 rows per workgroup step, so at most 8 rows
// of each per thread) are loaded at entry, so the chunk costs one round trip to
// memory and the scores overlap the V rows still in flight.  Scores: each lane
// dots its 8 dimensions with the group's query heads and the 16 lanes of a row add
// theirs up with DPP row operations; the chunk's softmax statistics (max, sum of
// exponentials) per head come from LDS; the unnormalised partial output sums the
// value rows held in registers, reduced over the 16 rows in LDS in row order.  The
// last chunk of a kv head to finish merges the chunks in chunk order
// (deterministic), in registers.
constexpr int kAttThreads = 256;
constexpr int kMaxGroup = 8;      // query heads per kv head
constexpr int kAttHd = 128;       // head dimension of the vectorised path
constexpr int kMaxChunks = 256;   // chunks per kv head
constexpr int kMaxKeys = 128;     // keys per chunk: 8 row steps of 16
constexpr int kSteps = kMaxKeys / 16;

// Sum over the 16 lanes of each row (every lane of the row gets the row's sum).
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int s = 0; s < 4; ++s) v += dppf(v, s);
  return v;
}

template <int GM>
__global__ __launch_bounds__(kAttThreads) void attention_kernel(const AttnParams p) {
  extern __shared__ __align__(16) float sm[];
  constexpr int hd = kAttHd;
  const int grp = p.n_q / p.n_kv;
  const int g = blockIdx.x, c = blockIdx.y, C = gridDim.y;
  const int n_keys = p.n_ctx + 1;
  const int j0 = (int)((long)c * n_keys / C), j1 = (int)((long)(c + 1) * n_keys / C);
  const int nk = j1 - j0;                  // <= kMaxKeys (the host sizes C)
  float* qs = sm;                          // [GM][hd] query heads of the group, pre-scaled
  float* sc = qs + GM * hd;                // [GM][kMaxKeys] scores, then exp(score - max)
  float* red = sc + GM * kMaxKeys;         // [16][GM][hd] per key-row partial outputs
  __shared__ float s_m[kMaxGroup], s_l[kMaxGroup];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = tid >> 4, l16 = tid & 15;   // key row slot 0..15, 8 dimensions 8 l16 ..
  const int dd0 = 8 * l16;

  // the group's query heads first (small, read by every key row), then every K row
  // and then every V row of the chunk, issued together: the scores start as the K
  // rows arrive while the V rows are still in flight (rows past the chunk repeat its
  // last row; the current token's own row is fp32 and taken apart below)
  constexpr int kQPer = (GM * kAttHd + kAttThreads - 1) / kAttThreads;
  float qv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int i = tid + u * kAttThreads;
    qv[u] = i < grp * hd ? p.q[(long)(g * grp) * hd + i] : 0.f;
  }
  const bool has_fresh = j1 == n_keys;     // this chunk holds the current token's key
  float kf[8], vf[8];
  if (has_fresh) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = p.k_new[(long)g * hd + dd0 + e];
      vf[e] = p.v_new[(long)g * hd + dd0 + e];
    }
  }
  u32x4 kr[kSteps], vr[kSteps];
  long roff[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    int jj = ks + 16 * s;
    jj = jj < nk ? jj : nk - 1;
    int j = j0 + jj;
    j = j < p.n_ctx ? j : (p.n_ctx > 0 ? p.n_ctx - 1 : 0);
    roff[s] = ((long)j * p.n_kv + g) * hd + dd0;
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
    kr[s] = p.n_ctx > 0 ? *reinterpret_cast<const u32x4*>(p.k_cache + roff[s]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
    vr[s] = p.n_ctx > 0 ? *reinterpret_cast<const u32x4*>(p.v_cache + roff[s]) : u32x4{0u, 0u, 0u, 0u};
  const float scale = 1.0f / sqrtf((float)hd);
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int i = tid + u * kAttThreads;
    if (i < grp * hd) qs[i] = qv[u] * scale;
  }
  __syncthreads();

  // scores
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int jj = ks + 16 * s;
    if (16 * s < nk) {                     // uniform over the workgroup
      float kv[8];
      if (has_fresh && j0 + jj == p.n_ctx) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = kf[e];
      } else {
        unpack8<DT_BF16>(kr[s], kv);
      }
#pragma unroll
      for (int a = 0; a < GM; ++a) {
        if (a < grp) {
          const float4 q0 = *reinterpret_cast<const float4*>(qs + a * hd + dd0);
          const float4 q1 = *reinterpret_cast<const float4*>(qs + a * hd + dd0 + 4);
          float v = q0.x * kv[0];
          v = fmaf(q0.y, kv[1], v);
          v = fmaf(q0.z, kv[2], v);
          v = fmaf(q0.w, kv[3], v);
          v = fmaf(q1.x, kv[4], v);
          v = fmaf(q1.y, kv[5], v);
          v = fmaf(q1.z, kv[6], v);
          v = fmaf(q1.w, kv[7], v);
          v = row16_sum(v);
          if (l16 == 0 && jj < nk) sc[a * kMaxKeys + jj] = v;
        }
      }
    }
  }
  __syncthreads();
  // chunk softmax statistics per query head (one wave per head)
  for (int a = wave; a < grp; a += kAttThreads / 64) {
    float m = -INFINITY;
    for (int t = lane; t < nk; t += 64) m = fmaxf(m, sc[a * kMaxKeys + t]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < nk; t += 64) {
      const float e = expf(sc[a * kMaxKeys + t] - m);
      sc[a * kMaxKeys + t] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { s_m[a] = m; s_l[a] = l; }
  }
  __syncthreads();
  // unnormalised partial outputs of this thread's rows and 8 dimensions
  {
    float acc[GM][8];
#pragma unroll
    for (int a = 0; a < GM; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[a][e] = 0.f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int jj = ks + 16 * s;
      if (jj < nk) {
        float vv[8];
        if (has_fresh && j0 + jj == p.n_ctx) {
#pragma unroll
          for (int e = 0; e < 8; ++e) vv[e] = vf[e];
        } else {
          unpack8<DT_BF16>(vr[s], vv);
        }
#pragma unroll
        for (int a = 0; a < GM; ++a)
          if (a < grp) {
            const float pa = sc[a * kMaxKeys + jj];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[a][e] = fmaf(pa, vv[e], acc[a][e]);
          }
      }
    }
#pragma unroll
    for (int a = 0; a < GM; ++a)
      if (a < grp) {
        float4* dst = reinterpret_cast<float4*>(red + (ks * GM + a) * hd + dd0);
        dst[0] = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
        dst[1] = make_float4(acc[a][4], acc[a][5], acc[a][6], acc[a][7]);
      }
  }
  __syncthreads();
  for (int i = tid; i < grp * hd; i += kAttThreads) {
    const int a = i / hd, dd = i % hd;
    float o = 0.f;
    for (int r = 0; r < 16; ++r) o += red[(r * GM + a) * hd + dd];
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
  // merge: O = sum_c exp(m_c - M) o_c / sum_c exp(m_c - M) l_c per query head, M the
  // largest chunk maximum, chunks in chunk order.  Thread t takes kPer consecutive
  // outputs of one head; the statistics and partial outputs of a batch of chunks
  // are loaded at once (one round trip per batch) and everything else stays in
  // registers (no LDS, no barrier).  Over several batches the running sums are
  // rescaled to the new maximum; with one batch (C <= kB) the arithmetic is the
  // two-pass formula.
  constexpr int kPer = GM * kAttHd >= kAttThreads ? GM * kAttHd / kAttThreads : 1;
  constexpr int kB = GM >= 8 ? 16 : 32;
  const int i0 = tid * kPer;
  if (i0 >= grp * hd) return;
  const int a = i0 / hd;
  float M = -INFINITY, L = 0.f, O[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) O[u] = 0.f;
  for (int c0 = 0; c0 < C; c0 += kB) {
    float mc[kB], lc[kB], ov[kPer][kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const long rec = ((long)g * C + min(c0 + k, C - 1)) * grp + a;
      // (m, l) and the kPer outputs are adjacent: 8-byte coherent loads
      const uint64_t ml = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p.part_ml + rec * 2),
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      mc[k] = __uint_as_float((uint32_t)ml);
      lc[k] = __uint_as_float((uint32_t)(ml >> 32));
      const float* po = p.part_o + rec * hd + i0 % hd;
      if constexpr (kPer % 2 == 0) {
#pragma unroll
        for (int u = 0; u < kPer; u += 2) {
          const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(po + u), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          ov[u][k] = __uint_as_float((uint32_t)v);
          ov[u + 1][k] = __uint_as_float((uint32_t)(v >> 32));
        }
      } else {
#pragma unroll
        for (int u = 0; u < kPer; ++u) ov[u][k] = load_coherent(po + u);
      }
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (c0 + k < C) Mb = fmaxf(Mb, mc[k]);
    if (M != -INFINITY) {
      const float r = expf(M - Mb);
      L *= r;
#pragma unroll
      for (int u = 0; u < kPer; ++u) O[u] *= r;
    }
#pragma unroll
    for (int k = 0; k < kB; ++k)
      if (c0 + k < C) {
        const float w = expf(mc[k] - Mb);
        L = fmaf(w, lc[k], L);
#pragma unroll
        for (int u = 0; u < kPer; ++u) O[u] = fmaf(w, ov[u][k], O[u]);
      }
    M = Mb;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) p.o[(long)(g * grp + a) * hd + (i0 + u) % hd] = O[u] / L;
}

template <int GM>
hipError_t launch_attention_g(const AttnParams& p, int chunks, hipStream_t s) {
  const size_t smem = (size_t(GM) * kAttHd + size_t(GM) * kMaxKeys + size_t(16) * GM * kAttHd) * 4;
  auto k = attention_kernel<GM>;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       int(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(p.n_kv, chunks), dim3(kAttThreads), smem, s, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, int chunks, hipStream_t s) {
  const int grp = p.n_q / p.n_kv;
  if (chunks < 1 || chunks > kMaxChunks || (p.n_ctx + 1 + chunks - 1) / chunks > kMaxKeys) return hipErrorInvalidValue;
  if (grp <= 1) return launch_attention_g<1>(p, chunks, s);
  if (grp <= 2) return launch_attention_g<2>(p, chunks, s);
  if (grp <= 4) return launch_attention_g<4>(p, chunks, s);
  return launch_attention_g<8>(p, chunks, s);
}

int attention_max_group() { return kMaxGroup; }
int attention_head_dim() { return kAttHd; }
int attention_max_chunks() { return kMaxChunks; }
int attention_max_keys() { return kMaxKeys; }

}  // namespace as
