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
// One decode token.  The n_ctx cached keys of each kv head are cut into C equal
// chunks of at most 32 * KS keys; the current token's own key (fp32) rides with the
// last chunk as one extra row.  Workgroup (kv head g, chunk c): 32 row slots of 16
// lanes (one 256-byte row per slot and step, 8 dimensions per lane; two waves per
// SIMD, so the dependent score and value chains of one wave hide behind the
// other's).  The group's query heads go straight from memory into registers, then
// every K row and every V row of the chunk are issued, so the chunk costs one round
// trip and the scores overlap the V rows still in flight.  Scores: 8-dimension dot
// products summed over the 16 lanes of a row by DPP, kept in registers; the chunk
// maximum per head from per-wave maxima through LDS (first barrier); exponentials
// (base 2: the query scale carries log2(e), so every exponential is one hardware
// exp2) and the value sums in registers; the partial outputs of a wave's four slots
// added by cross-row lane swaps, then the eight waves' through LDS in wave order
// (second barrier).  These phases are bound by instructions and latency, so heads
// past the group and slots past the chunk are masked by selects, never branched
// over.  The chunk's (max, sum, output) record is stored device-coherently and
// counted; the last chunk of a kv head to arrive merges every record of the head
// in one round trip: the statistics give each chunk its weight 2^(m_c - M) (M the
// largest chunk maximum), the weighted outputs are added in chunk order and divided
// by sum_c 2^(m_c - M) l_c (deterministic).
constexpr int kAttThreads = 512;
constexpr int kSlots = kAttThreads / 16;   // row slots
constexpr int kMaxGroup = 8;      // query heads per kv head
constexpr int kAttHd = 128;       // head dimension of the vectorised path
constexpr int kMaxChunks = 256;   // chunks per kv head
constexpr int kMaxKeys = 128;     // cached keys per chunk: 4 row steps of 32

// Sum over the 16 lanes of each row (every lane of the row gets the row's sum).
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int s = 0; s < 4; ++s) v += dppf(v, s);
  return v;
}

__device__ __forceinline__ float dot8(const float (&q)[8], const float (&k)[8]) {
  float v = q[0] * k[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) v = fmaf(q[e], k[e], v);
  return v;
}

// Phase timeline (libactsparse_timeline.so only): thread 0 of each workgroup writes
// the device's 100 MHz clock at the phase boundaries listed with
// as_attention_timeline_arm.
#ifdef AS_PHASE_TIMELINE
#define AS_ATT_PHASE(p, slot)                                                                           \
  do {                                                                                                  \
    if ((p).phase_tl != nullptr && threadIdx.x == 0)                                                    \
      (p).phase_tl[((long)blockIdx.x + (long)gridDim.x * blockIdx.y) * 16 + (slot)] =                   \
          __builtin_amdgcn_s_memrealtime();                                                              \
  } while (0)
#else
#define AS_ATT_PHASE(p, slot) do {} while (0)
#endif

// 2^x by the hardware instruction alone (no range fix-up: arguments below -126,
// whose results would be subnormal, give 0 or a subnormal; softmax weights that
// small do not change a sum of weights of which the largest is 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two adjacent fp32 values read device-coherently (one 8-byte load).
__device__ __forceinline__ float2 load_coherent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

template <int GM, int KS>
__global__ __launch_bounds__(kAttThreads) void attention_kernel(const AttnParams p) {
  extern __shared__ __align__(16) float red[];   // [NWV][GM][hd] wave partial outputs; merge weights later
  constexpr int NWV = kAttThreads / 64;
  __shared__ __align__(16) float s_mx[NWV * GM];
  __shared__ float s_ls[NWV * GM], s_L[GM];
  __shared__ int s_last;
  constexpr int hd = kAttHd;
  const int grp = p.n_q / p.n_kv;
  const int g = blockIdx.x, c = blockIdx.y, C = gridDim.y;
  const int j0 = (int)((long)c * p.n_ctx / C), j1 = (int)((long)(c + 1) * p.n_ctx / C);
  const int nk = j1 - j0;                  // cached keys of the chunk, <= kSlots * KS (the host sizes C)
  const bool has_fresh = c == C - 1;       // the current token's key and value
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = tid >> 4, l16 = tid & 15;   // row slot 0..31, dimensions 8 l16 .. 8 l16 + 7
  const int dd0 = 8 * l16;
  AS_ATT_PHASE(p, 0);

  // this lane's 8 dimensions of every query head of the group, scaled by
  // log2(e) / sqrt(hd): the scores are in base-2 units
  const float scale = 1.4426950408889634f / sqrtf((float)hd);
  float qv[GM][8];
#pragma unroll
  for (int a = 0; a < GM; ++a) {
    if (a < grp) {
      const float4* qp = reinterpret_cast<const float4*>(p.q + (long)(g * grp + a) * hd + dd0);
      const float4 x0 = qp[0], x1 = qp[1];
      qv[a][0] = x0.x * scale; qv[a][1] = x0.y * scale; qv[a][2] = x0.z * scale; qv[a][3] = x0.w * scale;
      qv[a][4] = x1.x * scale; qv[a][5] = x1.y * scale; qv[a][6] = x1.z * scale; qv[a][7] = x1.w * scale;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[a][e] = 0.f;
    }
  }
  float kf[8], vf[8];
  if (has_fresh) {
    const float4* kp = reinterpret_cast<const float4*>(p.k_new + (long)g * hd + dd0);
    const float4* vp = reinterpret_cast<const float4*>(p.v_new + (long)g * hd + dd0);
    const float4 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
    kf[0] = k0.x; kf[1] = k0.y; kf[2] = k0.z; kf[3] = k0.w; kf[4] = k1.x; kf[5] = k1.y; kf[6] = k1.z; kf[7] = k1.w;
    vf[0] = v0.x; vf[1] = v0.y; vf[2] = v0.z; vf[3] = v0.w; vf[4] = v1.x; vf[5] = v1.y; vf[6] = v1.z; vf[7] = v1.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[e] = vf[e] = 0.f;
  }

  // K rows, then V rows (slots past the chunk re-read its last row; their weights
  // are 0 and they are skipped in the value sums)
  u32x4 kr[KS], vr[KS];
  if (nk > 0) {
    long roff[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) roff[s] = ((long)(j0 + min(ks + kSlots * s, nk - 1)) * p.n_kv + g) * hd + dd0;
#pragma unroll
    for (int s = 0; s < KS; ++s) kr[s] = *reinterpret_cast<const u32x4*>(p.k_cache + roff[s]);
#pragma unroll
    for (int s = 0; s < KS; ++s) vr[s] = *reinterpret_cast<const u32x4*>(p.v_cache + roff[s]);
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) kr[s] = vr[s] = u32x4{0u, 0u, 0u, 0u};
  }
  // scores: sc[s][a] for the row of slot ks at step s; step KS is the current
  // token's key, held by slot 0 of the last chunk (-inf marks no row)
  float sc[KS + 1][GM];
  // every head and step is computed (no branch per head: the heads' dot products and
  // DPP sums are independent chains the compiler can interleave); heads past the
  // group (zero queries) and slots past the chunk are masked to -inf by selects
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const bool valid = ks + kSlots * s < nk;
    float kv[8];
    unpack8<DT_BF16>(kr[s], kv);
#pragma unroll
    for (int a = 0; a < GM; ++a) {
      const float v = row16_sum(dot8(qv[a], kv));
      sc[s][a] = (valid && a < grp) ? v : -INFINITY;
    }
  }
  if (has_fresh) {                         // uniform over the workgroup
#pragma unroll
    for (int a = 0; a < GM; ++a) {
      const float v = row16_sum(dot8(qv[a], kf));
      sc[KS][a] = (ks == 0 && a < grp) ? v : -INFINITY;
    }
  } else {
#pragma unroll
    for (int a = 0; a < GM; ++a) sc[KS][a] = -INFINITY;
  }
  AS_ATT_PHASE(p, 1);
  // chunk maximum per head: the wave's maximum over its 4 row slots (every lane of
  // a slot holds the slot's value), one entry per wave in LDS
#pragma unroll
  for (int a = 0; a < GM; ++a) {
    float m = sc[0][a];
#pragma unroll
    for (int s = 1; s <= KS; ++s) m = fmaxf(m, sc[s][a]);
    m = fmaxf(fmaxf(readlane_f(m, 0), readlane_f(m, 16)), fmaxf(readlane_f(m, 32), readlane_f(m, 48)));
    if (lane == 0) s_mx[wave * GM + a] = m;
  }
  __syncthreads();
  AS_ATT_PHASE(p, 2);
  float l_loc[GM];
  float Mx[GM];
#pragma unroll
  for (int a = 0; a < GM; ++a) Mx[a] = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    if constexpr (GM % 4 == 0) {
#pragma unroll
      for (int a = 0; a < GM; a += 4) {
        const float4 v = *reinterpret_cast<const float4*>(s_mx + w * GM + a);
        Mx[a] = fmaxf(Mx[a], v.x); Mx[a + 1] = fmaxf(Mx[a + 1], v.y);
        Mx[a + 2] = fmaxf(Mx[a + 2], v.z); Mx[a + 3] = fmaxf(Mx[a + 3], v.w);
      }
    } else {
#pragma unroll
      for (int a = 0; a < GM; ++a) Mx[a] = fmaxf(Mx[a], s_mx[w * GM + a]);
    }
  }
#pragma unroll
  for (int a = 0; a < GM; ++a) {
    // a row without a key has score -inf and weight 2^-inf = 0; a chunk maximum of
    // -inf (no finite score) is taken as 0 so that -inf - M is not NaN
    const float M = Mx[a] == -INFINITY ? 0.f : Mx[a];
    float l = 0.f;
#pragma unroll
    for (int s = 0; s <= KS; ++s) {
      const float e = fast_exp2(sc[s][a] - M);
      sc[s][a] = e;
      l += e;
    }
    l_loc[a] = (readlane_f(l, 0) + readlane_f(l, 16)) + (readlane_f(l, 32) + readlane_f(l, 48));
  }
  // unnormalised partial outputs of this slot's rows, 8 dimensions.  Every step is
  // summed without a branch: a slot past the chunk (weight 0) has its re-read row
  // replaced by zeros, so it adds exactly 0 whatever that row holds; heads past the
  // group have weight 0 and are never read out.
  float acc[GM][8];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const bool valid = ks + kSlots * s < nk;
    u32x4 v = vr[s];
    v.x = valid ? v.x : 0u;
    v.y = valid ? v.y : 0u;
    v.z = valid ? v.z : 0u;
    v.w = valid ? v.w : 0u;
    float vv[8];
    unpack8<DT_BF16>(v, vv);
#pragma unroll
    for (int a = 0; a < GM; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[a][e] = s == 0 ? sc[0][a] * vv[e] : fmaf(sc[s][a], vv[e], acc[a][e]);
  }
  if (has_fresh && ks == 0) {
#pragma unroll
    for (int a = 0; a < GM; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[a][e] = fmaf(sc[KS][a], vf[e], acc[a][e]);
  }
  // The wave's four row slots are summed with cross-row lane swaps: four values
  // (A, B, E, F) become one register whose row r holds the slot sum of the value
  // 4q + {0, 2, 1, 3}[r], i.e. (A.R0 + A.R2) + (A.R1 + A.R3) etc. (fixed order).
  constexpr int NQ = GM * 8 / 4;
  float outq[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int v = 4 * q;
    const float A = acc[v / 8][v % 8], B = acc[(v + 1) / 8][(v + 1) % 8];
    const float E = acc[(v + 2) / 8][(v + 2) % 8], F = acc[(v + 3) / 8][(v + 3) % 8];
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(A), __float_as_uint(B), false, false);
    const float Cq = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(E), __float_as_uint(F), false, false);
    const float Dq = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(Cq), __float_as_uint(Dq), false, false);
    outq[q] = __uint_as_float(z[0]) + __uint_as_float(z[1]);
  }
  {
    const int rr = lane >> 4;
    const int pr = rr == 1 ? 2 : (rr == 2 ? 1 : rr);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int v = 4 * q + pr, a = v >> 3, e = v & 7;
      red[(wave * GM + a) * hd + dd0 + e] = outq[q];
    }
#pragma unroll
    for (int a = 0; a < GM; ++a)
      if (a < grp && lane == 0) s_ls[wave * GM + a] = l_loc[a];
  }
  __syncthreads();
  AS_ATT_PHASE(p, 3);
  // the chunk's record: outputs summed over the waves in wave order, (max, sum)
  for (int i = tid; i < grp * hd; i += kAttThreads) {
    const int a = i / hd, dd = i % hd;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) o += red[(w * GM + a) * hd + dd];
    const long rec = ((long)g * C + c) * grp + a;
    store_coherent(p.part_o + rec * hd + dd, o);
  }
  if (tid < grp) {
    float M = s_mx[tid], l = 0.f;
#pragma unroll
    for (int w = 1; w < NWV; ++w) M = fmaxf(M, s_mx[w * GM + tid]);
#pragma unroll
    for (int w = 0; w < NWV; ++w) l += s_ls[w * GM + tid];
    const long rec = ((long)g * C + c) * grp + tid;
    store_coherent(p.part_ml + rec * 2, M);
    store_coherent(p.part_ml + rec * 2 + 1, l);
  }
  wait_vmem();
  AS_ATT_PHASE(p, 4);
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.counters + (long)g * kCounterStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == unsigned(C - 1);
    if (s_last) __hip_atomic_store(p.counters + (long)g * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  AS_ATT_PHASE(p, 5);
  if (!s_last) return;

  // merge.  Wave w takes head a = w % GM and the w / GM-th of NWV / GM equal runs of
  // chunks; a record (128 floats) is one 512-byte load instruction of the wave,
  // lane l holding dimensions 2l, 2l + 1.  Every wave first loads its head's
  // statistics (lane c: chunks c, c + 64, ..), then a batch of up to kB records;
  // the chunk weights 2^(m_c - M) go to LDS while the records are in flight.  The
  // runs are added in order through LDS at the end.
  constexpr int WPH = NWV / GM;            // waves per head
  constexpr int kB = 16;
  const int a = min(wave % GM, grp - 1), run = wave / GM;
  const bool live = wave % GM < grp;
  const int cb = run * C / WPH, ce = (run + 1) * C / WPH;
  float2 ml[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int cc = min(lane + 64 * u, C - 1);
    ml[u] = load_coherent2(p.part_ml + (((long)g * C + cc) * grp + a) * 2);
  }
  float2 ob[kB];
  const float* rec0 = p.part_o + ((long)g * C * grp + a) * hd + 2 * lane;
  const long rec_ld = (long)grp * hd;      // floats between the records of consecutive chunks
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int k = 0; k < kB; ++k) ob[k] = load_coherent2(rec0 + (long)min(c0 + k, C - 1) * rec_ld);
  };
  load_batch(cb);
  float Mh = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (lane + 64 * u < C) Mh = fmaxf(Mh, ml[u].x);
  Mh = wave_max(Mh);
  float lsum = 0.f;
  if (Mh == -INFINITY) Mh = 0.f;           // no finite chunk maximum: weights 2^-inf = 0
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int cc = lane + 64 * u;
    if (cc < C) {
      const float w = fast_exp2(ml[u].x - Mh);
      if (live && run == 0) red[a * C + cc] = w;
      lsum = fmaf(w, ml[u].y, lsum);
    }
  }
  lsum = wave_sum(lsum);
  if (live && run == 0 && lane == 0) s_L[a] = lsum;
  __syncthreads();
  AS_ATT_PHASE(p, 6);
  float2 O = make_float2(0.f, 0.f);
  for (int c0 = cb; c0 < ce; c0 += kB) {
    if (c0 != cb) load_batch(c0);
    // chunks past the run (re-read records) are selected away, not branched over
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const bool in = c0 + k < ce;
      const float w = red[a * C + min(c0 + k, C - 1)];
      const float x = fmaf(w, ob[k].x, O.x), y = fmaf(w, ob[k].y, O.y);
      O.x = in ? x : O.x;
      O.y = in ? y : O.y;
    }
  }
  // runs of one head added in run order (LDS past the weights)
  float2* s_run = reinterpret_cast<float2*>(red + ((GM * C + 1) & ~1));
  if constexpr (WPH > 1) {
    if (live && run > 0) s_run[((run - 1) * GM + a) * 64 + lane] = O;
    __syncthreads();
    if (run == 0) {
#pragma unroll
      for (int r = 1; r < WPH; ++r) {
        const float2 v = s_run[((r - 1) * GM + a) * 64 + lane];
        O.x += v.x;
        O.y += v.y;
      }
    }
  }
  if (live && run == 0) {
    const float L = s_L[a];
    float* dst = p.o + (long)(g * grp + a) * hd + 2 * lane;
    dst[0] = O.x / L;
    dst[1] = O.y / L;
  }
#ifdef AS_PHASE_TIMELINE
  if (p.phase_tl != nullptr && tid == 0) wait_vmem();
#endif
  AS_ATT_PHASE(p, 7);
}

template <int GM, int KS>
hipError_t launch_attention_g(const AttnParams& p, int chunks, hipStream_t s) {
  constexpr int NWV = kAttThreads / 64, WPH = NWV / GM;
  // wave partial outputs, or the merge's chunk weights and run sums
  const size_t chunk_f = size_t(NWV) * GM * kAttHd;
  const size_t merge_f = size_t(GM) * kMaxChunks + 2 + size_t(WPH - 1) * GM * 128;
  const size_t smem = (chunk_f > merge_f ? chunk_f : merge_f) * 4;
  auto k = attention_kernel<GM, KS>;
  if (smem > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       int(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(p.n_kv, chunks), dim3(kAttThreads), smem, s, p);
  return hipGetLastError();
}

template <int KS>
hipError_t launch_attention_ks(const AttnParams& p, int chunks, hipStream_t s) {
  const int grp = p.n_q / p.n_kv;
  if (grp <= 1) return launch_attention_g<1, KS>(p, chunks, s);
  if (grp <= 2) return launch_attention_g<2, KS>(p, chunks, s);
  if (grp <= 4) return launch_attention_g<4, KS>(p, chunks, s);
  return launch_attention_g<8, KS>(p, chunks, s);
}

hipError_t launch_attention(const AttnParams& p, int chunks, hipStream_t s) {
  if (chunks < 1 || chunks > kMaxChunks || p.n_q / p.n_kv > kMaxGroup) return hipErrorInvalidValue;
  const int longest = (p.n_ctx + chunks - 1) / chunks;     // cached keys of the longest chunk
  if (longest > kMaxKeys) return hipErrorInvalidValue;
  return longest <= 2 * kSlots ? launch_attention_ks<2>(p, chunks, s) : launch_attention_ks<4>(p, chunks, s);
}

int attention_max_group() { return kMaxGroup; }
int attention_head_dim() { return kAttHd; }
int attention_max_chunks() { return kMaxChunks; }
int attention_max_keys() { return kMaxKeys; }

}  // namespace as
