/*
 * actsparse.h -- C ABI of libactsparse: activation-sparse GEMV for LLM decode on
 * AMD Instinct MI355X (gfx950).
 *
 * The library implements training-free activation sparsity at decode time:
 * the input of a projection is thresholded by magnitude (|x| > t), or reduced
 * to a top-k neuron set, and only the weight rows of the surviving input
 * neurons are streamed from HBM into an fp32-accumulated GEMV.
 *
 * Sources of the operations (web pages; cited by title and section):
 *  - TEAL slides: "【DL輪読会】Training-Free Activation Sparsity in Large
 *    Language Models" -- magnitude thresholding of every projection input
 *    (method slide), thresholds from calibration data (method slide, setup
 *    slide), fused mask + sparse GEMV that loads only the needed weights
 *    (slide 11, Hardware-Aware Acceleration).
 *  - GLASS summary: "技術概要：GLASS – LLM の推論時スパース化のための
 *    グローバル・ローカル集約" -- rank aggregation of a local and a global
 *    importance signal and top-k selection of a static FFN mask (section 2.2).
 *  - Intra-expert summary: "Uncovering Intra-expert Activation Sparsity for
 *    Efficient Mixture-of-Expert Model Execution" -- dense gate scoring,
 *    masking, and gathered up/down projections inside routed experts, shared
 *    experts and router unchanged (method section, system implementation).
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless stated otherwise, 16-byte aligned.
 *    Tensors are row-major and contiguous.  The caller owns every buffer,
 *    including the workspace; the library allocates nothing, never copies
 *    between host and device and never synchronises: each call only enqueues
 *    kernels on `stream` (0 = the default stream).
 *  - Inputs are never written.  Outputs are fully overwritten unless
 *    AS_FLAG_ACCUMULATE is set (then Y += result).
 *  - Workspace: `ws` must hold at least the size returned by the matching
 *    *_ws_size query and must be zero-filled before its first use (any zero
 *    fill, or as_workspace_init).  Every call leaves the counters it uses at
 *    zero again, so a workspace is reusable by later calls on the same stream
 *    with the same shapes.  The carve-up follows the call's launch plan, which
 *    depends only on the shapes, the flags passed and the device's CU count
 *    (the library reads no environment variables).  Calls that may run
 *    concurrently need distinct workspaces.
 *  - Errors: arguments are validated on the host before anything is enqueued
 *    (AS_ERR_INVALID_ARG / AS_ERR_UNSUPPORTED / AS_ERR_WORKSPACE); a launch
 *    failure returns AS_ERR_HIP.  as_last_error() gives the message of the last
 *    failure on the calling thread.  Device faults surface at the caller's next
 *    synchronisation.  NaN, Inf, all-masked and k = n inputs are defined
 *    semantics, not errors.
 *  - Determinism: for fixed inputs, sizes and flags every output is bitwise
 *    reproducible (split-K partial sums are combined in a fixed order).
 *  - Accumulation is fp32; bf16 x bf16 and fp16 x fp16 products are exact in fp32.
 */
#ifndef ACTSPARSE_H
#define ACTSPARSE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AS_VERSION 202

typedef enum {
  AS_OK = 0,
  AS_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned pointer          */
  AS_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement         */
  AS_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the size query    */
  AS_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed          */
} as_status;

typedef enum { AS_F16 = 0, AS_BF16 = 1, AS_F32 = 2, AS_I8 = 3 } as_dtype;   /* AS_I8: as_threshold_gemv_i8 weights only */

enum {
  AS_FLAG_ACCUMULATE = 1u << 0,   /* Y += result instead of Y = result                   */
  AS_FLAG_ATOMIC_SPLITK = 1u << 1, /* row slices add into fp32 Y with atomics: no partial
                                      round trip or last-workgroup combine, not bitwise
                                      reproducible (see the GEMV and MLP calls)           */
  AS_FLAG_NO_NT_LOADS = 1u << 2,  /* plain (cached) weight loads instead of nontemporal  */
  AS_FLAG_FORCE_DENSE = 1u << 3,  /* ignore thresholds / neuron lists: dense baseline   */
  AS_FLAG_NO_FUSION = 1u << 4,    /* decoder block: RMS normalisations and residual adds as
                                     launches of their own (seven instead of five)       */
  AS_FLAG_AUTO = 1u << 5          /* as_sparse_swiglu_mlp, THRESHOLD: the batch-size switch
                                     (dense from AS_AUTO_DENSE_MIN_TOKENS tokens on)     */
};

/* Tokens from which AS_FLAG_AUTO runs the dense path (measured on MI355X: from
 * eight tokens on, the union of the tokens' threshold masks keeps nearly every
 * row and the sparse launches cost more than the dense ones). */
#define AS_AUTO_DENSE_MIN_TOKENS 8

/* Verification exports of a mask (every field may be NULL).
   bits: [M, ceil(n/64)] uint64, bit i%64 of word i/64 set when element i is kept.
   idx:  [M, n] int32, kept indices ascending; the first nnz[m] entries are valid.
   nnz:  [M] int32. */
typedef struct {
  uint64_t *bits;
  int32_t *idx;
  int32_t *nnz;
} as_mask_out;

/* ------------------------------------------------------------------ library */
int as_version(void);
const char *as_status_string(as_status s);
const char *as_last_error(void);
/* Zero-fill `bytes` of device memory at `ws` with a kernel (no memset node). */
as_status as_workspace_init(void *ws, size_t bytes, hipStream_t stream);

/* ------------------------------------------------------------ calibration
 * TEAL slides, method slide: the threshold t_p of a projection input is fixed
 * from calibration data for the target sparsity p.  Reading: t is the
 * nearest-rank order statistic of the pooled magnitudes:
 *   rank = ceil(p * n) with p = p_num / p_den exactly (integer arithmetic);
 *   *t_out = the rank-th smallest |pool[i]| (1-based), as fp32;
 *   p = 0 (p_num = 0) gives -INFINITY (sparsity 0 keeps every input).
 * NaN magnitudes order above +inf.
 * pool: [n] of dtype dt (f16/bf16/f32).  t_out: one device float.
 * ws: caller-owned device workspace of as_calibrate_threshold_ws_size(n) bytes
 * (zero-filled once; every call leaves it zeroed); calls sharing a workspace
 * must be ordered on one stream.
 * Errors: INVALID_ARG if pool/t_out is NULL, n < 1 or n >= 2^31, p_den < 1,
 * p_num < 0 or p_num > p_den; WORKSPACE if ws is NULL or too small. */
size_t as_calibrate_threshold_ws_size(int64_t n);
as_status as_calibrate_threshold(const void *pool, as_dtype dt, int64_t n, int64_t p_num, int64_t p_den,
                                 float *t_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ threshold GEMV
 * TEAL slides, slide 11: mask generation fused with the sparse product,
 * loading only the weight rows whose input survives:
 *   Y[m, :] = sum over i with |X[m, i]| > t of X[m, i] * W[i, :]
 * X: [M, K] (f16/bf16/f32), 1 <= M <= 16 (M > 8 runs on the matrix cores and
 * needs bf16 weights), 1 <= K <= 2^24.  W: [K, N] input-major (f16/bf16),
 * N % 8 == 0.  Y: [M, N] (f16/bf16/f32).  t is compared in fp32 with strict
 * '>': t = -INFINITY keeps every row; NaN inputs are dropped.  A weight row is
 * read once for all M tokens if any token keeps it; each token still uses only
 * its own kept inputs.
 * mask_out (nullable): the per-token input masks (bits and nnz for any M,
 * idx only for M == 1).
 * AS_FLAG_ATOMIC_SPLITK without AS_FLAG_ACCUMULATE clears Y before X is read, so
 * there X and Y must not overlap (INVALID_ARG otherwise).
 * AS_FLAG_FORCE_DENSE runs the dense baseline (every row, t ignored).
 * AS_FLAG_ATOMIC_SPLITK (Y fp32 only, else UNSUPPORTED): where the launch plan
 * splits the rows of a column tile over several workgroups, each adds its
 * partial tile into Y with fp32 atomic adds instead of the deterministic
 * store / count / last-workgroup sum (same terms, order of the additions
 * unspecified).  Without AS_FLAG_ACCUMULATE, Y is cleared by an extra fill
 * launch first.  Also taken by as_dense_gemv. */
size_t as_threshold_gemv_ws_size(int M, int K, int N);
as_status as_threshold_gemv(const void *X, as_dtype x_dt, int M, int K,
                            const void *W, as_dtype w_dt, int N, float t,
                            void *Y, as_dtype y_dt, unsigned flags, as_mask_out *mask_out,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* Sparse GEMV over int8 weight rows with a per-row scale (attribution notes,
 * discussion: activation sparsity combined with weight quantization such as W8A8
 * or INT4 compounds the byte savings):
 *   Y[0, :] = sum over i with |X[0, i]| > t of X[0, i] * row_scale[i] * W[i, :]
 * One token.  X: [K] (f16/bf16/f32, 16-byte aligned, K % 8 == 0); W: [K, N] int8
 * input-major (16-byte aligned, N % 8 == 0); row_scale: [K] fp32 (16-byte aligned);
 * Y: [N] (f16/bf16/f32).  The mask is on X, not on X * row_scale.  Each kept row
 * reads N bytes instead of 2N.  Flags as
 * for as_threshold_gemv (AS_FLAG_FORCE_DENSE: every row).  Errors: INVALID_ARG for
 * NULL or misaligned pointers or a bad N; UNSUPPORTED for an unaligned X or K % 8.
 * ws: as_threshold_gemv_i8_ws_size(K, N) bytes (zero-filled once, left zeroed). */
size_t as_threshold_gemv_i8_ws_size(int K, int N);
as_status as_threshold_gemv_i8(const void *X, as_dtype x_dt, int K, const int8_t *W, const float *row_scale,
                               int N, float t, void *Y, as_dtype y_dt, unsigned flags,
                               void *ws, size_t ws_bytes, hipStream_t stream);

/* Dense GEMV baseline Y = X W over every row (the speedup denominator): the
 * same kernel and launch shape as as_threshold_gemv without the mask. */
as_status as_dense_gemv(const void *X, as_dtype x_dt, int M, int K,
                        const void *W, as_dtype w_dt, int N,
                        void *Y, as_dtype y_dt, unsigned flags,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ sparse SwiGLU MLP */
typedef enum { AS_MLP_THRESHOLD = 0, AS_MLP_NEURON_SET = 1, AS_MLP_GATE_SCORE = 2 } as_mlp_mode;

typedef struct {
  const void *w_gate_up;  /* THRESHOLD: [d_model, 2, d_ff] input-major (row i = gate row i
                             then up row i).  NEURON_SET and GATE_SCORE: [d_ff, 3, d_model]
                             neuron-major (gate row, up row, down row of neuron j adjacent). */
  const void *w_down;     /* THRESHOLD: [d_ff, d_model] input-major.  Otherwise NULL. */
  as_dtype w_dt;          /* AS_F16 or AS_BF16 */
  int d_model;            /* multiple of 8, at most 2^24 */
  int d_ff;               /* multiple of 64, at most 2^24 */
} as_mlp_weights;

typedef struct {
  float *h;               /* THRESHOLD: [M, d_ff] fp32 intermediate silu(g)*u of every
                             neuron.  NEURON_SET: [M, n_active] for the listed neurons.
                             GATE_SCORE: [M, d_ff], 0 where the token drops the neuron. */
  as_mask_out x_mask;     /* input mask |X| > t_x (THRESHOLD only; see as_threshold_gemv) */
  as_mask_out h_mask;     /* THRESHOLD: |h| > t_h; GATE_SCORE: the keep mask |silu(g)| > t_h.
                             bits [M, ceil(d_ff/64)] and nnz [M]; idx must be NULL */
  hipEvent_t ev[3];       /* if non-NULL: recorded before stage 1, between the stages,
                             and after stage 2 (per-kernel timing) */
  float *a;               /* GATE_SCORE only: [M, d_ff] fp32 gate activation silu(g) of
                             every neuron (the score the keep mask thresholds) */
} as_mlp_debug;

/* THRESHOLD (TEAL slides, method slide; every projection input thresholded):
 *   x~ = X * [|X| > t_x];  g = x~ Wg;  u = x~ Wu;  h = silu(g) * u  (fp32)
 *   Y = (h * [|h| > t_h]) Wd
 * NEURON_SET (GLASS summary, section 2.2: a static top-k neuron mask applied
 * through decode): the same SwiGLU restricted to neurons
 * neuron_idx[0 .. n_active) (int32, device, ascending, distinct, < d_ff);
 * t_x and t_h are ignored.
 * GATE_SCORE (Intra-expert summary, system implementation: dense gate projection,
 * one threshold pass over the scores, up and down over the active neurons only;
 * TEAL slides, slides 5-6: the CATS score |SiLU(x W_gate)|):
 *   g = X Wg (every neuron);  a = silu(g);  token m keeps neuron j iff |a[m,j]| > t_h
 *   h[m,j] = a[m,j] * (X[m] . Wu[j]) where kept, else 0;  Y = h Wd
 * The up and down rows of a neuron are read once if any token keeps it.  t_x
 * must be -INFINITY (X is not thresholded; UNSUPPORTED otherwise); M <= 8;
 * d_model <= 8192; neuron_idx is ignored.  AS_FLAG_FORCE_DENSE keeps every neuron.
 * X: [M, d_model] (f16/bf16/f32), 1 <= M <= 16 (M > 8: THRESHOLD mode with bf16
 * weights, on the matrix cores); THRESHOLD mode without debug exports also takes
 * 16 < M <= 256, run as consecutive groups of 16 tokens on `stream` (the full
 * groups and a partial last group each use a region of the workspace of their
 * own, as as_sparse_swiglu_mlp_ws_size(M) sizes it).  Y: [M, d_model].
 * AS_FLAG_AUTO (THRESHOLD; Intra-expert summary, system implementation: the sparse
 * path for low latency, the dense one for throughput, switched by batch size):
 * the call runs as AS_FLAG_FORCE_DENSE when M >= AS_AUTO_DENSE_MIN_TOKENS.
 * silu(z) = z / (1 + exp(-z)).  AS_FLAG_FORCE_DENSE: dense SwiGLU over all
 * neurons and inputs (the baseline).  AS_FLAG_ATOMIC_SPLITK (fp32 Y only): the
 * down projection's row slices add into Y with fp32 atomic adds (as in
 * as_threshold_gemv); without AS_FLAG_ACCUMULATE, Y is cleared by the first
 * launch, so Y must not overlap X (INVALID_ARG otherwise).  dbg is nullable;
 * the masks it exports are those of the masked tensors as the kernels computed
 * them (h in fp32). */
size_t as_sparse_swiglu_mlp_ws_size(int M, const as_mlp_weights *w, as_mlp_mode mode);
as_status as_sparse_swiglu_mlp(const void *X, as_dtype x_dt, int M, const as_mlp_weights *w,
                               as_mlp_mode mode, float t_x, float t_h,
                               const int32_t *neuron_idx, int n_active,
                               void *Y, as_dtype y_dt, unsigned flags, as_mlp_debug *dbg,
                               void *ws, size_t ws_bytes, hipStream_t stream);

/* Compact packing of a static neuron set (GLASS summary, section 2.2 and its
 * edge-deployment discussion: a static mask keeps one compact subset of the
 * weights resident for the whole decode).  From THRESHOLD-layout weights w (gate/up
 * [d_model, 2, d_ff], down [d_ff, d_model]) and the kept neurons idx[0..k) (device
 * int32, each < d_ff), writes gate_up_out [d_model, 2, k] (columns idx of every
 * input row) and down_out [k, d_model] (rows idx), in w->w_dt.  The packed pair is
 * an ordinary THRESHOLD-layout MLP with d_ff = k: as_sparse_swiglu_mlp on it with
 * AS_FLAG_FORCE_DENSE (or t_x = t_h = -INFINITY) is the static-set SwiGLU of a
 * whole batch, each packed row read once per 16 tokens.  k must be a multiple of 64
 * (the MLP's d_ff rule) and at most d_ff; both outputs 16-byte aligned.
 * Errors: INVALID_ARG for NULL pointers, a bad k or misaligned outputs. */
as_status as_pack_neuron_set(const as_mlp_weights *w, const int32_t *idx, int k,
                             void *gate_up_out, void *down_out, hipStream_t stream);

/* Allocation-free as_sparse_swiglu_mlp, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The workspace is a static device array of 16 MiB (enough for up to 8
 * tokens at d_model 4096, d_ff 14336) that every GPU the library runs on holds until
 * the process ends; the call allocates nothing.  Arguments, results and errors are
 * those of as_sparse_swiglu_mlp, which it runs on that memory (the same kernels and
 * bits); UNSUPPORTED when the call needs a larger workspace than the array (see
 * as_sparse_swiglu_mlp_ws_size).  The bytes a call uses are cleared (one fill kernel
 * on `stream`) on a device's first call and whenever the shapes change.  Every call
 * on a GPU shares that GPU's array: calls that overlap on one GPU (from several
 * streams or threads) race. */
as_status as_sparse_swiglu_mlp_noalloc(const void *X, as_dtype x_dt, int M, const as_mlp_weights *w,
                                       as_mlp_mode mode, float t_x, float t_h,
                                       const int32_t *neuron_idx, int n_active,
                                       void *Y, as_dtype y_dt, unsigned flags, as_mlp_debug *dbg,
                                       hipStream_t stream);

/* ------------------------------------------------------------ top-k neuron masks */
typedef enum { AS_TOPK_VALUE = 0, AS_TOPK_RANK_BLEND = 1 } as_topk_mode;

/* Exact top-k per row, ties broken by index (the smaller index wins).
 * VALUE (intra-expert summary, method section: the lowest-scoring neurons are
 * skipped; GLASS summary, section 2.2: the top-k neurons form the mask): the k
 * largest score[r, :], comparing -0.0 == +0.0, NaN below every number.
 * RANK_BLEND (GLASS summary, section 2.2: GLASS_j = (1 - lambda) R^(l)_j +
 * lambda R^(g)_j): ordinal ranks R^(l) of score[r, :] and R^(g) of prior[r, :]
 * (largest value -> n; equal values: the smaller index ranks higher), blended in
 * 16-bit fixed point, S_j = (65536 - lq) R^(l)_j + lq R^(g)_j with
 * lq = floor(lambda * 65536 + 0.5), then the k largest S.
 * score, prior: [rows, n] fp32 (prior only for RANK_BLEND, else may be NULL).
 * Outputs (either may be NULL, not both): mask [rows, ceil(n/64)] uint64 (bit
 * i%64 of word i/64 = kept), idx [rows, k] int32 ascending.
 * Errors: INVALID_ARG for k < 0, k > n, n < 1, rows < 1, lambda outside [0, 1];
 * UNSUPPORTED for RANK_BLEND with n > 65535.  VALUE needs no workspace. */
size_t as_topk_mask_ws_size(int rows, int n, as_topk_mode mode);
as_status as_topk_mask(const float *score, const float *prior, int rows, int n, int k,
                       as_topk_mode mode, float lambda, uint64_t *mask, int32_t *idx,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* GLASS local signal (GLASS summary, sections 1 and 2.2: the local importance
 * of a neuron comes from the prompt's prefill activations).  Reading:
 *   local[j] = (1/P) sum_t |silu(X[t] . Wg_j) * (X[t] . Wu_j)|,
 * the mean magnitude of the down-projection input over the P prompt tokens,
 * computed on the matrix cores (fp32 accumulation).  It is the score argument
 * of as_topk_mask in RANK_BLEND mode.
 * X: [P, d_model] bf16; w: NEURON_SET layout [d_ff, 3, d_model] bf16
 * (w->w_down unused); local: [d_ff] fp32.
 * Errors: UNSUPPORTED unless X and the weights are bf16 and d_model % 32 == 0. */
as_status as_glass_local_signal(const void *X, as_dtype x_dt, int P, const as_mlp_weights *w,
                                float *local, hipStream_t stream);

/* ------------------------------------------------------------ MoE: router and routed experts */
typedef struct {
  const void *w_gate_up;  /* [E, d_ff_e, 2, d_model] neuron-major: gate row then up row of
                             every neuron of every expert, contiguous */
  const void *w_down;     /* [E, d_ff_e, d_model]: row n = neuron n's output weights */
  as_dtype w_dt;          /* AS_F16 or AS_BF16 */
  int n_experts;          /* E, 1..1024 */
  int d_model;            /* multiple of 8 */
  int d_ff_e;             /* neurons per expert, at most 8192 */
} as_moe_weights;

/* Router (intra-expert summary, method section: routed experts are chosen by the
 * router, whose logic is unchanged).  Reading: per token t, the top_k experts
 * with the largest logits[t, :] (ties to the smaller index), in descending
 * logit order, weights = softmax over the selected logits.
 * logits: [T, E] fp32.  ids: [T, top_k] int32.  weights: [T, top_k] fp32.
 * Errors: INVALID_ARG for T < 1, E < 1 or > 1024, top_k < 1 or > min(E, 64). */
as_status as_moe_router(const float *logits, int T, int E, int top_k,
                        int32_t *ids, float *weights, hipStream_t stream);

/* Router logits and routing in one launch: logits = X W_router (dense GEMV,
 * fp32 accumulation), then exactly what as_moe_router does with them.  The
 * logits are the same bits as as_dense_gemv's for E <= 128.
 * X: [T, d_model] (f16/bf16/f32); w_router: [d_model, E] (f16/bf16, 16-byte
 * aligned); logits: [T, E] fp32 (output); ids [T, top_k] int32 and weights
 * [T, top_k] fp32 as for as_moe_router.  ws: as_moe_router_gemv_ws_size(T,
 * d_model, E) bytes, zero-filled once, left zeroed.
 * Errors: INVALID_ARG for NULL pointers, E not a multiple of 8, top_k outside
 * 1..min(E, 64); UNSUPPORTED for T > 8 or E > 512 (use as_dense_gemv and
 * as_moe_router); WORKSPACE if ws is too small. */
size_t as_moe_router_gemv_ws_size(int T, int d_model, int E);
as_status as_moe_router_gemv(const void *X, as_dtype x_dt, int T, const void *w_router, as_dtype w_dt,
                             int d_model, int E, int top_k, float *logits, int32_t *ids, float *weights,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* Routed experts with intra-expert activation sparsity (intra-expert summary,
 * system implementation: dense gate scoring, low-scoring neurons masked, only
 * the active neurons' weights gathered):
 *   Y[t, :] (+)= sum_j expert_w[t, j] * y_{t,j},
 *   y_{t,j} = sum over n in keep(t, j) of h_n * Wd_e[n, :],   e = expert_ids[t, j],
 *   h = silu(x_t Wg_e^T) * (x_t Wu_e^T) over all d_ff_e neurons (fp32),
 *   keep(t, j) = the keep_k neurons with the largest |h_n| (ties to the smaller n).
 * X: [T, d_model] (f16/bf16/f32); expert_ids [T, top_k] int32 (ids outside
 * [0, E) contribute nothing); expert_w [T, top_k] fp32; Y [T, d_model].
 * Gate/up weights of an expert are read once per call for all tokens routed to
 * it.  Shared experts are not part of this call (run them densely and combine
 * with AS_FLAG_ACCUMULATE).  AS_FLAG_FORCE_DENSE keeps every neuron.
 * AS_FLAG_ATOMIC_SPLITK (fp32 Y only, else UNSUPPORTED): each (token, slot)
 * adds its weighted rows' sum into Y with fp32 atomic adds instead of the
 * slot-order sum by the last slot to finish (order of the additions
 * unspecified); without AS_FLAG_ACCUMULATE, Y is cleared by a fill launch
 * first (which does not wait for y_ready), so Y must not overlap X
 * (INVALID_ARG otherwise).
 * Debug exports (nullable): h_dbg [T, top_k, d_ff_e] fp32, keep_dbg
 * [T, top_k, keep_k] int32 ascending.
 * y_ready (nullable): an event recorded after whatever produces Y on another
 * stream (e.g. the shared expert, for AS_FLAG_ACCUMULATE); the stream waits for
 * it only before the down stage, the only one that touches Y, so the grouping
 * and the gate/up stage overlap that producer.
 * Errors: INVALID_ARG for T < 1, top_k < 1 or > 32, T * top_k > 256,
 * keep_k < 0 or > d_ff_e. */
size_t as_sparse_moe_expert_ws_size(int T, int top_k, const as_moe_weights *w);
as_status as_sparse_moe_expert(const void *X, as_dtype x_dt, int T,
                               const int32_t *expert_ids, const float *expert_w, int top_k,
                               const as_moe_weights *w, int keep_k,
                               void *Y, as_dtype y_dt, unsigned flags,
                               float *h_dbg, int32_t *keep_dbg, hipEvent_t y_ready,
                               void *ws, size_t ws_bytes, hipStream_t stream);

/* Routed experts with the gate-score keep rule (TEAL slides, slides 5-6, CATS;
 * intra-expert summary, system implementation: the gate projection runs densely
 * to score the neurons, one threshold pass masks them, only the active neurons'
 * weights are read for the rest):
 *   a = silu(x_t Wg_e^T) over all d_ff_e neurons (fp32),
 *   keep(t, j) = { n : |a_n| > t_gate } (strict),
 *   h_n = a_n * (x_t . Wu_e[n]) for kept n (the up row read only where some token
 *   routed to the expert keeps n), h_n = 0 otherwise,
 *   Y[t, :] (+)= sum_j expert_w[t, j] * sum over n with h_n != 0 of h_n Wd_e[n, :].
 * Arguments, layouts, workspace (as_sparse_moe_expert_ws_size), y_ready and the
 * flags AS_FLAG_ACCUMULATE / AS_FLAG_ATOMIC_SPLITK / AS_FLAG_FORCE_DENSE (t_gate
 * taken as -inf) as for as_sparse_moe_expert.  Debug exports (nullable): h_dbg
 * [T, top_k, d_ff_e] (exactly 0 where dropped) and a_dbg [T, top_k, d_ff_e] fp32.
 * Errors: those of as_sparse_moe_expert; INVALID_ARG for a NaN t_gate. */
as_status as_sparse_moe_expert_gate(const void *X, as_dtype x_dt, int T,
                                    const int32_t *expert_ids, const float *expert_w, int top_k,
                                    const as_moe_weights *w, float t_gate,
                                    void *Y, as_dtype y_dt, unsigned flags,
                                    float *h_dbg, float *a_dbg, hipEvent_t y_ready,
                                    void *ws, size_t ws_bytes, hipStream_t stream);

/* One MoE layer for up to 8 tokens on `stream` alone, in three launches
 * (intra-expert summary, system implementation: the router and the shared expert
 * are unchanged; the routed experts score their neurons densely and read only the
 * kept neurons' down rows):
 *   logits = X Wr;  (ids, weights) = the routing of as_moe_router;
 *   Y = dense shared-expert SwiGLU MLP of X
 *       + sum_j weights[t, j] * expert_{ids[t, j]}(X[t]) with the exact top keep_k
 *         neurons of each (token, slot), as in as_sparse_moe_expert.
 * Launch 1 runs the router logits GEMV (its last workgroup routes every token)
 * beside the shared expert's gate/up; launch 2 the routed experts' gate/up beside
 * the shared expert's down projection (which writes Y); launch 3 the routed down
 * stage, added onto Y.  No piece waits on another stream.  logits, ids, weights,
 * h and the keep sets are the bits of as_moe_router_gemv and as_sparse_moe_expert;
 * Y is the composition with as_sparse_swiglu_mlp (AS_FLAG_FORCE_DENSE, gate/up
 * partials summed in the down stage) up to the split of the shared expert's down
 * stage, which here takes one row range per CU and column tile (another fp32
 * summation order of the same terms).
 * X: [T, d_model] (f16/bf16/f32).  Y: [T, d_model] fp32.  logits: [T, E] fp32,
 * ids: [T, top_k] int32, weights: [T, top_k] fp32 (outputs, device).
 * h_dbg [T * top_k, d_ff_e] and keep_dbg [T * top_k, keep_k]: optional, as in
 * as_sparse_moe_expert.  flags: AS_FLAG_FORCE_DENSE (every routed neuron kept),
 * AS_FLAG_ATOMIC_SPLITK (the routed down stage adds into Y atomically, as in
 * as_sparse_moe_expert); any other flag is AS_ERR_UNSUPPORTED.
 * Weights: bf16 throughout; w_router [d_model, E] input-major, 16-byte aligned;
 * the shared expert in THRESHOLD layout with the experts' d_model.
 * Limits: 1 <= T <= 8, E % 8 == 0, 8 <= E <= 512, 1 <= top_k <= min(32, E),
 * T * top_k <= 256, d_ff_e <= 8192.  as_moe_layer_ws_size returns 0 where the
 * shapes are outside these limits (then use the separate entry points);
 * as_moe_layer returns AS_ERR_UNSUPPORTED there. */
typedef struct {
  const void *w_router;   /* [d_model, E] input-major */
  as_moe_weights experts; /* routed experts */
  as_mlp_weights shared;  /* shared expert, THRESHOLD layout, used densely */
} as_moe_layer_weights;

size_t as_moe_layer_ws_size(int T, int top_k, const as_moe_layer_weights *w);
as_status as_moe_layer(const void *X, as_dtype x_dt, int T, const as_moe_layer_weights *w,
                       int top_k, int keep_k, float *Y, unsigned flags,
                       float *logits, int32_t *ids, float *weights,
                       float *h_dbg, int32_t *keep_dbg,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* as_moe_layer with the routed experts under the gate-score keep rule of
 * as_sparse_moe_expert_gate (threshold t_gate on |silu(g)|; the shared expert
 * stays dense).  Same launches, workspace (as_moe_layer_ws_size), limits and
 * flags; h_dbg and a_dbg [T * top_k, d_ff_e] as in as_sparse_moe_expert_gate.
 * Errors: those of as_moe_layer; INVALID_ARG for a NaN t_gate. */
as_status as_moe_layer_gate(const void *X, as_dtype x_dt, int T, const as_moe_layer_weights *w,
                            int top_k, float t_gate, float *Y, unsigned flags,
                            float *logits, int32_t *ids, float *weights,
                            float *h_dbg, float *a_dbg,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ attribution-based selection
 * Attribution notes (Attribution-based Sparse Activation in LLMs): neurons are
 * ranked by an attribution score rather than by their output magnitude, and each
 * layer keeps a fixed fraction of its neurons (Approach 1); in attention the
 * neuron is a head.  The scores come from outside the decode path (a backward pass
 * on representative data, or a predictor trained on it); the calls below turn them
 * into kept sets and use those sets. */

/* Corrected GxO score (attribution notes, correction term), per row (layer):
 *   score[r, i] = grad[r, i] * x[r, i] + 0.5 * |x[r, i]| * sqrt(sum_k grad[r, k]^2)
 * x, grad, score: device [rows, n] fp32.  The squared-gradient sum is formed in a
 * fixed order (the same bits on every call).  Errors: INVALID_ARG for NULL
 * pointers, rows < 1 or n < 1. */
as_status as_corrected_gxo(const float *x, const float *grad, int rows, int n, float *score,
                           hipStream_t stream);

/* Number of neurons a layer of n keeps at activation ratio ar_num / ar_den:
 * ceil(ar_num * n / ar_den), computed exactly; -1 for n < 0, ar_den <= 0 or a
 * ratio outside [0, 1]. */
int as_top_fraction_count(int n, int ar_num, int ar_den);

/* Approach 1: per row (layer), the k = as_top_fraction_count(n, ar_num, ar_den)
 * neurons with the largest score[r, :] (by value: a negative attribution ranks
 * lowest; ties to the smaller index; NaN ranks below every number), as a bitmask
 * [rows, ceil(n/64)] and/or ascending indices [rows, k] (either output nullable).
 * The kept indices feed AS_MLP_NEURON_SET (MLP neurons) or as_head_masked_gemv
 * (attention heads).  Errors: INVALID_ARG for NULL score or both outputs NULL,
 * rows < 1, n < 1, a ratio outside [0, 1]. */
as_status as_select_top_fraction(const float *score, int rows, int n, int ar_num, int ar_den,
                                 uint64_t *mask, int32_t *idx, hipStream_t stream);

/* Output projection over the kept heads only (attribution notes: a deactivated
 * head's weights are zeroed; here its head_dim-row block of W is not read):
 *   Y[0, :] = sum over listed heads h of X[h*hd .. h*hd+hd) W[h*hd .. h*hd+hd, :]
 * One token.  X: [n_heads * head_dim] (f16/bf16/f32); heads: device int32 [n_keep]
 * (indices outside [0, n_heads) are ignored, repeats count once); W: [n_heads *
 * head_dim, N] input-major (f16/bf16, 16-byte aligned, N % 8 == 0); Y: [N].  One
 * launch: each workgroup marks the listed heads in LDS, lists them in ascending
 * order and gathers an equal share of their rows (every input of a kept head
 * counts, zeros and NaN included).
 * ws: as_head_masked_gemv_ws_size bytes, zero-filled once.  flags:
 * AS_FLAG_ATOMIC_SPLITK, AS_FLAG_NO_NT_LOADS (others UNSUPPORTED).
 * Errors: INVALID_ARG for NULL pointers, n_heads outside 1..1024, n_keep outside
 * 0..n_heads, bad dtypes or N; UNSUPPORTED for an X not 16-byte aligned or
 * n_heads * head_dim not a multiple of 8. */
size_t as_head_masked_gemv_ws_size(int n_heads, int head_dim, int N);
as_status as_head_masked_gemv(const void *X, as_dtype x_dt, int n_heads, int head_dim,
                              const int32_t *heads, int n_keep, const void *W, as_dtype w_dt, int N,
                              void *Y, as_dtype y_dt, unsigned flags, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------ offline sparsity allocation
 * Block-wise greedy sparsity allocation (TEAL slides, slide 10): under a
 * model-wide sparsity target, every block starts at sparsity 0 and, one step at
 * a time, the block whose error would grow least is raised one level, until the
 * target is met.  Host-side (it runs once, offline; inference then uses the
 * fixed per-block levels).
 *   err      host, [n_blocks][n_levels] doubles: block b's l2 activation error at
 *            sparsity l * step (measured beforehand, e.g. with the sparse and dense
 *            paths of this library on calibration inputs)
 *   weights  host, [n_blocks] doubles > 0: each block's share of the model-wide
 *            sparsity (e.g. its count of thresholded inputs); the overall sparsity
 *            is the weighted mean of step * level
 *   step     > 0: sparsity per level; target in [0, 1]
 *   levels   host, [n_blocks] int32 output
 * A step raises the block with the least error increase err[b][l+1] - err[b][l]
 * (ties to the smaller index; blocks at level n_levels - 1 are not raised); the
 * loop stops at the first step whose overall sparsity reaches target (relative
 * slack 1e-12) or when no block can be raised.
 * Errors: INVALID_ARG for NULL pointers, n_blocks < 1, n_levels < 1, a weight
 * <= 0 or not finite, step <= 0, target outside [0, 1], a non-finite error. */
as_status as_greedy_sparsity(const double *err, int n_blocks, int n_levels, const double *weights,
                             double step, double target, int32_t *levels);

/* ------------------------------------------------------------ decoder-block glue
 * TEAL slides, method slide: every projection input of the attention and MLP
 * blocks is thresholded; the attention core stays dense.  Readings (the pages
 * give no block): pre-norm RMSNorm with unit gain, no rotary embedding, query
 * head h reads key/value head h / (n_q / n_kv), keys = cached context + the
 * current token. */

/* Y[r, :] = X[r, :] / sqrt(mean(X[r, :]^2) + eps) in fp32; copy[r, :] = X[r, :]
 * as fp32 when copy is non-NULL (the residual branch).  X: [rows, d]. */
as_status as_rmsnorm(const void *X, as_dtype x_dt, int rows, int d, float eps,
                     float *Y, float *copy, hipStream_t stream);

/* Dense softmax attention of one decode token, scale 1/sqrt(head_dim):
 * o[h, :] = sum_j softmax_j(q[h] . K_j / sqrt(hd)) V_j over the n_ctx cached keys
 * of kv head h / (n_q / n_kv) followed by the current token's k_new / v_new.
 * q: [n_q, hd] fp32; k_new, v_new: [n_kv, hd] fp32; caches: [n_ctx, n_kv, hd]
 * (AS_BF16 only); o: [n_q, hd] fp32.  n_q % n_kv == 0, n_q / n_kv <= 8,
 * head_dim == 128, 0 <= n_ctx <= 32767 (UNSUPPORTED above).  q, k_new, v_new
 * and the caches 16-byte aligned (INVALID_ARG otherwise).  The cached keys of a
 * kv head are split into up to 256 chunks reduced side by side and merged in
 * chunk order by the last one to finish (bitwise reproducible); the workspace
 * holds the chunk records and one counter per kv head, zero between calls. */
size_t as_gqa_decode_attention_ws_size(int n_ctx, int n_q, int n_kv, int head_dim);
as_status as_gqa_decode_attention(const float *q, const float *k_new, const float *v_new,
                                  const void *k_cache, const void *v_cache, as_dtype kv_dt,
                                  int n_ctx, int n_q, int n_kv, int head_dim, float *o,
                                  void *ws, size_t ws_bytes, hipStream_t stream);

typedef struct {
  const void *w_qkv;      /* [d_model, (n_q + 2 n_kv) * head_dim] input-major, columns q | k | v */
  const void *w_o;        /* [n_q * head_dim, d_model] input-major */
  as_mlp_weights mlp;     /* THRESHOLD layout (gate/up [d_model, 2, d_ff], down [d_ff, d_model]) */
  int n_q, n_kv, head_dim;
} as_block_weights;

typedef struct { float qkv, o, gate_up, down; } as_block_thresholds;

typedef struct {          /* every field nullable; fp32 intermediates of one call */
  float *xn;              /* [d_model] rmsnorm(x) */
  float *qkv;             /* [(n_q + 2 n_kv) * head_dim] */
  float *o;               /* [n_q * head_dim] attention output (o-proj input) */
  float *h1;              /* [d_model] x + o-proj */
  float *xn2;             /* [d_model] rmsnorm(h1) */
  float *h;               /* [d_ff] MLP intermediate */
  /* masks of the four thresholded inputs, as the kernels applied them (see
     as_mask_out; M = 1): |xn| > t.qkv, |o| > t.o, |xn2| > t.gate_up (bits, idx,
     nnz), |h| > t.down (bits and nnz; idx must be NULL) */
  as_mask_out qkv_in, o_in, gate_up_in, down_in;
} as_block_debug;

/* One decoder block for one decode token, every projection input thresholded:
 *   xn = rmsnorm(x); qkv = (xn * [|xn| > t.qkv]) Wqkv; o = attention(q, caches + k, v)
 *   h1 = x + (o * [|o| > t.o]) Wo;  Y = h1 + MLP(rmsnorm(h1)) with t.gate_up, t.down.
 * X: [d_model] (f16/bf16/f32); Y: [d_model] fp32.  AS_FLAG_FORCE_DENSE ignores
 * every threshold (the dense block).  By default the two normalisations run in
 * the prologues of the projections that read them and the residual adds in the
 * epilogues of the projections that produce them (five launches);
 * AS_FLAG_NO_FUSION runs them as launches of their own (seven). */
size_t as_decoder_block_ws_size(const as_block_weights *w, int n_ctx);
as_status as_decoder_block(const void *X, as_dtype x_dt, const as_block_weights *w,
                           const void *k_cache, const void *v_cache, int n_ctx,
                           const as_block_thresholds *t, float *Y, unsigned flags,
                           as_block_debug *dbg, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ benchmark support
 * Overwrite `bytes` of device memory at `buf` with a kernel, evicting the
 * Infinity Cache and L2 between timed calls. */
as_status as_bench_flush(void *buf, size_t bytes, hipStream_t stream);

/* Read `bytes` of device memory at `buf` with 16-byte nontemporal loads, eight in
 * flight per thread over a grid of eight workgroups per CU: a probe of the
 * achievable streaming-read bandwidth, against which the kernels' rates are also
 * reported.  buf 16-byte aligned, bytes a multiple of 16; *sink (one device
 * unsigned) is written only in the unlikely case that the loaded data fold to one
 * particular value.  Errors: INVALID_ARG for NULL pointers or misalignment. */
as_status as_bench_read(const void *buf, size_t bytes, unsigned *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ACTSPARSE_H */
