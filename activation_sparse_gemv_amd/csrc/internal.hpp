// Internal launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/actsparse.h"

namespace as {

// Arrival counters (split-K tiles, MoE down tiles, attention kv heads) sit
// kCounterStride uints apart, one 256-byte line each: counters that share a line
// have every workgroup's atomic queue on that one line.
constexpr int kCounterStride = 64;

enum { IN_THRESH = 0, IN_LISTS = 1, IN_ALL = 2, IN_RANGE = 4, IN_PARTS = 5 };
enum { OUT_Y = 0, OUT_SWIGLU = 1, OUT_PARTS = 2, OUT_ROUTER = 3 };

// One row-gather GEMV launch: Y[m, c] = sum over listed rows i of xv[m, i] * W[i, c].
// The rows come from a magnitude mask of a vector (IN_THRESH: the whole vector,
// split evenly over the slices; IN_RANGE: each slice masks its own range), from
// per-tile compacted lists written by an earlier stage (IN_LISTS) or
// are all rows (IN_ALL); or the input is h = silu(g) * u of an earlier paired
// gate/up launch that left its split-K partials unsummed (IN_PARTS: each slice
// sums the partials of its own range of h in slice order, applies SwiGLU and the
// mask |h| > t).
// The grid is n_tiles column tiles x S slices of the row list (split-K); the
// last workgroup of a tile sums the S partials in slice order and runs the
// epilogue (OUT_Y: store y; OUT_SWIGLU: h = silu(g) * u, |h| > t_h, per-tile list;
// OUT_ROUTER: store the logits and route every token from them),
// or every workgroup stores its partial and stops (OUT_PARTS: the next launch
// sums them).
struct GemvParams {
  // input vector (IN_THRESH, IN_RANGE, IN_ALL): x[m * ldx + i], i < K
  const void* x; int x_dt; int M; int K; long ldx; float t;
  // input lists (IN_LISTS): tile q holds list_cnt[q] entries at (q * lt_stride + e)
  const int* list_cnt; const int* list_idx; const float* list_val; int n_lt; int lt_stride;
  // weights: row i, column c at W[i * ldw + c]; GU: gate column n, up column gu_off + n
  const uint16_t* W; long ldw; int N; long gu_off;
  // split
  int n_tiles; int S; int cap;
  float* partials; unsigned* counters; long part_ld;
  // OUT_Y
  void* y; int y_dt; long ldy; int accumulate;
  // OUT_Y with split rows: each slice adds its partial tile into y (fp32) with
  // atomic adds (slice 0 also adds res) instead of the last-workgroup combine
  int atomic_y;
  // OUT_Y / OUT_SWIGLU with split rows: the slices store their partial tiles and
  // end; the next launch on the stream (sum_slices_kernel, sum_swiglu_kernel) sums
  // them in slice order
  int defer_sum;
  // OUT_PARTS / OUT_SWIGLU: when set, one workgroup (column tile 0) clears zero_n
  // floats at zero_y (the y that the next launch adds into)
  float* zero_y; long zero_n;
  // OUT_SWIGLU
  float t_h; float* h; long ldh; int* o_cnt; int* o_idx; float* o_val; uint64_t* h_bits; long h_bits_ld;
  int* h_nnz;              // per-token count of the h mask (IN_PARTS, OUT_SWIGLU; cleared by the host)
  // input-mask verification exports (IN_THRESH)
  uint64_t* x_bits; long x_bits_ld; int* x_idx; int* x_nnz;
  // IN_PARTS: x = gate/up partials [x_parts][M][ldx] fp32 (gate column i at i, up at
  // x_up + i); the range's h goes to h[m * ldh + i] and its mask to h_bits when set
  // (written by the workgroups of column tile 0 only)
  int x_parts; long x_up;
  int keep_all;            // IN_PARTS: keep every row (dense baseline), no mask
  // RMS normalisation of the input in the threshold prologue (IN_THRESH, one token,
  // 16-byte chunks): x is scaled by 1 / sqrt(sum x^2 / K + norm_eps) before the mask
  // and the products; xn_out (nullable) receives the normalised vector
  int norm_x; float norm_eps; float* xn_out;
  // OUT_Y: a residual added after the split-K sum, res[m * ldres + c] (nullable)
  const void* res; int res_dt; long ldres;
  // OUT_ROUTER (one column tile holding all N logits): y = logits, then per token
  // the top route_top experts and their softmax weights
  int route_top; int* route_ids; float* route_wts;
  // phase timeline (libactsparse_timeline.so only): 16 words per workgroup
  unsigned long long* phase_tl;
  // int8 weights (DT_I8): row i is W[i, :] * row_scale[i] (fp32, K entries)
  const float* row_scale;
  // head mask (IN_RANGE / IN_THRESH, one token; on when head_dim > 0): only rows of
  // the listed heads (row i belongs to head i / head_dim) are kept, besides the
  // threshold
  const int* heads; int n_heads_keep; int head_dim; int n_heads;
};

struct GemvConfig {
  int wdt;   // DT_F16 / DT_BF16
  int mt;    // template token count (1, 2, 4, 8) >= M
  int lpr;   // lanes per row segment (16, 32, 64): tile width lpr * 8 columns
  int in;    // IN_*
  int out;   // OUT_*
  bool gu;   // paired gate/up columns
  bool nt;   // nontemporal weight loads
  int nv = -1;  // threshold prologue chunk (16-byte vectors per thread); -1 = choose, 0 = general
};

size_t gemv_smem_bytes(const GemvConfig& c, int cap, int n_lt);
// Compute units of the current device (read once per process).
int device_cus();

hipError_t launch_gather_gemv(const GemvConfig& c, const GemvParams& p, hipStream_t s);
// int8 weights with a per-row scale: one token, IN_THRESH (16-byte aligned x) or
// IN_ALL, OUT_Y.
hipError_t launch_gemv_i8_m1(const GemvConfig& c, const GemvParams& p, size_t smem, hipStream_t s);
int pick_chunk_vectors(const void* x, int x_dt, int K, long ldx);

// Neuron-major gate/up dot products for a neuron list (static neuron set).
struct NeuronGuParams {
  const void* x; int x_dt; int M; long ldx; int d_model;
  const uint16_t* W; long ld_neuron; long up_off;   // gate row of neuron j at W + j*ld_neuron, up at + up_off
  const int* idx; int n_active;                       // idx == nullptr: neuron p is p
  float* h_dbg; long ld_hdbg;                         // optional [M, n_active]
  int* o_cnt; int* o_idx; float* o_val;               // single-tile list for the down stage
  int neurons_per_wave;
};
hipError_t launch_neuron_gu(int wdt, int mt, bool nt, const NeuronGuParams& p, hipStream_t s);

// Gate-score neuron selection (dense gate, |silu(g)| > t, up over the kept):
// workgroup b scores neurons [b * npb, (b + 1) * npb) and writes h[m * ldh + j]
// for each of them (0 where token m drops neuron j).
constexpr int kGsMaxNpb = 64;
struct GateScoreParams {
  const void* x; int x_dt; int M; long ldx; int d_model; int d_ff;
  const uint16_t* W; long ld_neuron; long up_off;    // gate row of neuron j at W + j*ld_neuron, up at + up_off
  float t; int keep_all;
  int npb;                                            // neurons per workgroup, divides 64
  float* h; long ldh;                                 // [M, d_ff] output
  float* a_dbg;                                       // optional [M, d_ff] silu(g) (stride ldh)
  uint64_t* bits; long bits_ld; int* nnz;             // optional keep masks (cleared by the host)
};
int gate_score_grid(int d_ff, int npb);
hipError_t launch_gate_score(int wdt, int mt, bool nt, const GateScoreParams& p, hipStream_t s);

// Top-k masks.
hipError_t launch_topk_value(const float* score, int rows, int n, int k, uint64_t* mask, int* idx, hipStream_t s);
size_t topk_blend_ws_bytes(int rows, int n);
hipError_t launch_topk_blend(const float* score, const float* prior, int rows, int n, int k, uint32_t lq,
                             uint64_t* mask, int* idx, unsigned* cnt, hipStream_t s);

// Routed MoE experts with intra-expert top-k (see moe.hip).
struct MoeParams {
  const void* x; int x_dt; long ldx; int T; int top; int E; int d_model; int d_ff; int keep_k;
  const int* ids; const float* wts;
  const uint16_t* w_gu; const uint16_t* w_down;     // [E, d_ff, 2, d_model], [E, d_ff, d_model]
  float* h; float* h_dbg; int* keep_dbg; float* partials; unsigned* counters; int n_tiles;
  void* y; int y_dt; int accumulate; int neurons_per_block;
  int atomic_y;            // down stage: each (token, slot) adds its weighted tile into y (fp32) atomically
  int x_vec;               // token rows 16-byte aligned (vector staging of x)
  // keep sets chosen at the end of the gate/up stage (keep != nullptr, d_ff <= 1024):
  // finished neuron blocks per touched expert [256], kept indices and their h
  // [T * top][keep_k]; else the down stage selects them itself
  unsigned* gu_cnt; int* keep; float* kval;
  // gate-score mode: keep neuron n of an item iff |silu(g_n)| > gate_t, up row read
  // only for kept neurons (h = 0 elsewhere); the down stage keeps the nonzero h
  int gate_mode; float gate_t; float* a_dbg;
};
hipError_t launch_router(const float* logits, int T, int E, int top, int* ids, float* wts, hipStream_t s);
hipError_t launch_moe(int wdt, const MoeParams& p, int max_unique, hipEvent_t y_ready, hipStream_t s);
hipError_t launch_moe_down(int wdt, const MoeParams& p, hipStream_t s);
int moe_down_tiles(int d_model, int items);   // column tiles of the routed down stage
// Launch shape of the routed gate/up stage (register chunks NK, neuron blocks, LDS).
int moe_gu_nk_of(const MoeParams& p);
int moe_gu_blocks_of(const MoeParams& p);
size_t moe_gu_smem_of(const MoeParams& p);

// One-stream MoE layer (moe_layer_impl.hpp): launch 1 = router logits GEMV with
// routing | shared expert gate/up (OUT_PARTS); launch 2 = routed gate/up | shared
// expert down (IN_PARTS, OUT_Y); launch 3 = launch_moe_down.  bf16 weights, up to
// 8 tokens; lpr_r in {16, 32, 64}, lpr_g in {32, 64}, lpr_d in {16, 64},
// nk in {0, 1, 2, 4, 8}.
struct MoeLayerCfg { int wdt, mt, lpr_r, lpr_g, lpr_d, nk; };
bool moe_layer_supported(const MoeLayerCfg& c);
hipError_t launch_moe_route_gu(const MoeLayerCfg& c, const GemvParams& pr, const GemvParams& pg, size_t smem,
                               hipStream_t s);
hipError_t launch_moe_gu_down(const MoeLayerCfg& c, const MoeParams& pm, int n_u, int n_gu, const GemvParams& pd,
                              size_t smem, hipStream_t s);

// Decoder-block glue (see glue.hip).
struct AttnParams {
  const float* q; const float* k_new; const float* v_new;     // fp32 projections of the current token
  const uint16_t* k_cache; const uint16_t* v_cache;            // bf16 [n_ctx, n_kv, head_dim]
  int n_ctx, n_q, n_kv, head_dim;
  float* o; float* part_o; float* part_ml; unsigned* counters;
  unsigned long long* phase_tl = nullptr;   // timeline build only: per-workgroup stamps
};
hipError_t launch_rmsnorm(const void* x, int x_dt, int rows, int d, float eps, float* y, float* copy, hipStream_t s);
hipError_t launch_attention(const AttnParams& p, int chunks, hipStream_t s);
int attention_max_group();
int attention_head_dim();
int attention_max_chunks();
int attention_max_keys();

// GLASS local signal (see glass.hip).
hipError_t launch_local_signal(const uint16_t* X, int P, int d, const uint16_t* W, long ld_neuron, long up_off,
                               int d_ff, float* local, hipStream_t s);

// Sets the calling thread's last-error text (as_last_error) and returns s.
as_status report_error(as_status s, const char* msg);

// Misc kernels.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_pack_neuron_set(const uint16_t* gu, const uint16_t* dn, int d, int f, const int* idx, int k,
                                  uint16_t* gu_out, uint16_t* dn_out, hipStream_t s);
hipError_t launch_corrected_gxo(const float* x, const float* g, int rows, int n, float* score, hipStream_t s);
hipError_t launch_fill_pattern(void* p, size_t bytes, uint32_t v, hipStream_t s);
hipError_t launch_read_probe(const void* p, size_t bytes, unsigned* sink, int cus, hipStream_t s);
size_t calibrate_ws_bytes();
hipError_t launch_calibrate(const void* pool, int dt, int64_t n, int64_t rank, float* t_out, unsigned* ghist,
                            hipStream_t s);

}  // namespace as
