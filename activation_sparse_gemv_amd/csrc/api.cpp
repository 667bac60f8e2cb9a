// C ABI of libactsparse: argument validation, workspace layout, launch planning.
#include "../../include/actsparse.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <string>

#include "internal.hpp"
#include "api_range.hpp"
#ifdef AS_PHASE_TIMELINE
#include "../../include/actsparse_timeline.h"
#endif

using namespace as;

namespace {

thread_local std::string g_last_error;

as_status fail(as_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

}  // namespace

// Error reporting for the entry points defined in other source files.
as_status as::report_error(as_status s, const char* msg) { return fail(s, "%s", msg); }

namespace {

as_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return AS_OK;
  return fail(AS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_wdt(as_dtype d) { return d == AS_F16 || d == AS_BF16; }
bool is_dt(as_dtype d) { return d == AS_F16 || d == AS_BF16 || d == AS_F32; }
int mt_for(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }
size_t up256(size_t b) { return (b + 255) & ~size_t(255); }
size_t dt_bytes(as_dtype d) { return d == AS_F32 ? 4 : 2; }
// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

int num_cus() { return device_cus(); }

// Launch plan of one row-gather GEMV over at most `rows` rows and `cols` output
// columns (paired gate/up: `cols` neurons, 2*cols columns).
struct Plan {
  int lpr, n_tiles, S, cap;
};

// LDS per workgroup on gfx950, and what a plan keeps free of it beyond the row list
// and its activations (slot reduction or staged MFMA chunk, list prefix sums).
constexpr int kLdsBytes = 160 * 1024;
// Largest contraction length (rows of W): the kernels split row lists in 32-bit arithmetic.
constexpr int kMaxRows = 1 << 24;
constexpr int kLdsReserve = 40 * 1024;

// The plan is a function of the shapes (and the device's CU count) only, so the
// workspace size a query returns always matches the call.
Plan plan_gemv(int rows, int cols, bool gu, int mt) {
  // Tile width: lanes_per_row * 8 columns.  Wider tiles give longer bursts per
  // row; narrower tiles give more tiles (less split-K, cheaper final combine).
  const long tot_cols = gu ? 2L * cols : cols;
  int lpr;
  if (tot_cols >= 512L * 48) lpr = 64;
  else if (gu) lpr = 32;
  else lpr = 16;
  if (mt >= 16) {
    // matrix-core path: slices of <= 512 rows; widen the tile until the grid fits
    // two workgroups per CU (a second round of workgroups would double the time)
    const int s16 = (rows + 511) / 512;
    while (lpr < 64) {
      const int tn2 = lpr * 8;
      const long nt2 = gu ? (cols + tn2 / 2 - 1) / (tn2 / 2) : (cols + tn2 - 1) / tn2;
      if (nt2 * s16 <= 2L * num_cus()) break;
      lpr *= 2;
    }
  }
  const int tn = lpr * 8;
  const int n_tiles = gu ? (cols + tn / 2 - 1) / (tn / 2) : (cols + tn - 1) / tn;
  // Slices: about 1.75 workgroups per CU in total, at least 128 rows per slice
  // (the last workgroup of a tile reads every slice's partial).
  // Every workgroup pays a fixed chain of round trips (input compaction, partial
  // store, tile counter, final combine), so fewer, longer workgroups win as long
  // as every CU has work (measured on MI355X for the 4096 -> 2x14336 and
  // 14336 -> 4096 shapes).
  const int target = (7 * num_cus()) / 4;
  int S = (target + n_tiles - 1) / n_tiles;
  int smax = rows / 128;
  if (smax < 1) smax = 1;
  if (S > smax) S = smax;
  if (S > 256) S = 256;
  if (S < 1) S = 1;
  // The row list and its activations ([mt][cap] fp32) sit in LDS: the matrix-core
  // path (mt 16) keeps slices at <= 512 rows so two workgroups share a CU, and every
  // plan, forced ones included, stays within the LDS of one workgroup.
  const int hard_cap = (kLdsBytes - kLdsReserve) / (4 + 4 * mt);
  if (mt >= 16) {
    const int s16 = (rows + 511) / 512;
    if (S < s16) S = s16;
  }
  if ((rows + S - 1) / S > hard_cap) S = (rows + hard_cap - 1) / hard_cap;
  // multiple of 8 rows: the MFMA loop reads activations as aligned 16-byte vectors
  const int cap = (((rows + S - 1) / S) + 7) & ~7;
  return Plan{lpr, n_tiles, S, cap};
}

// int8 rows (one token): twice the lanes per row segment of the 16-bit plan, so a
// workgroup's piece of a row is as many bytes, and the slices re-chosen for the
// halved tile count (the same ~1.75 workgroups per CU).
Plan plan_gemv_i8(int rows, int cols) {
  Plan pl = plan_gemv(rows, cols, false, 1);
  if (pl.lpr >= 64) return pl;
  pl.lpr *= 2;
  pl.n_tiles = (cols + pl.lpr * 8 - 1) / (pl.lpr * 8);
  const int target = (7 * num_cus()) / 4;
  int S = (target + pl.n_tiles - 1) / pl.n_tiles;
  const int smax = rows / 128 > 1 ? rows / 128 : 1;
  if (S > smax) S = smax;
  if (S > 256) S = 256;
  if (S < 1) S = 1;
  const int hard_cap = (kLdsBytes - kLdsReserve) / 8;
  if ((rows + S - 1) / S > hard_cap) S = (rows + hard_cap - 1) / hard_cap;
  pl.S = S;
  pl.cap = (((rows + S - 1) / S) + 7) & ~7;
  return pl;
}

struct Carver {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += up256(count * sizeof(T));
    return p;
  }
};

// Workspace of one GEMV: counters, partials.
struct GemvWs {
  unsigned* counters;
  float* partials;
};
GemvWs carve_gemv(Carver& c, const Plan& pl, int M, long part_ld) {
  GemvWs w;
  w.counters = c.take<unsigned>(size_t(pl.n_tiles) * kCounterStride);
  w.partials = c.take<float>(size_t(pl.S) * M * part_ld);
  return w;
}

// Workspace of a two-stage MLP.
struct MlpWs {
  GemvWs g1, g2;
  float* h;
  int* l_cnt;
  int* l_idx;
  float* l_val;
};

struct MlpPlan {
  Plan p1, p2;
  int n_lt, lt_stride;
  int parts2;             // partial slots of the down stage (max of its split and the ranges)
  int s2_range, cap2_range;  // down stage masking h by range: slices, max range length
  int cap1_range;            // gate/up stage masking x by range (several tokens): max range length
};

// Gate-score mode: neurons per workgroup of the scoring launch (four waves, two
// neurons each: small workgroups that the hardware refills as they finish).
// Measured on the Llama-shaped MLP, one token, 50 / 90% sparsity: 4 neurons per
// workgroup 48.9 / 36.7 us, 8: 49.3 / 36.6, 16: 50.4 / 36.8, 32: 52.2 / 38.5.
constexpr int kGateScoreNpb = 8;

MlpPlan plan_mlp(int M, const as_mlp_weights* w, as_mlp_mode mode, bool dense) {
  MlpPlan mp;
  if (mode == AS_MLP_THRESHOLD) {
    mp.p1 = plan_gemv(w->d_model, w->d_ff, true, mt_for(M));
    // One token with the down stage summing the unsummed gate/up partials: at most
    // one gate/up workgroup per CU (fewer partials for the down prologue to read,
    // and the workgroups finish together; measured on the Llama shape).
    // (The dense baseline takes the same plan, and the workspace size does not
    // depend on the flags.)
    if (M == 1) {
      const int per_cu = num_cus() / (mp.p1.n_tiles > 0 ? mp.p1.n_tiles : 1);
      if (per_cu >= 2 && per_cu < mp.p1.S) {
        mp.p1.S = per_cu;
        mp.p1.cap = (((w->d_model + per_cu - 1) / per_cu) + 7) & ~7;
      }
    }
    mp.n_lt = mp.p1.n_tiles;
    mp.lt_stride = mp.p1.lpr * 4;   // tile neurons = tile columns / 2
  } else {
    mp.p1 = Plan{0, 0, 1, 0};
    mp.n_lt = 1;
    mp.lt_stride = w->d_ff;
  }
  {
    const int units = (w->d_model + 63) / 64;
    mp.cap1_range = ((units + mp.p1.S - 1) / mp.p1.S) * 64;
  }
  (void)dense;
  mp.p2 = plan_gemv(w->d_ff, w->d_model, false, mt_for(M));
  {
    // threshold mode, two launches: down slice s masks its own 64-aligned range of h
    // (several tokens also stage the range of every token in LDS)
    const int units = (w->d_ff + 63) / 64;
    const int mt = mt_for(M);
    // per row: index, activations and the staged range (IN_RANGE with several
    // tokens, IN_PARTS)
    const int hard = (kLdsBytes - kLdsReserve) / (4 + 8 * mt);
    int S = mp.p2.S;
    // a whole number of workgroups per CU (two) where the tiles allow it: with 1.75
    // per CU the CUs holding two workgroups set the finish (measured on MI355X for
    // the 14336 -> 4096 down projection)
    if ((2 * num_cus()) % mp.p2.n_tiles == 0) S = 2 * num_cus() / mp.p2.n_tiles;
    if (S > units / 2) S = units / 2 > 1 ? units / 2 : 1;      // ranges of at least 128 rows
    while (S < units && ((units + S - 1) / S) * 64 > hard) ++S;
    mp.s2_range = S;
    mp.cap2_range = ((units + S - 1) / S) * 64;
  }
  mp.parts2 = mp.p2.S > mp.n_lt ? mp.p2.S : mp.n_lt;
  if (mp.s2_range > mp.parts2) mp.parts2 = mp.s2_range;
  return mp;
}

MlpWs carve_mlp(Carver& c, const MlpPlan& mp, int M, const as_mlp_weights* w, as_mlp_mode mode) {
  MlpWs ws;
  if (mode == AS_MLP_THRESHOLD) ws.g1 = carve_gemv(c, mp.p1, M, 2L * w->d_ff);
  else ws.g1 = GemvWs{nullptr, nullptr};
  Plan p2 = mp.p2;
  p2.S = mp.parts2;
  ws.g2 = carve_gemv(c, p2, M, w->d_model);
  ws.h = c.take<float>(size_t(M) * w->d_ff);
  ws.l_cnt = c.take<int>(mp.n_lt);
  const size_t list_len = std::max(size_t(w->d_ff), size_t(mp.n_lt) * mp.lt_stride);
  ws.l_idx = c.take<int>(list_len);
  ws.l_val = c.take<float>(list_len * M);
  return ws;
}

GemvParams base_params() {
  GemvParams p;
  memset(&p, 0, sizeof p);
  return p;
}

as_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need > 0 && ws == nullptr) return fail(AS_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (ws_bytes < need) return fail(AS_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  if (ws && !aligned16(ws)) return fail(AS_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  return AS_OK;
}

}  // namespace

// =====================================================================================
extern "C" {

int as_version(void) { return AS_VERSION; }

const char* as_status_string(as_status s) {
  switch (s) {
    case AS_OK: return "AS_OK";
    case AS_ERR_INVALID_ARG: return "AS_ERR_INVALID_ARG";
    case AS_ERR_UNSUPPORTED: return "AS_ERR_UNSUPPORTED";
    case AS_ERR_WORKSPACE: return "AS_ERR_WORKSPACE";
    case AS_ERR_HIP: return "AS_ERR_HIP";
  }
  return "AS_ERR_UNKNOWN";
}

const char* as_last_error(void) { return g_last_error.c_str(); }

as_status as_workspace_init(void* ws, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return AS_OK;
  if (!ws) return fail(AS_ERR_INVALID_ARG, "as_workspace_init: ws is NULL");
  return hip_check(launch_fill_zero(ws, bytes, stream), "as_workspace_init");
}

as_status as_bench_flush(void* buf, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return AS_OK;
  if (!buf) return fail(AS_ERR_INVALID_ARG, "as_bench_flush: buf is NULL");
  static std::atomic<uint32_t> salt{1};
  return hip_check(launch_fill_pattern(buf, bytes, 0x9e3779b9u * salt.fetch_add(1u), stream), "as_bench_flush");
}

as_status as_bench_read(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream) {
  if (bytes == 0) return AS_OK;
  if (!buf || !sink) return fail(AS_ERR_INVALID_ARG, "as_bench_read: NULL pointer");
  if (!aligned16(buf) || bytes % 16 != 0)
    return fail(AS_ERR_INVALID_ARG, "as_bench_read: buf must be 16-byte aligned and bytes a multiple of 16");
  return hip_check(launch_read_probe(buf, bytes, sink, num_cus(), stream), "as_bench_read");
}

size_t as_calibrate_threshold_ws_size(int64_t n) { return n < 1 ? 0 : up256(calibrate_ws_bytes()); }

as_status as_calibrate_threshold(const void* pool, as_dtype dt, int64_t n, int64_t p_num, int64_t p_den,
                                 float* t_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  if (!pool || !t_out) return fail(AS_ERR_INVALID_ARG, "as_calibrate_threshold: NULL pointer");
  if (!is_dt(dt)) return fail(AS_ERR_INVALID_ARG, "as_calibrate_threshold: bad dtype %d", int(dt));
  if (n < 1 || n > 2147483647LL || p_den < 1 || p_num < 0 || p_num > p_den)
    return fail(AS_ERR_INVALID_ARG, "as_calibrate_threshold: n=%lld p=%lld/%lld", (long long)n, (long long)p_num,
                (long long)p_den);
  // nearest rank ceil(p n), exact in 128-bit integers; p = 0 keeps every input
  const unsigned __int128 num = (unsigned __int128)(uint64_t)p_num * (uint64_t)n;
  const int64_t rank = p_num == 0 ? 0 : (int64_t)((num + (uint64_t)p_den - 1) / (uint64_t)p_den);
  as_status st = check_ws(ws, ws_bytes, calibrate_ws_bytes());
  if (st != AS_OK) return st;
  return hip_check(launch_calibrate(pool, int(dt), n, rank, t_out, reinterpret_cast<unsigned*>(ws), stream),
                   "as_calibrate_threshold");
}

// ------------------------------------------------------------------ GEMV
size_t as_threshold_gemv_i8_ws_size(int K, int N) {
  if (K < 1 || N < 1) return 0;
  const Plan pl = plan_gemv_i8(K, N);
  Carver c{nullptr};
  carve_gemv(c, pl, 1, N);
  return c.off;
}

size_t as_threshold_gemv_ws_size(int M, int K, int N) {
  if (M < 1 || K < 1 || N < 1) return 0;
  const Plan pl = plan_gemv(K, N, false, mt_for(M));
  Carver c{nullptr};
  carve_gemv(c, pl, M, N);
  return c.off;
}

// Work a decoder block folds into a projection (not part of the public calls):
// RMS normalisation of the input in the threshold prologue (one token, the whole
// vector in 16-byte chunks; the normalised vector optionally exported), and a
// residual added to the output.
struct GemvFuse {
  bool norm = false;
  float eps = 1e-5f;
  float* xn_out = nullptr;
  const void* res = nullptr;
  int res_dt = AS_F32;
};

// Whether the threshold prologue can normalise X itself (one token, 16-byte chunks).
static bool can_norm_in_prologue(const void* X, as_dtype x_dt, int K) {
  return pick_chunk_vectors(X, int(x_dt), K, K) > 0 && K % 8 == 0;
}

static as_status gemv_common(const void* X, as_dtype x_dt, int M, int K, const void* W, as_dtype w_dt, int N,
                             float t, void* Y, as_dtype y_dt, unsigned flags, as_mask_out* mo, void* ws,
                             size_t ws_bytes, hipStream_t stream, bool dense, const char* fn,
                             const GemvFuse* fz = nullptr, const float* row_scale = nullptr,
                             const int32_t* heads = nullptr, int n_keep = 0, int head_dim = 0) {
  if (!X || !W || !Y) return fail(AS_ERR_INVALID_ARG, "%s: NULL X, W or Y", fn);
  const bool i8 = w_dt == AS_I8;
  if (!is_dt(x_dt) || !(is_wdt(w_dt) || i8) || !is_dt(y_dt)) return fail(AS_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (i8) {
    if (!row_scale) return fail(AS_ERR_INVALID_ARG, "%s: row_scale is NULL", fn);
    if (!aligned16(row_scale)) return fail(AS_ERR_INVALID_ARG, "%s: row_scale not 16-byte aligned", fn);
    if (M != 1) return fail(AS_ERR_UNSUPPORTED, "%s: int8 weights take one token", fn);
    if (!aligned16(X) || (K % 8) != 0) return fail(AS_ERR_UNSUPPORTED, "%s: int8 weights need a 16-byte aligned X and K %% 8 == 0", fn);
    if (mo && (mo->bits || mo->idx || mo->nnz)) return fail(AS_ERR_UNSUPPORTED, "%s: int8 weights export no mask", fn);
    if (fz != nullptr) return fail(AS_ERR_UNSUPPORTED, "%s: int8 weights take no fused work", fn);
  }
  if (M < 1 || M > 16) return fail(AS_ERR_UNSUPPORTED, "%s: M=%d outside 1..16", fn, M);
  if (M > 8 && w_dt != AS_BF16) return fail(AS_ERR_UNSUPPORTED, "%s: M > 8 (MFMA path) needs bf16 weights", fn);
  if (K < 1 || N < 8 || N % 8 != 0) return fail(AS_ERR_INVALID_ARG, "%s: K=%d N=%d (N must be a multiple of 8)", fn, K, N);
  if (K > kMaxRows) return fail(AS_ERR_UNSUPPORTED, "%s: K=%d above %d", fn, K, kMaxRows);
  if (!aligned16(W)) return fail(AS_ERR_INVALID_ARG, "%s: W not 16-byte aligned", fn);
  if (mo && mo->idx && M != 1) return fail(AS_ERR_UNSUPPORTED, "%s: mask idx export needs M == 1", fn);
  const Plan pl = i8 ? plan_gemv_i8(K, N) : plan_gemv(K, N, false, mt_for(M));
  if ((long)pl.S * M * N >= (1L << 31))
    return fail(AS_ERR_UNSUPPORTED, "%s: split-K partials of %d x %d x %d exceed 2^31 elements", fn, pl.S, M, N);
  Carver c{reinterpret_cast<char*>(ws)};
  GemvWs gw = carve_gemv(c, pl, M, N);
  as_status st = check_ws(ws, ws_bytes, c.off);
  if (st != AS_OK) return st;

  GemvParams p = base_params();
  p.x = X; p.x_dt = int(x_dt); p.M = M; p.K = K; p.ldx = K; p.t = t;
  p.W = reinterpret_cast<const uint16_t*>(W); p.ldw = N; p.N = N;
  p.n_tiles = pl.n_tiles; p.S = pl.S; p.cap = pl.cap;
  // Without mask exports each slice masks its own 64-aligned range of x (no
  // whole-vector scan per workgroup); ranges of at least 128 rows.
  const bool exports = mo && (mo->bits || mo->idx || mo->nnz);
  bool range = false;
  const bool norm = fz != nullptr && fz->norm;
  if (norm && (M != 1 || !can_norm_in_prologue(X, x_dt, K)))
    return fail(AS_ERR_UNSUPPORTED, "%s: input normalisation needs one aligned token", fn);
  if (!dense && !exports && !norm) {
    const int units = (K + 63) / 64;
    int S = pl.S;
    if (S > units / 2) S = units / 2 > 1 ? units / 2 : 1;
    const int cap = ((units + S - 1) / S) * 64;
    const int mt = mt_for(M);
    if ((long)cap * (mt > 1 ? 4 + 8 * mt : 4 + 4 * mt) <= kLdsBytes - kLdsReserve) {
      range = true;
      p.S = S;
      p.cap = cap;
    }
  }
  p.partials = gw.partials; p.counters = gw.counters; p.part_ld = N;
  p.y = Y; p.y_dt = int(y_dt); p.ldy = N; p.accumulate = (flags & AS_FLAG_ACCUMULATE) ? 1 : 0;
  p.row_scale = row_scale;
  if (head_dim > 0) {
    // every input of a listed head is kept (zeros and NaN too), no other row
    p.heads = heads; p.n_heads_keep = n_keep; p.head_dim = head_dim; p.n_heads = K / head_dim; p.keep_all = 1;
  }
  if (mo && !dense) {
    p.x_bits = mo->bits; p.x_bits_ld = (K + 63) / 64; p.x_idx = mo->idx; p.x_nnz = mo->nnz;
  }
  // a head list: the dense prologue over the listed heads' rows (equal shares per slice)
  int in = (dense || head_dim > 0) ? IN_ALL : (range ? IN_RANGE : IN_THRESH);
  if (fz != nullptr) {
    if (norm) {
      // the whole vector is read by every workgroup; the dense baseline keeps every row
      in = IN_THRESH;
      p.norm_x = 1; p.norm_eps = fz->eps; p.xn_out = fz->xn_out; p.keep_all = dense ? 1 : 0;
    }
    p.res = fz->res; p.res_dt = fz->res_dt; p.ldres = N;
  }
  GemvConfig cfg{int(w_dt), mt_for(M), pl.lpr, in, OUT_Y, false, (flags & AS_FLAG_NO_NT_LOADS) == 0};
  if (flags & AS_FLAG_ATOMIC_SPLITK) {
    if (y_dt != AS_F32) return fail(AS_ERR_UNSUPPORTED, "%s: AS_FLAG_ATOMIC_SPLITK needs an fp32 Y", fn);
    p.atomic_y = 1;
    // the fill launch clears Y before X is read: they must not overlap
    if (!p.accumulate && overlaps(X, size_t(M) * K * dt_bytes(x_dt), Y, size_t(M) * N * 4))
      return fail(AS_ERR_INVALID_ARG, "%s: AS_FLAG_ATOMIC_SPLITK without AS_FLAG_ACCUMULATE needs Y apart from X", fn);
    if (!p.accumulate) {
      as_status st2 = hip_check(launch_fill_zero(Y, size_t(M) * N * sizeof(float), stream), fn);
      if (st2 != AS_OK) return st2;
    }
  }
  return hip_check(launch_gather_gemv(cfg, p, stream), fn);
}

as_status as_threshold_gemv(const void* X, as_dtype x_dt, int M, int K, const void* W, as_dtype w_dt, int N,
                            float t, void* Y, as_dtype y_dt, unsigned flags, as_mask_out* mask_out, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  const bool dense = (flags & AS_FLAG_FORCE_DENSE) != 0;
  return gemv_common(X, x_dt, M, K, W, w_dt, N, t, Y, y_dt, flags, mask_out, ws, ws_bytes, stream, dense,
                     "as_threshold_gemv");
}

as_status as_threshold_gemv_i8(const void* X, as_dtype x_dt, int K, const int8_t* W, const float* row_scale,
                               int N, float t, void* Y, as_dtype y_dt, unsigned flags, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  AS_API_RANGE();
  const bool dense = (flags & AS_FLAG_FORCE_DENSE) != 0;
  return gemv_common(X, x_dt, 1, K, W, AS_I8, N, dense ? -INFINITY : t, Y, y_dt, flags, nullptr, ws, ws_bytes,
                     stream, dense, "as_threshold_gemv_i8", nullptr, row_scale);
}

as_status as_dense_gemv(const void* X, as_dtype x_dt, int M, int K, const void* W, as_dtype w_dt, int N, void* Y,
                        as_dtype y_dt, unsigned flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  return gemv_common(X, x_dt, M, K, W, w_dt, N, -INFINITY, Y, y_dt, flags, nullptr, ws, ws_bytes, stream, true,
                     "as_dense_gemv");
}

// ------------------------------------------------------------------ MLP
static as_status check_mlp_weights(const as_mlp_weights* w, as_mlp_mode mode, const char* fn) {
  if (!w) return fail(AS_ERR_INVALID_ARG, "%s: weights struct is NULL", fn);
  if (!w->w_gate_up) return fail(AS_ERR_INVALID_ARG, "%s: w_gate_up is NULL", fn);
  if (!is_wdt(w->w_dt)) return fail(AS_ERR_INVALID_ARG, "%s: weight dtype must be f16 or bf16", fn);
  if (w->d_model < 8 || w->d_model % 8 != 0) return fail(AS_ERR_INVALID_ARG, "%s: d_model=%d not a multiple of 8", fn, w->d_model);
  if (w->d_ff < 64 || w->d_ff % 64 != 0) return fail(AS_ERR_INVALID_ARG, "%s: d_ff=%d not a multiple of 64", fn, w->d_ff);
  if (w->d_model > kMaxRows || w->d_ff > kMaxRows)
    return fail(AS_ERR_UNSUPPORTED, "%s: d_model=%d or d_ff=%d above %d", fn, w->d_model, w->d_ff, kMaxRows);
  if (!aligned16(w->w_gate_up)) return fail(AS_ERR_INVALID_ARG, "%s: w_gate_up not 16-byte aligned", fn);
  if (mode == AS_MLP_THRESHOLD) {
    if (!w->w_down) return fail(AS_ERR_INVALID_ARG, "%s: w_down is NULL", fn);
    if (!aligned16(w->w_down)) return fail(AS_ERR_INVALID_ARG, "%s: w_down not 16-byte aligned", fn);
  } else if (mode == AS_MLP_GATE_SCORE) {
    if (w->d_model > 8192) return fail(AS_ERR_UNSUPPORTED, "%s: GATE_SCORE needs d_model <= 8192", fn);
  } else if (mode != AS_MLP_NEURON_SET) {
    return fail(AS_ERR_INVALID_ARG, "%s: bad mode %d", fn, int(mode));
  }
  return AS_OK;
}

size_t as_sparse_swiglu_mlp_ws_size(int M, const as_mlp_weights* w, as_mlp_mode mode) {
  if (M < 1 || !w || w->d_model < 1 || w->d_ff < 1) return 0;
  if (M > 16 && mode == AS_MLP_THRESHOLD) {
    // groups of 16 tokens: one region for the full groups, one for a partial last group
    const size_t full = up256(as_sparse_swiglu_mlp_ws_size(16, w, mode));
    return M % 16 ? full + as_sparse_swiglu_mlp_ws_size(M % 16, w, mode) : full;
  }
  const MlpPlan mp = plan_mlp(M, w, mode, false);
  Carver c{nullptr};
  carve_mlp(c, mp, M, w, mode);
  return c.off;
}

static as_status mlp_impl(const void* X, as_dtype x_dt, int M, const as_mlp_weights* w, as_mlp_mode mode,
                          float t_x, float t_h, const int32_t* neuron_idx, int n_active, void* Y, as_dtype y_dt,
                          unsigned flags, as_mlp_debug* dbg, void* ws, size_t ws_bytes, hipStream_t stream,
                          const GemvFuse* fz);

#ifdef AS_PHASE_TIMELINE
static std::atomic<unsigned long long*> g_attn_phase_buf{nullptr};
static std::atomic<size_t> g_attn_phase_words{0};

as_status as_attention_timeline_arm(uint64_t* buf, size_t words) {
  if (buf == nullptr || words < 32)
    return fail(AS_ERR_INVALID_ARG, "as_attention_timeline_arm: NULL buffer or < 32 words");
  g_attn_phase_words.store(words);
  g_attn_phase_buf.store(reinterpret_cast<unsigned long long*>(buf));
  return AS_OK;
}

static std::atomic<unsigned long long*> g_phase_buf{nullptr};
static std::atomic<size_t> g_phase_words{0};

as_status as_phase_timeline_arm(uint64_t* buf, size_t words) {
  if (buf == nullptr || words < 32) return fail(AS_ERR_INVALID_ARG, "as_phase_timeline_arm: NULL buffer or < 32 words");
  g_phase_words.store(words);
  g_phase_buf.store(reinterpret_cast<unsigned long long*>(buf));
  return AS_OK;
}
#endif

as_status as_sparse_swiglu_mlp(const void* X, as_dtype x_dt, int M, const as_mlp_weights* w, as_mlp_mode mode,
                               float t_x, float t_h, const int32_t* neuron_idx, int n_active, void* Y,
                               as_dtype y_dt, unsigned flags, as_mlp_debug* dbg, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_sparse_swiglu_mlp";
  if (flags & AS_FLAG_AUTO) {
    if (mode != AS_MLP_THRESHOLD) return fail(AS_ERR_UNSUPPORTED, "%s: AS_FLAG_AUTO is for THRESHOLD mode", fn);
    flags &= ~unsigned(AS_FLAG_AUTO);
    if (M >= AS_AUTO_DENSE_MIN_TOKENS) flags |= AS_FLAG_FORCE_DENSE;
  }
  if (M > 16 && mode == AS_MLP_THRESHOLD) {
    // consecutive groups of 16 tokens on one stream, each a call of its own (the
    // workspace is reused in stream order; every call leaves its counters at zero)
    if (M > 256) return fail(AS_ERR_UNSUPPORTED, "%s: M=%d above 256", fn, M);
    if (dbg) return fail(AS_ERR_UNSUPPORTED, "%s: debug exports take at most 16 tokens", fn);
    if (!X || !Y || !w) return fail(AS_ERR_INVALID_ARG, "%s: NULL X, Y or weights", fn);
    if (!is_dt(x_dt) || !is_dt(y_dt)) return fail(AS_ERR_INVALID_ARG, "%s: bad dtype", fn);
    const size_t xr = size_t(w->d_model) * dt_bytes(x_dt), yr = size_t(w->d_model) * dt_bytes(y_dt);
    // the full groups use the first region of the workspace and a partial last group
    // its own second region, so each region always holds one carve-up
    const size_t ws16 = up256(as_sparse_swiglu_mlp_ws_size(16, w, mode));
    if (ws_bytes < as_sparse_swiglu_mlp_ws_size(M, w, mode))
      return fail(AS_ERR_WORKSPACE, "%s: workspace too small for %d tokens", fn, M);
    for (int m0 = 0; m0 < M; m0 += 16) {
      const int mg = M - m0 < 16 ? M - m0 : 16;
      char* wsg = reinterpret_cast<char*>(ws) + (mg == 16 ? 0 : ws16);
      const size_t wsb = mg == 16 ? ws16 : ws_bytes - ws16;
      const as_status st = mlp_impl(reinterpret_cast<const char*>(X) + m0 * xr, x_dt, mg, w, mode, t_x, t_h,
                                    neuron_idx, n_active, reinterpret_cast<char*>(Y) + m0 * yr, y_dt, flags, nullptr,
                                    wsg, wsb, stream, nullptr);
      if (st != AS_OK) return st;
    }
    return AS_OK;
  }
  return mlp_impl(X, x_dt, M, w, mode, t_x, t_h, neuron_idx, n_active, Y, y_dt, flags, dbg, ws, ws_bytes, stream,
                  nullptr);
}

as_status as_pack_neuron_set(const as_mlp_weights* w, const int32_t* idx, int k, void* gate_up_out,
                             void* down_out, hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_pack_neuron_set";
  as_status st = check_mlp_weights(w, AS_MLP_THRESHOLD, fn);
  if (st != AS_OK) return st;
  if (!idx || !gate_up_out || !down_out) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (k < 64 || k % 64 != 0 || k > w->d_ff) return fail(AS_ERR_INVALID_ARG, "%s: k=%d (multiple of 64, <= d_ff)", fn, k);
  if (!aligned16(gate_up_out) || !aligned16(down_out)) return fail(AS_ERR_INVALID_ARG, "%s: outputs not 16-byte aligned", fn);
  return hip_check(launch_pack_neuron_set(reinterpret_cast<const uint16_t*>(w->w_gate_up),
                                          reinterpret_cast<const uint16_t*>(w->w_down), w->d_model, w->d_ff, idx, k,
                                          reinterpret_cast<uint16_t*>(gate_up_out),
                                          reinterpret_cast<uint16_t*>(down_out), stream), fn);
}

// fz (nullable): the input normalised in the gate/up prologue and/or a residual
// added to y (threshold mode, two launches, one token for the normalisation).
static as_status mlp_impl(const void* X, as_dtype x_dt, int M, const as_mlp_weights* w, as_mlp_mode mode,
                          float t_x, float t_h, const int32_t* neuron_idx, int n_active, void* Y, as_dtype y_dt,
                          unsigned flags, as_mlp_debug* dbg, void* ws, size_t ws_bytes, hipStream_t stream,
                          const GemvFuse* fz) {
  const char* fn = "as_sparse_swiglu_mlp";
  as_status st = check_mlp_weights(w, mode, fn);
  if (st != AS_OK) return st;
  if (!X || !Y) return fail(AS_ERR_INVALID_ARG, "%s: NULL X or Y", fn);
  if (!is_dt(x_dt) || !is_dt(y_dt)) return fail(AS_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (M < 1 || M > 16) return fail(AS_ERR_UNSUPPORTED, "%s: M=%d outside 1..16", fn, M);
  if (M > 8 && (w->w_dt != AS_BF16 || mode != AS_MLP_THRESHOLD))
    return fail(AS_ERR_UNSUPPORTED, "%s: M > 8 (MFMA path) needs bf16 weights in THRESHOLD mode", fn);
  const bool dense = (flags & AS_FLAG_FORCE_DENSE) != 0;
  const bool atomic = (flags & AS_FLAG_ATOMIC_SPLITK) != 0;
  const bool clear_y = atomic && (flags & AS_FLAG_ACCUMULATE) == 0;
  if (atomic && y_dt != AS_F32) return fail(AS_ERR_UNSUPPORTED, "%s: AS_FLAG_ATOMIC_SPLITK needs an fp32 Y", fn);
  // with the atomic down stage, Y is cleared by the first launch while X may still be read
  if (clear_y && overlaps(X, size_t(M) * w->d_model * dt_bytes(x_dt), Y, size_t(M) * w->d_model * 4))
    return fail(AS_ERR_INVALID_ARG, "%s: AS_FLAG_ATOMIC_SPLITK without AS_FLAG_ACCUMULATE needs Y apart from X", fn);
  if (mode == AS_MLP_NEURON_SET && !dense) {
    if (n_active < 0 || n_active > w->d_ff) return fail(AS_ERR_INVALID_ARG, "%s: n_active=%d", fn, n_active);
    if (n_active > 0 && !neuron_idx) return fail(AS_ERR_INVALID_ARG, "%s: neuron_idx is NULL", fn);
  }
  if (dbg && dbg->h_mask.idx) return fail(AS_ERR_UNSUPPORTED, "%s: the h mask exports bits and nnz only", fn);
  if (dbg && dbg->x_mask.idx && M != 1) return fail(AS_ERR_UNSUPPORTED, "%s: x mask idx export needs M == 1", fn);
  if (dbg && mode == AS_MLP_NEURON_SET && (dbg->x_mask.bits || dbg->x_mask.idx || dbg->x_mask.nnz || dbg->h_mask.bits))
    return fail(AS_ERR_UNSUPPORTED, "%s: NEURON_SET exports no masks", fn);
  if (mode == AS_MLP_GATE_SCORE) {
    if (M > 8) return fail(AS_ERR_UNSUPPORTED, "%s: GATE_SCORE takes at most 8 tokens", fn);
    if (!(t_x == -INFINITY)) return fail(AS_ERR_UNSUPPORTED, "%s: GATE_SCORE does not threshold X (t_x must be -inf)", fn);
    if (dbg && (dbg->x_mask.bits || dbg->x_mask.idx || dbg->x_mask.nnz))
      return fail(AS_ERR_UNSUPPORTED, "%s: GATE_SCORE has no input mask", fn);
  }
  if (dbg && mode != AS_MLP_GATE_SCORE && dbg->a)
    return fail(AS_ERR_UNSUPPORTED, "%s: the gate activation export exists in GATE_SCORE mode only", fn);

#ifdef AS_PHASE_TIMELINE
  // an armed timeline buffer is taken by this call (first half: gate/up launch,
  // second half: down launch)
  unsigned long long* tl_buf = g_phase_buf.exchange(nullptr);
  const size_t tl_half = g_phase_words.load() / 2;
#endif
  const MlpPlan mp = plan_mlp(M, w, mode, dense);
  if ((long)mp.p1.S * M * 2L * w->d_ff >= (1L << 31) || (long)mp.parts2 * M * w->d_model >= (1L << 31))
    return fail(AS_ERR_UNSUPPORTED, "%s: split-K partials exceed 2^31 elements", fn);
  Carver c{reinterpret_cast<char*>(ws)};
  MlpWs mw = carve_mlp(c, mp, M, w, mode);
  st = check_ws(ws, ws_bytes, c.off);
  if (st != AS_OK) return st;

  const int d = w->d_model, f = w->d_ff;
  const int mt = mt_for(M);
  const bool nt = (flags & AS_FLAG_NO_NT_LOADS) == 0;
  hipEvent_t* ev = dbg ? dbg->ev : nullptr;
  auto rec = [&](int i) -> as_status {
    if (ev && ev[i]) return hip_check(hipEventRecord(ev[i], stream), "hipEventRecord");
    return AS_OK;
  };
  if ((st = rec(0)) != AS_OK) return st;

  float* hbuf = (dbg && dbg->h && mode == AS_MLP_THRESHOLD) ? dbg->h : mw.h;
  GemvParams p2 = base_params();
  GemvConfig c2{int(w->w_dt), mt, mp.p2.lpr, IN_LISTS, OUT_Y, false, nt};

  if (mode == AS_MLP_THRESHOLD) {
    // stage 1: x mask -> gate/up gather GEMV -> split-K partials, or the combined
    // g and u -> SwiGLU -> h
    // several tokens: each gate/up slice masks its own range of x (the union mask
    // over tokens is nearly dense, so equal ranges are balanced); the x mask exports
    // and one token use the evenly split compacted list
    const bool x_exports = dbg && (dbg->x_mask.bits || dbg->x_mask.idx || dbg->x_mask.nnz);
    const bool gu_range = !dense && M > 1 && !x_exports &&
                          (long)mp.cap1_range * (4 + 8 * mt) <= kLdsBytes - kLdsReserve;
    // The gate/up launch stores its split-K partials unsummed and the down launch
    // sums them for its own range of h (SwiGLU, mask and compaction in its
    // prologue): the gate/up launch then ends without the chain of partial store,
    // tile counter and combine of its last workgroups.  One token by default (the
    // down prologue reads every gate/up slice's partial of its range, which for
    // several tokens costs more than the combine it replaces).
    const bool dn_parts = mt == 1 && (long)mp.cap2_range * (4 + 8 * mt) <= kLdsBytes - kLdsReserve;
    GemvParams p = base_params();
    p.x = X; p.x_dt = int(x_dt); p.M = M; p.K = d; p.ldx = d; p.t = t_x;
    p.W = reinterpret_cast<const uint16_t*>(w->w_gate_up); p.ldw = 2L * f; p.N = f; p.gu_off = f;
    p.n_tiles = mp.p1.n_tiles; p.S = mp.p1.S; p.cap = mp.p1.cap;
    p.partials = mw.g1.partials; p.counters = mw.g1.counters; p.part_ld = 2L * f;
    p.t_h = dense ? -INFINITY : t_h; p.h = hbuf; p.ldh = f;
    if (dbg && !dense) {
      p.h_bits = dbg->h_mask.bits; p.h_bits_ld = (f + 63) / 64;
      p.x_bits = dbg->x_mask.bits; p.x_bits_ld = (d + 63) / 64; p.x_idx = dbg->x_mask.idx; p.x_nnz = dbg->x_mask.nnz;
    }
    int* h_nnz = (dbg && !dense) ? dbg->h_mask.nnz : nullptr;
    if (h_nnz != nullptr) {
      // the count is accumulated with atomics by the stage that masks h
      if ((st = hip_check(launch_fill_zero(h_nnz, size_t(M) * sizeof(int), stream), fn)) != AS_OK) return st;
    }
    if (dn_parts) { p.h = nullptr; p.h_bits = nullptr; } else { p.h_nnz = h_nnz; }
    int in1 = dense ? IN_ALL : (gu_range ? IN_RANGE : IN_THRESH);
    if (fz != nullptr && fz->norm) {
      if (M != 1 || !can_norm_in_prologue(X, x_dt, d))
        return fail(AS_ERR_UNSUPPORTED, "%s: input normalisation needs one aligned token", fn);
      // the whole vector is read by every workgroup; the dense baseline keeps every row
      in1 = IN_THRESH;
      p.norm_x = 1; p.norm_eps = fz->eps; p.xn_out = fz->xn_out; p.keep_all = dense ? 1 : 0;
    }
    GemvConfig c1{int(w->w_dt), mt, mp.p1.lpr, in1, dn_parts ? OUT_PARTS : OUT_SWIGLU, true, nt};
    if (gu_range) p.cap = mp.cap1_range;
    // the down stage adds into Y: the gate/up launch clears it (Y does not alias X)
    if (clear_y) { p.zero_y = reinterpret_cast<float*>(Y); p.zero_n = long(M) * d; }
#ifdef AS_PHASE_TIMELINE
    if (tl_buf != nullptr && (size_t)p.n_tiles * p.S * 16 <= tl_half) p.phase_tl = tl_buf;
#endif
    if ((st = hip_check(launch_gather_gemv(c1, p, stream), fn)) != AS_OK) return st;
    if ((st = rec(1)) != AS_OK) return st;
    // stage 2: down projection over the surviving h rows; each slice masks its
    // own range of h
    p2.W = reinterpret_cast<const uint16_t*>(w->w_down); p2.ldw = d;
    if (dn_parts) {
      c2.in = IN_PARTS;
      p2.x = mw.g1.partials; p2.x_dt = AS_F32; p2.K = f; p2.ldx = 2L * f; p2.t = dense ? -INFINITY : t_h;
      p2.x_parts = mp.p1.S; p2.x_up = f; p2.keep_all = dense ? 1 : 0;
      p2.h = (dbg && dbg->h) ? dbg->h : nullptr; p2.ldh = f;
      if (dbg && !dense) { p2.h_bits = dbg->h_mask.bits; p2.h_bits_ld = (f + 63) / 64; p2.h_nnz = h_nnz; }
    } else if (dense) {
      c2.in = IN_ALL;
      p2.x = hbuf; p2.x_dt = AS_F32; p2.K = f; p2.ldx = f; p2.t = -INFINITY;
    } else {
      c2.in = IN_RANGE;
      p2.x = hbuf; p2.x_dt = AS_F32; p2.K = f; p2.ldx = f; p2.t = t_h;
    }
  } else if (mode == AS_MLP_GATE_SCORE) {
    // stage 1: dense gate over every neuron, |silu(g)| > t_h, up over the kept ones;
    // the kept neurons' h values go out as one list tile per workgroup
    if (clear_y && (st = hip_check(launch_fill_zero(Y, size_t(M) * d * sizeof(float), stream), fn)) != AS_OK)
      return st;
    const bool want_bits = dbg && !dense && dbg->h_mask.bits;
    const bool want_nnz = dbg && !dense && dbg->h_mask.nnz;
    if (want_bits && (st = hip_check(launch_fill_zero(dbg->h_mask.bits, size_t(M) * ((f + 63) / 64) * 8, stream), fn)) != AS_OK)
      return st;
    if (want_nnz && (st = hip_check(launch_fill_zero(dbg->h_mask.nnz, size_t(M) * sizeof(int), stream), fn)) != AS_OK)
      return st;
    float* hg = (dbg && dbg->h) ? dbg->h : mw.h;
    GateScoreParams q;
    memset(&q, 0, sizeof q);
    q.x = X; q.x_dt = int(x_dt); q.M = M; q.ldx = d; q.d_model = d; q.d_ff = f;
    q.W = reinterpret_cast<const uint16_t*>(w->w_gate_up); q.ld_neuron = 3L * d; q.up_off = d;
    q.t = t_h; q.keep_all = dense ? 1 : 0; q.npb = kGateScoreNpb;
    q.h = hg; q.ldh = f; q.a_dbg = dbg ? dbg->a : nullptr;
    q.bits = want_bits ? dbg->h_mask.bits : nullptr; q.bits_ld = (f + 63) / 64;
    q.nnz = want_nnz ? dbg->h_mask.nnz : nullptr;
    if ((st = hip_check(launch_gate_score(int(w->w_dt), mt, nt, q, stream), fn)) != AS_OK) return st;
    if ((st = rec(1)) != AS_OK) return st;
    // stage 2: down rows of the neurons with a nonzero h; each slice compacts its own
    // range of h (a dropped neuron's h is exactly 0; the dense baseline reads every row)
    p2.W = reinterpret_cast<const uint16_t*>(w->w_gate_up) + 2L * d; p2.ldw = 3L * d;
    p2.x = hg; p2.x_dt = AS_F32; p2.K = f; p2.ldx = f; p2.t = 0.0f;
    c2.in = dense ? IN_ALL : IN_RANGE;
  } else {
    // stage 1: gate/up dot products of the listed neurons (neuron-major rows)
    if (clear_y && (st = hip_check(launch_fill_zero(Y, size_t(M) * d * sizeof(float), stream), fn)) != AS_OK)
      return st;
    NeuronGuParams q;
    memset(&q, 0, sizeof q);
    q.x = X; q.x_dt = int(x_dt); q.M = M; q.ldx = d; q.d_model = d;
    q.W = reinterpret_cast<const uint16_t*>(w->w_gate_up); q.ld_neuron = 3L * d; q.up_off = d;
    q.idx = dense ? nullptr : neuron_idx; q.n_active = dense ? f : n_active;
    q.h_dbg = dbg ? dbg->h : nullptr; q.ld_hdbg = q.n_active;
    q.o_cnt = mw.l_cnt; q.o_idx = mw.l_idx; q.o_val = mw.l_val;
    q.neurons_per_wave = 2;
    if ((st = hip_check(launch_neuron_gu(int(w->w_dt), mt, nt, q, stream), fn)) != AS_OK) return st;
    if ((st = rec(1)) != AS_OK) return st;
    p2.W = reinterpret_cast<const uint16_t*>(w->w_gate_up) + 2L * d; p2.ldw = 3L * d;
  }
  p2.M = M;
  p2.list_cnt = mw.l_cnt; p2.list_idx = mw.l_idx; p2.list_val = mw.l_val;
  p2.n_lt = mp.n_lt; p2.lt_stride = mp.lt_stride;
  p2.N = d;
  p2.n_tiles = mp.p2.n_tiles; p2.S = mp.p2.S; p2.cap = mp.p2.cap;
  if (c2.in == IN_RANGE || c2.in == IN_PARTS) { p2.S = mp.s2_range; p2.cap = mp.cap2_range; }
  p2.partials = mw.g2.partials; p2.counters = mw.g2.counters; p2.part_ld = d;
  p2.y = Y; p2.y_dt = int(y_dt); p2.ldy = d; p2.accumulate = (flags & AS_FLAG_ACCUMULATE) ? 1 : 0;
  p2.atomic_y = atomic ? 1 : 0;
  if (fz != nullptr) { p2.res = fz->res; p2.res_dt = fz->res_dt; p2.ldres = d; }
#ifdef AS_PHASE_TIMELINE
  if (tl_buf != nullptr && (size_t)p2.n_tiles * p2.S * 16 <= tl_half) p2.phase_tl = tl_buf + tl_half;
#endif
  if ((st = hip_check(launch_gather_gemv(c2, p2, stream), fn)) != AS_OK) return st;
  return rec(2);
}

// ------------------------------------------------------------------ attribution selection
as_status as_corrected_gxo(const float* x, const float* grad, int rows, int n, float* score, hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_corrected_gxo";
  if (!x || !grad || !score) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (rows < 1 || n < 1) return fail(AS_ERR_INVALID_ARG, "%s: rows=%d n=%d", fn, rows, n);
  return hip_check(launch_corrected_gxo(x, grad, rows, n, score, stream), fn);
}

int as_top_fraction_count(int n, int ar_num, int ar_den) {
  if (n < 0 || ar_den <= 0 || ar_num < 0 || ar_num > ar_den) return -1;
  const unsigned __int128 a = (unsigned __int128)(unsigned)ar_num * (unsigned)n;
  return (int)((a + (unsigned)ar_den - 1) / (unsigned)ar_den);
}

as_status as_select_top_fraction(const float* score, int rows, int n, int ar_num, int ar_den, uint64_t* mask,
                                 int32_t* idx, hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_select_top_fraction";
  if (!score) return fail(AS_ERR_INVALID_ARG, "%s: score is NULL", fn);
  if (!mask && !idx) return fail(AS_ERR_INVALID_ARG, "%s: both outputs are NULL", fn);
  if (rows < 1 || n < 1) return fail(AS_ERR_INVALID_ARG, "%s: rows=%d n=%d", fn, rows, n);
  const int k = as_top_fraction_count(n, ar_num, ar_den);
  if (k < 0) return fail(AS_ERR_INVALID_ARG, "%s: ratio %d/%d outside [0, 1]", fn, ar_num, ar_den);
  return hip_check(launch_topk_value(score, rows, n, k, mask, idx, stream), fn);
}

size_t as_head_masked_gemv_ws_size(int n_heads, int head_dim, int N) {
  if (n_heads < 1 || head_dim < 1 || N < 1) return 0;
  return as_threshold_gemv_ws_size(1, n_heads * head_dim, N);
}

as_status as_head_masked_gemv(const void* X, as_dtype x_dt, int n_heads, int head_dim, const int32_t* heads,
                              int n_keep, const void* W, as_dtype w_dt, int N, void* Y, as_dtype y_dt,
                              unsigned flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_head_masked_gemv";
  if (!X || !W || !Y) return fail(AS_ERR_INVALID_ARG, "%s: NULL X, W or Y", fn);
  if (n_heads < 1 || n_heads > 1024 || head_dim < 1) return fail(AS_ERR_INVALID_ARG, "%s: n_heads=%d head_dim=%d", fn, n_heads, head_dim);
  if (n_keep < 0 || n_keep > n_heads || (n_keep > 0 && !heads)) return fail(AS_ERR_INVALID_ARG, "%s: n_keep=%d", fn, n_keep);
  if (!is_dt(x_dt)) return fail(AS_ERR_INVALID_ARG, "%s: bad x dtype", fn);
  if (flags & (AS_FLAG_FORCE_DENSE | AS_FLAG_ACCUMULATE))
    return fail(AS_ERR_UNSUPPORTED, "%s: flags other than AS_FLAG_ATOMIC_SPLITK / AS_FLAG_NO_NT_LOADS", fn);
  const int K = n_heads * head_dim;
  if (!aligned16(X) || (K % 8) != 0)
    return fail(AS_ERR_UNSUPPORTED, "%s: needs a 16-byte aligned X and n_heads * head_dim %% 8 == 0", fn);
  // one launch: every slice masks its range of X by the head list (t = -inf: all of
  // a kept head's inputs, zeros and NaN included) and reads only the kept rows
  return gemv_common(X, x_dt, 1, K, W, w_dt, N, -INFINITY, Y, y_dt, flags, nullptr, ws, ws_bytes, stream, false,
                     fn, nullptr, nullptr, heads, n_keep, head_dim);
}

// ------------------------------------------------------------------ greedy allocation
as_status as_greedy_sparsity(const double* err, int n_blocks, int n_levels, const double* weights, double step,
                             double target, int32_t* levels) {
  AS_API_RANGE();
  const char* fn = "as_greedy_sparsity";
  if (!err || !weights || !levels) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (n_blocks < 1 || n_levels < 1) return fail(AS_ERR_INVALID_ARG, "%s: n_blocks=%d n_levels=%d", fn, n_blocks, n_levels);
  if (!(step > 0.0) || !std::isfinite(step)) return fail(AS_ERR_INVALID_ARG, "%s: step must be > 0", fn);
  if (!(target >= 0.0 && target <= 1.0)) return fail(AS_ERR_INVALID_ARG, "%s: target outside [0, 1]", fn);
  double wsum = 0.0;
  for (int b = 0; b < n_blocks; ++b) {
    if (!(weights[b] > 0.0) || !std::isfinite(weights[b])) return fail(AS_ERR_INVALID_ARG, "%s: weight %d", fn, b);
    wsum += weights[b];
    for (int l = 0; l < n_levels; ++l)
      if (!std::isfinite(err[(size_t)b * n_levels + l])) return fail(AS_ERR_INVALID_ARG, "%s: err[%d][%d]", fn, b, l);
  }
  for (int b = 0; b < n_blocks; ++b) levels[b] = 0;
  auto overall = [&]() {
    double s = 0.0;
    for (int b = 0; b < n_blocks; ++b) s += weights[b] * levels[b] * step;
    return s / wsum;
  };
  while (overall() < target * (1.0 - 1e-12)) {
    int best_b = -1;
    double best = 0.0;
    for (int b = 0; b < n_blocks; ++b) {
      if (levels[b] + 1 >= n_levels) continue;
      const double inc = err[(size_t)b * n_levels + levels[b] + 1] - err[(size_t)b * n_levels + levels[b]];
      if (best_b < 0 || inc < best) { best = inc; best_b = b; }
    }
    if (best_b < 0) break;
    ++levels[best_b];
  }
  return AS_OK;
}

// ------------------------------------------------------------------ top-k
size_t as_topk_mask_ws_size(int rows, int n, as_topk_mode mode) {
  if (mode != AS_TOPK_RANK_BLEND || rows < 1 || n < 1) return 0;
  return up256(topk_blend_ws_bytes(rows, n));
}

as_status as_topk_mask(const float* score, const float* prior, int rows, int n, int k, as_topk_mode mode,
                       float lambda, uint64_t* mask, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_topk_mask";
  if (!score) return fail(AS_ERR_INVALID_ARG, "%s: score is NULL", fn);
  if (!mask && !idx) return fail(AS_ERR_INVALID_ARG, "%s: both outputs are NULL", fn);
  if (rows < 1 || n < 1) return fail(AS_ERR_INVALID_ARG, "%s: rows=%d n=%d", fn, rows, n);
  if (k < 0 || k > n) return fail(AS_ERR_INVALID_ARG, "%s: k=%d outside 0..n=%d", fn, k, n);
  if (mode == AS_TOPK_VALUE) return hip_check(launch_topk_value(score, rows, n, k, mask, idx, stream), fn);
  if (mode != AS_TOPK_RANK_BLEND) return fail(AS_ERR_INVALID_ARG, "%s: bad mode %d", fn, int(mode));
  if (!prior) return fail(AS_ERR_INVALID_ARG, "%s: prior is NULL", fn);
  if (!(lambda >= 0.f && lambda <= 1.f)) return fail(AS_ERR_INVALID_ARG, "%s: lambda=%g outside [0, 1]", fn, lambda);
  if (n > 65535) return fail(AS_ERR_UNSUPPORTED, "%s: RANK_BLEND needs n <= 65535 (n=%d)", fn, n);
  as_status st = check_ws(ws, ws_bytes, as_topk_mask_ws_size(rows, n, mode));
  if (st != AS_OK) return st;
  const uint32_t lq = (uint32_t)floor((double)lambda * 65536.0 + 0.5);
  return hip_check(launch_topk_blend(score, prior, rows, n, k, lq, mask, idx, reinterpret_cast<unsigned*>(ws),
                                     stream), fn);
}

// ------------------------------------------------------------------ MoE
as_status as_moe_router(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                        hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_moe_router";
  if (!logits || !ids || !weights) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (T < 1 || E < 1 || E > 1024) return fail(AS_ERR_INVALID_ARG, "%s: T=%d E=%d", fn, T, E);
  if (top_k < 1 || top_k > E || top_k > 64) return fail(AS_ERR_INVALID_ARG, "%s: top_k=%d", fn, top_k);
  return hip_check(launch_router(logits, T, E, top_k, ids, weights, stream), fn);
}

// Router logits and routing in one launch: the dense logits GEMV whose single
// column tile's last workgroup routes every token (OUT_ROUTER).  Same plan as the
// dense GEMV of as_dense_gemv, so the logits are the same bits.
static Plan router_plan(int d_model, int E, int T) {
  Plan pl = plan_gemv(d_model, E, false, mt_for(T));
  const int lpr = E <= 128 ? 16 : E <= 256 ? 32 : 64;
  if (pl.lpr < lpr) pl.lpr = lpr;
  pl.n_tiles = 1;
  return pl;
}

size_t as_moe_router_gemv_ws_size(int T, int d_model, int E) {
  if (T < 1 || T > 8 || d_model < 1 || E < 8 || E > 512) return 0;
  const Plan pl = router_plan(d_model, E, T);
  Carver c{nullptr};
  carve_gemv(c, pl, T, E);
  return c.off;
}

as_status as_moe_router_gemv(const void* X, as_dtype x_dt, int T, const void* w_router, as_dtype w_dt, int d_model,
                             int E, int top_k, float* logits, int32_t* ids, float* weights, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_moe_router_gemv";
  if (!X || !w_router || !logits || !ids || !weights) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!is_dt(x_dt) || !is_wdt(w_dt)) return fail(AS_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (T < 1 || d_model < 1 || E < 8 || E % 8 != 0) return fail(AS_ERR_INVALID_ARG, "%s: T=%d d=%d E=%d", fn, T, d_model, E);
  if (top_k < 1 || top_k > E || top_k > 64) return fail(AS_ERR_INVALID_ARG, "%s: top_k=%d", fn, top_k);
  if (T > 8 || E > 512 || d_model > kMaxRows)
    return fail(AS_ERR_UNSUPPORTED, "%s: T=%d (<= 8), E=%d (<= 512), d=%d", fn, T, E, d_model);
  if (!aligned16(w_router)) return fail(AS_ERR_INVALID_ARG, "%s: w_router not 16-byte aligned", fn);
  const Plan pl = router_plan(d_model, E, T);
  Carver c{reinterpret_cast<char*>(ws)};
  GemvWs gw = carve_gemv(c, pl, T, E);
  as_status st = check_ws(ws, ws_bytes, c.off);
  if (st != AS_OK) return st;
  GemvParams p = base_params();
  p.x = X; p.x_dt = int(x_dt); p.M = T; p.K = d_model; p.ldx = d_model; p.t = -INFINITY;
  p.W = reinterpret_cast<const uint16_t*>(w_router); p.ldw = E; p.N = E;
  p.n_tiles = 1; p.S = pl.S; p.cap = pl.cap;
  p.partials = gw.partials; p.counters = gw.counters; p.part_ld = E;
  p.y = logits; p.y_dt = AS_F32; p.ldy = E;
  p.route_top = top_k; p.route_ids = ids; p.route_wts = weights;
  GemvConfig cfg{int(w_dt), mt_for(T), pl.lpr, IN_ALL, OUT_ROUTER, false, true};
  return hip_check(launch_gather_gemv(cfg, p, stream), fn);
}

namespace {
// Neurons per gate/up workgroup: 16 for one token's 8 items (more workgroups keep
// every CU busy), 32 beyond (fewer, longer workgroups; measured on the 128-expert,
// d_model 2048, d_ff_e 768 shape for 1 to 16 tokens).
int moe_npb(int items) { return items <= 8 ? 16 : 32; }

struct MoeWs {
  float* h;
  float* partials;
  unsigned* counters;
  unsigned* gu_cnt;     // finished neuron blocks per touched expert
  int* keep;            // keep sets [T * top][keep_k <= d_ff_e]
  float* kval;
};
MoeWs carve_moe(Carver& c, int T, int top, const as_moe_weights* w) {
  MoeWs m;
  m.h = c.take<float>(size_t(T) * top * w->d_ff_e);
  m.partials = c.take<float>(size_t(T) * top * w->d_model);
  m.counters = c.take<unsigned>(size_t(T) * moe_down_tiles(w->d_model, T * top) * kCounterStride);
  m.gu_cnt = c.take<unsigned>(size_t(256) * kCounterStride);
  m.keep = c.take<int>(size_t(T) * top * w->d_ff_e);
  m.kval = c.take<float>(size_t(T) * top * w->d_ff_e);
  return m;
}
// Where the keep sets are chosen: at the end of the gate/up stage (the last neuron
// block of each expert) or at the start of the down stage (every column tile of an
// item).  The first shortens the down stage and overlaps the selections of many
// experts with the gate/up stream; the second keeps the one-token chain shortest
// (the last gate/up block otherwise sets the end of its launch).  Measured on the
// 128-expert, d_ff_e 768 shape: one token 38 vs 41 us per layer, four tokens 72.8
// vs 68.5.  Rows longer than 1024 neurons always select in the down stage.
bool moe_select_in_gu(int items, int d_ff_e, bool layer) {
  if (d_ff_e > 1024) return false;
  return layer && items > 8;
}
}  // namespace

size_t as_sparse_moe_expert_ws_size(int T, int top_k, const as_moe_weights* w) {
  if (!w || T < 1 || top_k < 1 || w->n_experts < 1 || w->d_model < 1 || w->d_ff_e < 1) return 0;
  Carver c{nullptr};
  carve_moe(c, T, top_k, w);
  return c.off;
}

namespace {
// Keep rule of the routed experts: the exact top keep_k of |h| per (token, slot), or
// (gate) the neurons with |silu(g)| > t_gate.
struct MoeKeepRule {
  bool gate;
  float t_gate;
  float* a_dbg;
};

as_status moe_expert_impl(const char* fn, const void* X, as_dtype x_dt, int T, const int32_t* expert_ids,
                          const float* expert_w, int top_k, const as_moe_weights* w, int keep_k,
                          const MoeKeepRule& rule, void* Y, as_dtype y_dt, unsigned flags, float* h_dbg,
                          int32_t* keep_dbg, hipEvent_t y_ready, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!X || !expert_ids || !expert_w || !w || !Y) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!w->w_gate_up || !w->w_down) return fail(AS_ERR_INVALID_ARG, "%s: NULL weights", fn);
  if (!is_dt(x_dt) || !is_dt(y_dt) || !is_wdt(w->w_dt)) return fail(AS_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (T < 1 || top_k < 1 || top_k > 32 || T * top_k > 256)
    return fail(AS_ERR_INVALID_ARG, "%s: T=%d top_k=%d (top_k <= 32, T*top_k <= 256)", fn, T, top_k);
  if (w->n_experts < 1 || w->n_experts > 1024) return fail(AS_ERR_INVALID_ARG, "%s: E=%d", fn, w->n_experts);
  if (w->d_model < 8 || w->d_model % 8 != 0) return fail(AS_ERR_INVALID_ARG, "%s: d_model=%d", fn, w->d_model);
  if (w->d_ff_e < 1 || w->d_ff_e > 8192) return fail(AS_ERR_UNSUPPORTED, "%s: d_ff_e=%d outside 1..8192", fn, w->d_ff_e);
  if (keep_k < 0 || keep_k > w->d_ff_e) return fail(AS_ERR_INVALID_ARG, "%s: keep_k=%d", fn, keep_k);
  if (!aligned16(w->w_gate_up) || !aligned16(w->w_down)) return fail(AS_ERR_INVALID_ARG, "%s: weights not 16-byte aligned", fn);
  Carver c{reinterpret_cast<char*>(ws)};
  MoeWs m = carve_moe(c, T, top_k, w);
  as_status st = check_ws(ws, ws_bytes, c.off);
  if (st != AS_OK) return st;
  MoeParams p;
  memset(&p, 0, sizeof p);
  p.x = X; p.x_dt = int(x_dt); p.ldx = w->d_model; p.T = T; p.top = top_k; p.E = w->n_experts;
  p.d_model = w->d_model; p.d_ff = w->d_ff_e;
  p.keep_k = (flags & AS_FLAG_FORCE_DENSE) ? w->d_ff_e : keep_k;
  p.ids = expert_ids; p.wts = expert_w;
  p.w_gu = reinterpret_cast<const uint16_t*>(w->w_gate_up); p.w_down = reinterpret_cast<const uint16_t*>(w->w_down);
  p.h = m.h; p.h_dbg = h_dbg; p.keep_dbg = (flags & AS_FLAG_FORCE_DENSE) ? nullptr : keep_dbg;
  p.partials = m.partials; p.counters = m.counters; p.n_tiles = moe_down_tiles(w->d_model, T * top_k);
  if (moe_select_in_gu(T * top_k, w->d_ff_e, false)) { p.gu_cnt = m.gu_cnt; p.keep = m.keep; p.kval = m.kval; }
  if (rule.gate) {
    // every neuron's h is written (0 where dropped); the down stage keeps the nonzero
    p.gate_mode = 1;
    p.gate_t = (flags & AS_FLAG_FORCE_DENSE) ? -INFINITY : rule.t_gate;
    p.a_dbg = rule.a_dbg;
    p.keep_k = 0; p.keep_dbg = nullptr; p.keep = nullptr; p.kval = nullptr; p.gu_cnt = nullptr;
  }
  p.y = Y; p.y_dt = int(y_dt); p.accumulate = (flags & AS_FLAG_ACCUMULATE) ? 1 : 0;
  p.neurons_per_block = moe_npb(T * top_k);
  if (flags & AS_FLAG_ATOMIC_SPLITK) {
    if (y_dt != AS_F32) return fail(AS_ERR_UNSUPPORTED, "%s: AS_FLAG_ATOMIC_SPLITK needs an fp32 Y", fn);
    p.atomic_y = 1;
    if (!p.accumulate && overlaps(X, size_t(T) * w->d_model * dt_bytes(x_dt), Y, size_t(T) * w->d_model * 4))
      return fail(AS_ERR_INVALID_ARG, "%s: AS_FLAG_ATOMIC_SPLITK without AS_FLAG_ACCUMULATE needs Y apart from X", fn);
    if (!p.accumulate && (st = hip_check(launch_fill_zero(Y, size_t(T) * w->d_model * sizeof(float), stream), fn)) != AS_OK)
      return st;
  }
  {
    const int es = x_dt == AS_F32 ? 4 : 2;
    p.x_vec = aligned16(X) && (long(w->d_model) * es) % 16 == 0;
  }
  const int max_unique = T * top_k < w->n_experts ? T * top_k : w->n_experts;
  return hip_check(launch_moe(int(w->w_dt), p, max_unique, y_ready, stream), fn);
}
}  // namespace

as_status as_sparse_moe_expert(const void* X, as_dtype x_dt, int T, const int32_t* expert_ids,
                               const float* expert_w, int top_k, const as_moe_weights* w, int keep_k, void* Y,
                               as_dtype y_dt, unsigned flags, float* h_dbg, int32_t* keep_dbg,
                               hipEvent_t y_ready, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  const MoeKeepRule rule{false, 0.f, nullptr};
  return moe_expert_impl("as_sparse_moe_expert", X, x_dt, T, expert_ids, expert_w, top_k, w, keep_k, rule, Y, y_dt,
                         flags, h_dbg, keep_dbg, y_ready, ws, ws_bytes, stream);
}

as_status as_sparse_moe_expert_gate(const void* X, as_dtype x_dt, int T, const int32_t* expert_ids,
                                    const float* expert_w, int top_k, const as_moe_weights* w, float t_gate,
                                    void* Y, as_dtype y_dt, unsigned flags, float* h_dbg, float* a_dbg,
                                    hipEvent_t y_ready, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  if (std::isnan(t_gate)) return fail(AS_ERR_INVALID_ARG, "as_sparse_moe_expert_gate: t_gate is NaN");
  const MoeKeepRule rule{true, t_gate, a_dbg};
  return moe_expert_impl("as_sparse_moe_expert_gate", X, x_dt, T, expert_ids, expert_w, top_k, w, 0, rule, Y, y_dt,
                         flags, h_dbg, nullptr, y_ready, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ MoE layer (one stream)
namespace {
// Plans of the three pieces and the combined launches' shapes; ok = false when the
// shapes are outside the combined launches' limits.
struct MoeLayerPlan {
  bool ok;
  Plan router;
  MlpPlan shared;
  MoeLayerCfg cfg;    // nk filled in at the call (depends on X's alignment)
};

MoeLayerPlan moe_layer_plan(int T, int top_k, const as_moe_layer_weights* w) {
  MoeLayerPlan lp;
  memset(&lp, 0, sizeof lp);
  if (!w || T < 1 || T > 8 || top_k < 1) return lp;
  const as_moe_weights& e = w->experts;
  const as_mlp_weights& sh = w->shared;
  const int E = e.n_experts, d = e.d_model;
  if (E < 8 || E > 512 || E % 8 != 0 || top_k > 32 || top_k > E || T * top_k > 256) return lp;
  if (d < 8 || d % 8 != 0 || d > kMaxRows || e.d_ff_e < 1 || e.d_ff_e > 8192) return lp;
  if (sh.d_model != d || sh.d_ff < 64 || sh.d_ff % 64 != 0 || sh.d_ff > kMaxRows) return lp;
  if (e.w_dt != AS_BF16 || sh.w_dt != AS_BF16) return lp;
  lp.router = router_plan(d, E, T);
  lp.shared = plan_mlp(T, &sh, AS_MLP_THRESHOLD, true);
  {
    // The shared down stage shares its launch with the routed gate/up workgroups,
    // which take most of the device: one row range per CU and column tile, so the
    // launch fits one round of workgroups.
    MlpPlan& mp = lp.shared;
    const int units = (sh.d_ff + 63) / 64;
    const int per = num_cus() / (mp.p2.n_tiles > 0 ? mp.p2.n_tiles : 1);
    if (per >= 1 && per < mp.s2_range) {
      mp.s2_range = per;
      mp.cap2_range = ((units + per - 1) / per) * 64;
    }
  }
  const int mt = mt_for(T);
  lp.cfg = MoeLayerCfg{int(AS_BF16), mt, lp.router.lpr, lp.shared.p1.lpr, lp.shared.p2.lpr, 0};
  if (!moe_layer_supported(lp.cfg)) return lp;
  // the shared down stage stages its range of every token's partial sums in LDS
  if ((long)lp.shared.cap2_range * (4 + 8 * mt) > kLdsBytes - kLdsReserve) return lp;
  if ((long)lp.shared.p1.S * T * 2L * sh.d_ff >= (1L << 31) || (long)lp.shared.parts2 * T * d >= (1L << 31))
    return lp;
  lp.ok = true;
  return lp;
}

struct MoeLayerWs {
  GemvWs router;
  MlpWs shared;
  MoeWs moe;
};
MoeLayerWs carve_moe_layer(Carver& c, const MoeLayerPlan& lp, int T, int top_k, const as_moe_layer_weights* w) {
  MoeLayerWs m;
  m.router = carve_gemv(c, lp.router, T, w->experts.n_experts);
  m.shared = carve_mlp(c, lp.shared, T, &w->shared, AS_MLP_THRESHOLD);
  m.moe = carve_moe(c, T, top_k, &w->experts);
  return m;
}
}  // namespace

size_t as_moe_layer_ws_size(int T, int top_k, const as_moe_layer_weights* w) {
  const MoeLayerPlan lp = moe_layer_plan(T, top_k, w);
  if (!lp.ok) return 0;
  Carver c{nullptr};
  carve_moe_layer(c, lp, T, top_k, w);
  return c.off;
}

namespace {
as_status moe_layer_impl(const char* fn, const void* X, as_dtype x_dt, int T, const as_moe_layer_weights* w,
                         int top_k, int keep_k, const MoeKeepRule& rule, float* Y, unsigned flags, float* logits,
                         int32_t* ids, float* weights, float* h_dbg, int32_t* keep_dbg, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!X || !w || !Y || !logits || !ids || !weights) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!w->w_router || !w->experts.w_gate_up || !w->experts.w_down)
    return fail(AS_ERR_INVALID_ARG, "%s: NULL router or expert weights", fn);
  as_status st = check_mlp_weights(&w->shared, AS_MLP_THRESHOLD, fn);
  if (st != AS_OK) return st;
  if (!is_dt(x_dt)) return fail(AS_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (T < 1 || top_k < 1) return fail(AS_ERR_INVALID_ARG, "%s: T=%d top_k=%d", fn, T, top_k);
  const as_moe_weights& ew = w->experts;
  if (keep_k < 0 || keep_k > ew.d_ff_e) return fail(AS_ERR_INVALID_ARG, "%s: keep_k=%d", fn, keep_k);
  if ((flags & ~unsigned(AS_FLAG_FORCE_DENSE | AS_FLAG_ATOMIC_SPLITK)) != 0)
    return fail(AS_ERR_UNSUPPORTED, "%s: flags 0x%x", fn, flags);
  if (!aligned16(w->w_router) || !aligned16(ew.w_gate_up) || !aligned16(ew.w_down))
    return fail(AS_ERR_INVALID_ARG, "%s: weights not 16-byte aligned", fn);
  MoeLayerPlan lp = moe_layer_plan(T, top_k, w);
  if (!lp.ok)
    return fail(AS_ERR_UNSUPPORTED, "%s: T=%d E=%d top_k=%d d=%d d_ff_e=%d outside the one-stream layer's limits",
                fn, T, ew.n_experts, top_k, ew.d_model, ew.d_ff_e);
  Carver c{reinterpret_cast<char*>(ws)};
  const MoeLayerWs m = carve_moe_layer(c, lp, T, top_k, w);
  if ((st = check_ws(ws, ws_bytes, c.off)) != AS_OK) return st;

  const int E = ew.n_experts, d = ew.d_model, f = w->shared.d_ff, mt = lp.cfg.mt;
  const bool dense = (flags & AS_FLAG_FORCE_DENSE) != 0;
  // launch 1, first piece: router logits GEMV, its last workgroup routes (as in as_moe_router_gemv)
  GemvParams pr = base_params();
  pr.x = X; pr.x_dt = int(x_dt); pr.M = T; pr.K = d; pr.ldx = d; pr.t = -INFINITY;
  pr.W = reinterpret_cast<const uint16_t*>(w->w_router); pr.ldw = E; pr.N = E;
  pr.n_tiles = 1; pr.S = lp.router.S; pr.cap = lp.router.cap;
  pr.partials = m.router.partials; pr.counters = m.router.counters; pr.part_ld = E;
  pr.y = logits; pr.y_dt = AS_F32; pr.ldy = E;
  pr.route_top = top_k; pr.route_ids = ids; pr.route_wts = weights;
  // second piece: the shared expert's gate/up, every row, partials unsummed (as the
  // dense MLP's gate/up stage with the down stage summing the partials)
  const MlpPlan& mp = lp.shared;
  GemvParams pg = base_params();
  pg.x = X; pg.x_dt = int(x_dt); pg.M = T; pg.K = d; pg.ldx = d; pg.t = -INFINITY; pg.t_h = -INFINITY;
  pg.W = reinterpret_cast<const uint16_t*>(w->shared.w_gate_up); pg.ldw = 2L * f; pg.N = f; pg.gu_off = f;
  pg.n_tiles = mp.p1.n_tiles; pg.S = mp.p1.S; pg.cap = mp.p1.cap;
  pg.partials = m.shared.g1.partials; pg.counters = m.shared.g1.counters; pg.part_ld = 2L * f;
  const GemvConfig cr{int(AS_BF16), mt, lp.router.lpr, IN_ALL, OUT_ROUTER, false, true};
  const GemvConfig cg{int(AS_BF16), mt, mp.p1.lpr, IN_ALL, OUT_PARTS, true, true};
  size_t sm1 = gemv_smem_bytes(cr, pr.cap, 0);
  {
    const size_t b = gemv_smem_bytes(cg, pg.cap, 0);
    if (b > sm1) sm1 = b;
  }
  // launch 2, first piece: routed experts' gate/up (as in as_sparse_moe_expert)
  MoeParams pm;
  memset(&pm, 0, sizeof pm);
  pm.x = X; pm.x_dt = int(x_dt); pm.ldx = d; pm.T = T; pm.top = top_k; pm.E = E;
  pm.d_model = d; pm.d_ff = ew.d_ff_e;
  pm.keep_k = dense ? ew.d_ff_e : keep_k;
  pm.ids = ids; pm.wts = weights;
  pm.w_gu = reinterpret_cast<const uint16_t*>(ew.w_gate_up); pm.w_down = reinterpret_cast<const uint16_t*>(ew.w_down);
  pm.h = m.moe.h; pm.h_dbg = h_dbg; pm.keep_dbg = dense ? nullptr : keep_dbg;
  pm.partials = m.moe.partials; pm.counters = m.moe.counters; pm.n_tiles = moe_down_tiles(d, T * top_k);
  if (moe_select_in_gu(T * top_k, ew.d_ff_e, true)) { pm.gu_cnt = m.moe.gu_cnt; pm.keep = m.moe.keep; pm.kval = m.moe.kval; }
  if (rule.gate) {
    pm.gate_mode = 1;
    pm.gate_t = dense ? -INFINITY : rule.t_gate;
    pm.a_dbg = rule.a_dbg;
    pm.keep_k = 0; pm.keep_dbg = nullptr; pm.keep = nullptr; pm.kval = nullptr; pm.gu_cnt = nullptr;
  }
  pm.y = Y; pm.y_dt = AS_F32; pm.accumulate = 1;
  pm.atomic_y = (flags & AS_FLAG_ATOMIC_SPLITK) ? 1 : 0;
  pm.neurons_per_block = moe_npb(T * top_k);
  {
    const int es = x_dt == AS_F32 ? 4 : 2;
    pm.x_vec = aligned16(X) && (long(d) * es) % 16 == 0;
  }
  const int n_u = T * top_k < E ? T * top_k : E;
  const int n_gu = n_u * moe_gu_blocks_of(pm);
  lp.cfg.nk = moe_gu_nk_of(pm);
  // second piece: the shared expert's down projection; sums the gate/up partials of
  // its range of h, SwiGLU, every row kept; writes Y
  GemvParams pd = base_params();
  pd.M = T; pd.W = reinterpret_cast<const uint16_t*>(w->shared.w_down); pd.ldw = d;
  pd.x = m.shared.g1.partials; pd.x_dt = AS_F32; pd.K = f; pd.ldx = 2L * f; pd.t = -INFINITY;
  pd.x_parts = mp.p1.S; pd.x_up = f; pd.keep_all = 1;
  pd.list_cnt = m.shared.l_cnt; pd.list_idx = m.shared.l_idx; pd.list_val = m.shared.l_val;
  pd.n_lt = mp.n_lt; pd.lt_stride = mp.lt_stride;
  pd.N = d; pd.n_tiles = mp.p2.n_tiles; pd.S = mp.s2_range; pd.cap = mp.cap2_range;
  pd.partials = m.shared.g2.partials; pd.counters = m.shared.g2.counters; pd.part_ld = d;
  pd.y = Y; pd.y_dt = AS_F32; pd.ldy = d; pd.accumulate = 0;
  const GemvConfig cd{int(AS_BF16), mt, mp.p2.lpr, IN_PARTS, OUT_Y, false, true};
  size_t sm2 = moe_gu_smem_of(pm);
  {
    const size_t b = gemv_smem_bytes(cd, pd.cap, 0);
    if (b > sm2) sm2 = b;
  }
  if ((st = hip_check(launch_moe_route_gu(lp.cfg, pr, pg, sm1, stream), fn)) != AS_OK) return st;
  if ((st = hip_check(launch_moe_gu_down(lp.cfg, pm, n_u, n_gu, pd, sm2, stream), fn)) != AS_OK) return st;
  // launch 3: routed down stage over each (token, slot)'s keep set, added onto Y
  return hip_check(launch_moe_down(int(AS_BF16), pm, stream), fn);
}
}  // namespace

as_status as_moe_layer(const void* X, as_dtype x_dt, int T, const as_moe_layer_weights* w, int top_k, int keep_k,
                       float* Y, unsigned flags, float* logits, int32_t* ids, float* weights, float* h_dbg,
                       int32_t* keep_dbg, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  const MoeKeepRule rule{false, 0.f, nullptr};
  return moe_layer_impl("as_moe_layer", X, x_dt, T, w, top_k, keep_k, rule, Y, flags, logits, ids, weights, h_dbg,
                        keep_dbg, ws, ws_bytes, stream);
}

as_status as_moe_layer_gate(const void* X, as_dtype x_dt, int T, const as_moe_layer_weights* w, int top_k,
                            float t_gate, float* Y, unsigned flags, float* logits, int32_t* ids, float* weights,
                            float* h_dbg, float* a_dbg, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  if (std::isnan(t_gate)) return fail(AS_ERR_INVALID_ARG, "as_moe_layer_gate: t_gate is NaN");
  const MoeKeepRule rule{true, t_gate, a_dbg};
  return moe_layer_impl("as_moe_layer_gate", X, x_dt, T, w, top_k, 0, rule, Y, flags, logits, ids, weights, h_dbg,
                        nullptr, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ block glue
as_status as_rmsnorm(const void* X, as_dtype x_dt, int rows, int d, float eps, float* Y, float* copy,
                     hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_rmsnorm";
  if (!X || !Y) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!is_dt(x_dt)) return fail(AS_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (rows < 1 || d < 1 || !(eps >= 0.f)) return fail(AS_ERR_INVALID_ARG, "%s: rows=%d d=%d", fn, rows, d);
  return hip_check(launch_rmsnorm(X, int(x_dt), rows, d, eps, Y, copy, stream), fn);
}

namespace {
// Chunks of cached keys per kv head: about 64 keys each, at most about one
// workgroup per CU, but never more than attention_max_keys() keys in a chunk (0
// when the context needs more than attention_max_chunks() chunks).  The current
// token's key rides with the last chunk.
int attn_chunks(int n_ctx, int n_kv) {
  int c = (n_ctx + 63) / 64;
  const int max_c = (num_cus() + n_kv - 1) / n_kv;       // about one workgroup per CU
  if (c > max_c) c = max_c;
  const int min_c = (n_ctx + attention_max_keys() - 1) / attention_max_keys();
  if (c < min_c) c = min_c;
  if (c < 1) c = 1;
  return c > attention_max_chunks() ? 0 : c;
}
struct AttnWs {
  float* part_o;
  float* part_ml;
  unsigned* counters;
};
AttnWs carve_attn(Carver& c, int n_ctx, int n_q, int n_kv, int hd) {
  AttnWs a;
  const int C = attn_chunks(n_ctx, n_kv);
  const int grp = n_q / n_kv;
  a.part_o = c.take<float>(size_t(n_kv) * C * grp * hd);
  a.part_ml = c.take<float>(size_t(n_kv) * C * grp * 2);
  a.counters = c.take<unsigned>(size_t(n_kv) * kCounterStride);
  return a;
}
}  // namespace

size_t as_gqa_decode_attention_ws_size(int n_ctx, int n_q, int n_kv, int head_dim) {
  if (n_ctx < 0 || n_q < 1 || n_kv < 1 || head_dim < 1 || n_q % n_kv) return 0;
  Carver c{nullptr};
  carve_attn(c, n_ctx, n_q, n_kv, head_dim);
  return c.off;
}

as_status as_gqa_decode_attention(const float* q, const float* k_new, const float* v_new, const void* k_cache,
                                  const void* v_cache, as_dtype kv_dt, int n_ctx, int n_q, int n_kv, int head_dim,
                                  float* o, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_gqa_decode_attention";
  if (!q || !k_new || !v_new || !o) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (n_ctx > 0 && (!k_cache || !v_cache)) return fail(AS_ERR_INVALID_ARG, "%s: NULL cache", fn);
  if (kv_dt != AS_BF16) return fail(AS_ERR_UNSUPPORTED, "%s: caches must be bf16", fn);
  if (n_ctx < 0 || n_q < 1 || n_kv < 1 || n_q % n_kv || head_dim < 1)
    return fail(AS_ERR_INVALID_ARG, "%s: n_ctx=%d n_q=%d n_kv=%d hd=%d", fn, n_ctx, n_q, n_kv, head_dim);
  if (n_q / n_kv > attention_max_group() || head_dim != attention_head_dim())
    return fail(AS_ERR_UNSUPPORTED, "%s: group %d (max 8) or head_dim %d (must be 128)", fn, n_q / n_kv, head_dim);
  if (attn_chunks(n_ctx, n_kv) == 0)
    return fail(AS_ERR_UNSUPPORTED, "%s: n_ctx=%d above %d", fn, n_ctx,
                attention_max_chunks() * attention_max_keys() - 1);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(AS_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  Carver c{reinterpret_cast<char*>(ws)};
  AttnWs a = carve_attn(c, n_ctx, n_q, n_kv, head_dim);
  as_status st = check_ws(ws, ws_bytes, c.off);
  if (st != AS_OK) return st;
  AttnParams p;
  p.q = q; p.k_new = k_new; p.v_new = v_new;
  p.k_cache = reinterpret_cast<const uint16_t*>(k_cache); p.v_cache = reinterpret_cast<const uint16_t*>(v_cache);
  p.n_ctx = n_ctx; p.n_q = n_q; p.n_kv = n_kv; p.head_dim = head_dim;
  p.o = o; p.part_o = a.part_o; p.part_ml = a.part_ml; p.counters = a.counters;
  const int C = attn_chunks(n_ctx, n_kv);
#ifdef AS_PHASE_TIMELINE
  {
    unsigned long long* tl = g_attn_phase_buf.exchange(nullptr);
    if (tl != nullptr && size_t(n_kv) * C * 16 <= g_attn_phase_words.load()) p.phase_tl = tl;
  }
#endif
  return hip_check(launch_attention(p, C, stream), fn);
}

namespace {
struct BlockWs {
  float *xn, *qkv, *o, *h1, *xn2;
  void *ws_qkv, *ws_o, *ws_attn, *ws_mlp;
  size_t n_qkv, n_o, n_attn, n_mlp;
};
BlockWs carve_block(Carver& c, const as_block_weights* w, int n_ctx) {
  BlockWs b;
  const int d = w->mlp.d_model;
  const int nqkv = (w->n_q + 2 * w->n_kv) * w->head_dim, no = w->n_q * w->head_dim;
  b.xn = c.take<float>(d);
  b.qkv = c.take<float>(nqkv);
  b.o = c.take<float>(no);
  b.h1 = c.take<float>(d);
  b.xn2 = c.take<float>(d);
  b.n_qkv = as_threshold_gemv_ws_size(1, d, nqkv);
  b.n_o = as_threshold_gemv_ws_size(1, no, d);
  b.n_attn = as_gqa_decode_attention_ws_size(n_ctx, w->n_q, w->n_kv, w->head_dim);
  b.n_mlp = as_sparse_swiglu_mlp_ws_size(1, &w->mlp, AS_MLP_THRESHOLD);
  b.ws_qkv = c.take<char>(b.n_qkv);
  b.ws_o = c.take<char>(b.n_o);
  b.ws_attn = c.take<char>(b.n_attn);
  b.ws_mlp = c.take<char>(b.n_mlp);
  return b;
}
}  // namespace

size_t as_decoder_block_ws_size(const as_block_weights* w, int n_ctx) {
  if (!w || w->n_q < 1 || w->n_kv < 1 || w->head_dim < 1 || w->mlp.d_model < 1 || w->mlp.d_ff < 1) return 0;
  Carver c{nullptr};
  carve_block(c, w, n_ctx);
  return c.off;
}

as_status as_decoder_block(const void* X, as_dtype x_dt, const as_block_weights* w, const void* k_cache,
                           const void* v_cache, int n_ctx, const as_block_thresholds* t, float* Y, unsigned flags,
                           as_block_debug* dbg, void* ws, size_t ws_bytes, hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_decoder_block";
  if (!X || !w || !t || !Y || !w->w_qkv || !w->w_o) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  as_status st = check_mlp_weights(&w->mlp, AS_MLP_THRESHOLD, fn);
  if (st != AS_OK) return st;
  if (w->n_q < 1 || w->n_kv < 1 || w->head_dim < 1 || w->n_q % w->n_kv)
    return fail(AS_ERR_INVALID_ARG, "%s: heads %d/%d hd %d", fn, w->n_q, w->n_kv, w->head_dim);
  Carver c{reinterpret_cast<char*>(ws)};
  BlockWs b = carve_block(c, w, n_ctx);
  if ((st = check_ws(ws, ws_bytes, c.off)) != AS_OK) return st;
  const int d = w->mlp.d_model, hd = w->head_dim;
  const int nqkv = (w->n_q + 2 * w->n_kv) * hd, no = w->n_q * hd;
  const bool dense = (flags & AS_FLAG_FORCE_DENSE) != 0;
  const unsigned pass = flags & (AS_FLAG_NO_NT_LOADS | AS_FLAG_FORCE_DENSE);
  if (dbg && dbg->down_in.idx) return fail(AS_ERR_UNSUPPORTED, "%s: the down-input mask exports bits and nnz only", fn);
  // mask exports of the four thresholded inputs (nullable)
  as_mask_out* m_qkv = dbg ? &dbg->qkv_in : nullptr;
  as_mask_out* m_o = dbg ? &dbg->o_in : nullptr;
  float* xn = dbg && dbg->xn ? dbg->xn : b.xn;
  float* qkv = dbg && dbg->qkv ? dbg->qkv : b.qkv;
  float* o = dbg && dbg->o ? dbg->o : b.o;
  float* h1 = dbg && dbg->h1 ? dbg->h1 : b.h1;
  float* xn2 = dbg && dbg->xn2 ? dbg->xn2 : b.xn2;
  const float inf = -INFINITY;
  as_mlp_debug md;
  memset(&md, 0, sizeof md);
  if (dbg) {
    md.h = dbg->h;
    md.x_mask = dbg->gate_up_in;
    md.h_mask = dbg->down_in;
  }
  const bool want_md = dbg && (md.h || md.x_mask.bits || md.x_mask.idx || md.x_mask.nnz || md.h_mask.bits ||
                               md.h_mask.nnz);
  if (can_norm_in_prologue(X, x_dt, d) && can_norm_in_prologue(h1, AS_F32, d) &&
      (flags & AS_FLAG_NO_FUSION) == 0) {
    // The two RMS normalisations run in the prologues of the projections that read
    // them (qkv, and the MLP's gate/up), and the residual adds in the epilogues of
    // the o projection (h1 = X + o W_o) and of the MLP's down stage (Y = h1 + MLP):
    // five launches instead of seven, the same arithmetic order for the sums.
    GemvFuse f1;
    f1.norm = true;
    f1.xn_out = dbg ? dbg->xn : nullptr;
    if ((st = gemv_common(X, x_dt, 1, d, w->w_qkv, w->mlp.w_dt, nqkv, dense ? inf : t->qkv, qkv, AS_F32, pass,
                          m_qkv, b.ws_qkv, b.n_qkv, stream, dense, fn, &f1)) != AS_OK) return st;
    if ((st = as_gqa_decode_attention(qkv, qkv + no, qkv + no + w->n_kv * hd, k_cache, v_cache, AS_BF16, n_ctx,
                                      w->n_q, w->n_kv, hd, o, b.ws_attn, b.n_attn, stream)) != AS_OK) return st;
    GemvFuse f2;
    f2.res = X;
    f2.res_dt = int(x_dt);
    if ((st = gemv_common(o, AS_F32, 1, no, w->w_o, w->mlp.w_dt, d, dense ? inf : t->o, h1, AS_F32, pass, m_o,
                          b.ws_o, b.n_o, stream, dense, fn, &f2)) != AS_OK) return st;
    GemvFuse f3;
    f3.norm = true;
    f3.xn_out = dbg ? dbg->xn2 : nullptr;
    f3.res = h1;
    f3.res_dt = AS_F32;
    return mlp_impl(h1, AS_F32, 1, &w->mlp, AS_MLP_THRESHOLD, t->gate_up, t->down, nullptr, 0, Y, AS_F32, pass,
                    want_md ? &md : nullptr, b.ws_mlp, b.n_mlp, stream, &f3);
  }
  // AS_FLAG_NO_FUSION (or inputs the prologues cannot normalise): seven launches
  if ((st = as_rmsnorm(X, x_dt, 1, d, 1e-5f, xn, h1, stream)) != AS_OK) return st;
  if ((st = as_threshold_gemv(xn, AS_F32, 1, d, w->w_qkv, w->mlp.w_dt, nqkv, dense ? inf : t->qkv, qkv, AS_F32,
                              pass, m_qkv, b.ws_qkv, b.n_qkv, stream)) != AS_OK) return st;
  if ((st = as_gqa_decode_attention(qkv, qkv + no, qkv + no + w->n_kv * hd, k_cache, v_cache, AS_BF16, n_ctx,
                                    w->n_q, w->n_kv, hd, o, b.ws_attn, b.n_attn, stream)) != AS_OK) return st;
  if ((st = as_threshold_gemv(o, AS_F32, 1, no, w->w_o, w->mlp.w_dt, d, dense ? inf : t->o, h1, AS_F32,
                              pass | AS_FLAG_ACCUMULATE, m_o, b.ws_o, b.n_o, stream)) != AS_OK) return st;
  if ((st = as_rmsnorm(h1, AS_F32, 1, d, 1e-5f, xn2, Y, stream)) != AS_OK) return st;
  return as_sparse_swiglu_mlp(xn2, AS_F32, 1, &w->mlp, AS_MLP_THRESHOLD, t->gate_up, t->down, nullptr, 0, Y,
                              AS_F32, pass | AS_FLAG_ACCUMULATE, want_md ? &md : nullptr, b.ws_mlp, b.n_mlp, stream);
}

// ------------------------------------------------------------------ GLASS local signal
as_status as_glass_local_signal(const void* X, as_dtype x_dt, int P, const as_mlp_weights* w, float* local,
                                hipStream_t stream) {
  AS_API_RANGE();
  const char* fn = "as_glass_local_signal";
  if (!X || !w || !w->w_gate_up || !local) return fail(AS_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (P < 1 || w->d_model < 32 || w->d_ff < 16) return fail(AS_ERR_INVALID_ARG, "%s: P=%d d=%d d_ff=%d", fn, P, w->d_model, w->d_ff);
  if (x_dt != AS_BF16 || w->w_dt != AS_BF16 || w->d_model % 32 != 0)
    return fail(AS_ERR_UNSUPPORTED, "%s: needs bf16 X and weights and d_model %% 32 == 0", fn);
  if (!aligned16(X) || !aligned16(w->w_gate_up)) return fail(AS_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  const int d = w->d_model;
  return hip_check(launch_local_signal(reinterpret_cast<const uint16_t*>(X), P, d,
                                       reinterpret_cast<const uint16_t*>(w->w_gate_up), 3L * d, d, w->d_ff, local,
                                       stream), fn);
}

}  // extern "C"
