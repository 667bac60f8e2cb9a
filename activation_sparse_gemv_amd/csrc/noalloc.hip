// as_sparse_swiglu_mlp_noalloc: the sparse SwiGLU MLP for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its workspace is `scratch`, a file-scope
// device array of kScratchBytes that every GPU the library runs on holds until
// the process ends; its address on each device is resolved once with
// hipGetSymbolAddress (the array's name is a host-side stand-in, never passed to
// a kernel).  The call then runs as_sparse_swiglu_mlp with that memory as its
// workspace: the same kernels, plan and bits.
#include <cstdio>
#include <mutex>

#include "internal.hpp"
#include "api_range.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB per device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  void* ptr = nullptr;     // device address of `scratch` on this device
  uint64_t layout = 0;     // carve-up of the last call (0: none yet)
};
DeviceScratch g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The workspace carve-up is a function of these arguments (the launch plan depends
// on the shapes and the device only).
uint64_t layout_key(int M, const as_mlp_weights* w, as_mlp_mode mode) {
  uint64_t k = 1469598103934665603ull;
  const uint64_t parts[5] = {uint64_t(M), uint64_t(w->d_model), uint64_t(w->d_ff), uint64_t(mode), uint64_t(w->w_dt)};
  for (uint64_t v : parts) k = (k ^ v) * 1099511628211ull;
  return k | 1ull;
}

}  // namespace

extern "C" as_status as_sparse_swiglu_mlp_noalloc(const void* X, as_dtype x_dt, int M, const as_mlp_weights* w,
                                                  as_mlp_mode mode, float t_x, float t_h, const int32_t* neuron_idx,
                                                  int n_active, void* Y, as_dtype y_dt, unsigned flags,
                                                  as_mlp_debug* dbg, hipStream_t stream) {
  AS_API_RANGE();
  char msg[256];
  if (!w || M < 1) return as::report_error(AS_ERR_INVALID_ARG, "as_sparse_swiglu_mlp_noalloc: NULL weights or M < 1");
  const size_t need = as_sparse_swiglu_mlp_ws_size(M, w, mode);
  if (need > kScratchBytes) {
    snprintf(msg, sizeof msg,
             "as_sparse_swiglu_mlp_noalloc: M=%d d_model=%d d_ff=%d needs %zu bytes of scratch, above the %zu-byte "
             "static array (use as_sparse_swiglu_mlp with a workspace)", M, w->d_model, w->d_ff, need, kScratchBytes);
    return as::report_error(AS_ERR_UNSUPPORTED, msg);
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return as::report_error(AS_ERR_HIP, "as_sparse_swiglu_mlp_noalloc: no current device");
  void* ptr = nullptr;
  bool clear = false;
  const uint64_t key = layout_key(M, w, mode);
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    DeviceScratch& ds = g_scratch[dev];
    if (ds.ptr == nullptr) {
      // set-up, once per device, with that device current
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        snprintf(msg, sizeof msg, "as_sparse_swiglu_mlp_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        return as::report_error(AS_ERR_HIP, msg);
      }
      ds.ptr = p;
    }
    ptr = ds.ptr;
    // Every call leaves its counters at zero, but a call of another shape carves the
    // array differently (its partials may lie where this call keeps counters): the
    // bytes this call uses are cleared whenever the carve-up changes, and on the
    // device's first call.
    if (ds.layout != key) {
      clear = true;
      ds.layout = key;
    }
  }
  if (clear && need > 0) {
    const hipError_t e = as::launch_fill_zero(ptr, need, stream);
    if (e != hipSuccess) {
      snprintf(msg, sizeof msg, "as_sparse_swiglu_mlp_noalloc: clearing scratch: %s", hipGetErrorString(e));
      return as::report_error(AS_ERR_HIP, msg);
    }
  }
  return as_sparse_swiglu_mlp(X, x_dt, M, w, mode, t_x, t_h, neuron_idx, n_active, Y, y_dt, flags, dbg, ptr,
                              kScratchBytes, stream);
}
