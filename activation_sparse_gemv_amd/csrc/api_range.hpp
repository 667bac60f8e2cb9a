// Named ranges around the C entry points, for tracing: rocprofv3 --marker-trace
// shows each call of the library as a range with the entry point's name, with the
// kernels it launched inside it (nested calls nest).  Without a profiler attached
// the push and pop return at once.
#pragma once
#include <rocprofiler-sdk-roctx/roctx.h>

namespace as {

struct ApiRange {
  explicit ApiRange(const char* name) { roctxRangePushA(name); }
  ~ApiRange() { roctxRangePop(); }
  ApiRange(const ApiRange&) = delete;
  ApiRange& operator=(const ApiRange&) = delete;
};

}  // namespace as

#define AS_API_RANGE() const ::as::ApiRange as_api_range_(__func__)
