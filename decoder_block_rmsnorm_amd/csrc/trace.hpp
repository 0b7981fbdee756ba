// Host-side tracing aids of the library (no effect on what is computed):
//
//  * TraceRange: a roctx range around each entry point call (llama_block_prefill,
//    llama_block_decode, llama_stack_generate, ...), so that a marker trace
//    (rocprofv3 --marker-trace) groups the kernels of one call under its name.
//    Without a profiler attached a range costs two calls into an empty table.
//  * plan_log: with the environment variable LLAMA_LOG set to a value other
//    than 0, every launch plan the library picks (GEMM tile shape and split,
//    attention grid and key splits, the 4-bit kernel variant) is printed to
//    stderr, one line per launch, prefixed "[llama]".  Off by default; the
//    variable is read once per process.
#pragma once
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>

namespace lb {

inline bool plan_log_on() {
  static const bool on = [] {
    const char* v = std::getenv("LLAMA_LOG");
    return v && *v && !(v[0] == '0' && v[1] == 0);
  }();
  return on;
}

__attribute__((format(printf, 1, 2))) inline void plan_log(const char* fmt, ...) {
  if (!plan_log_on()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[llama] %s\n", buf);
}

struct TraceRange {
  explicit TraceRange(const char* name) { roctxRangePushA(name); }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

}  // namespace lb
