// Host-side helpers shared by the library's entry points: pointer checks,
// launch status, grid sizing and the launch tracer behind flce_trace_*.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "../../include/flce.h"

namespace flce {
namespace host {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// FLCE_OK, or FLCE_ERR_HIP (with a message) if a launch failed.
inline int launch_status() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    fprintf(stderr, "flce: HIP launch failed: %s\n", hipGetErrorString(e));
    return FLCE_ERR_HIP;
  }
  return FLCE_OK;
}

// Blocks for n items at per_block each, clamped to [1, cap].
inline unsigned grid_for(int64_t n, int64_t per_block, int64_t cap) {
  int64_t g = ceil_div(n, per_block);
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

// Launch tracing (flce_trace_*): (start, end) event pairs around launches.
// One process-wide instance, defined in flce.hip.
struct Tracer {
  bool on = false;
  uint32_t mask = 0xFFFFFFFFu;  // kinds recorded (bit 1 << kind)
  int cap = 0;
  int n = 0;
  std::vector<hipEvent_t> ev;
  std::vector<int> kind;
  std::vector<double> flops;
  void release() {
    for (hipEvent_t e : ev) hipEventDestroy(e);
    ev.clear();
    kind.clear();
    flops.clear();
    cap = n = 0;
    on = false;
  }
};
extern Tracer g_trace;

// Brackets one launch with trace events when a trace is running.
struct TraceScope {
  int slot = -1;
  hipStream_t s;
  TraceScope(int kind, double flops, hipStream_t stream) : s(stream) {
    if (!g_trace.on || g_trace.n >= g_trace.cap || !((g_trace.mask >> kind) & 1u)) return;
    slot = g_trace.n++;
    g_trace.kind[slot] = kind;
    g_trace.flops[slot] = flops;
    hipEventRecord(g_trace.ev[2 * slot], s);
  }
  ~TraceScope() {
    if (slot >= 0) hipEventRecord(g_trace.ev[2 * slot + 1], s);
  }
};

}  // namespace host
}  // namespace flce
