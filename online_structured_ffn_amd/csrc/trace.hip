// Measurement aids, not part of the path: opt-in kernel tracing (caller-created
// HIP events recorded around every kernel the library launches on the calling
// thread) and an HBM stream-read probe.
#include <hip/hip_runtime.h>

#include "pop_device.h"
#include "pop_internal.h"

namespace pop {

static thread_local hipEvent_t* g_trace_events = nullptr;
static thread_local int g_trace_n = 0;
static thread_local int g_trace_used = 0;

void trace_mark(void* stream) {
  if (g_trace_events == nullptr || g_trace_used >= g_trace_n) return;
  (void)hipEventRecord(g_trace_events[g_trace_used++], (hipStream_t)stream);
}

}  // namespace pop

extern "C" pop_status pop_set_trace_events(void* const* events, int32_t n_events) {
  pop::clear_error();
  if (n_events < 0 || (n_events > 0 && events == nullptr))
    return pop::fail(POP_ERR_INVALID_ARGUMENT, "events must be non-NULL when n_events > 0");
  pop::g_trace_events = n_events > 0 ? (hipEvent_t*)events : nullptr;
  pop::g_trace_n = n_events;
  pop::g_trace_used = 0;
  return POP_OK;
}

extern "C" int32_t pop_trace_recorded(void) { return pop::g_trace_used; }

// ---------------------------------------------------------------- HBM stream-read probe
// Every workgroup reads one contiguous chunk with non-temporal 16-byte loads,
// eight in flight per thread (the access pattern of the decode streams), and
// folds what it read into one word per thread so the loads cannot be dropped.
namespace pop {
__global__ __launch_bounds__(256) void k_read_probe(const u32x4* __restrict__ p, int64_t nvec, int64_t chunk,
                                                     uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const int64_t b0 = (int64_t)blockIdx.x * chunk;
  const int64_t b1 = b0 + chunk < nvec ? b0 + chunk : nvec;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = b0 + threadIdx.x; i < b1; i += 256 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + 256 * u < b1 ? i + 256 * u : b1 - 1;
      v[u] = __builtin_nontemporal_load(p + j);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}
}  // namespace pop

extern "C" pop_status pop_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                                         void* stream) {
  pop::clear_error();
  if (src == nullptr || sink == nullptr || bytes < 16 || blocks < 1 || blocks > 65536)
    return pop::fail(POP_ERR_INVALID_ARGUMENT, "src, sink non-NULL, bytes >= 16, blocks in [1, 65536] required");
  if (!pop::aligned16(src)) return pop::fail(POP_ERR_MISALIGNED, "src must be 16-byte aligned");
  const int64_t nvec = (int64_t)(bytes / 16);
  const int64_t chunk = (nvec + blocks - 1) / blocks;
  hipLaunchKernelGGL(pop::k_read_probe, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const pop::u32x4*)src, nvec, chunk, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pop::fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}
