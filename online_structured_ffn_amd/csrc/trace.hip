// Opt-in kernel tracing: caller-created HIP events recorded around every
// kernel the library launches on the calling thread.
#include <hip/hip_runtime.h>

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
