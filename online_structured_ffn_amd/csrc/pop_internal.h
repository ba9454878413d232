// Host-side helpers shared by the libpop translation units (no device code).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/pop.h"

namespace pop {

// Records a message for pop_last_error() and returns s.
pop_status fail(pop_status s, const char* fmt, ...);
// Clears the thread's last error.
void clear_error();
// pop_partition_counts without argument validation of `out`.
pop_counts counts(int32_t d_ff, double r, double gamma);
// Live count and per-step k for an existing partition.
int32_t live_count(int32_t d_ff, double r);
int32_t topk_count(int32_t d_ff, double r, int32_t n_R, int32_t n_C);

bool aligned16(const void* p);
int elem_bytes(pop_dtype dt);
// Checks dtype and that d suits the 16-byte vector width of dt.
pop_status check_dtype_width(pop_dtype dt, int64_t d);
pop_status check_rate(double r, double gamma);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// pop_check_lists on copies of the device lists R and C (R == NULL: the
// identity, not checked), copied on `stream` (a hipStream_t) and waited for.
// Called by the entry points that take R and C only in builds with POP_DEBUG
// defined (defined in decode.hip).
pop_status debug_check_device_lists(const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, int32_t d_ff,
                                    void* stream);
// Entry points calling other entry points on this thread: the debug check
// runs at the outermost call only, since an inner call may get lists the
// library built itself (retained rows followed by the selection, say) that
// need not be ascending.  A DebugNested object marks its scope as inner.
int& debug_nesting();
struct DebugNested {
  DebugNested() { ++debug_nesting(); }
  ~DebugNested() { --debug_nesting(); }
  DebugNested(const DebugNested&) = delete;
  DebugNested& operator=(const DebugNested&) = delete;
};
#ifdef POP_DEBUG
constexpr bool kDebugLists = true;
#else
constexpr bool kDebugLists = false;
#endif

// Prefill pieces shared with the fused prefill FFN (defined in prefill.hip;
// stream is a hipStream_t).  colsq_ws_bytes sizes the column-norm workspace
// (partial sums, then s2); launch_colsq writes s2 = sum over the prompt rows of
// X^2 into that workspace and returns it; launch_partition_lists launches the
// one-workgroup select and compaction into R, C, P.
size_t colsq_ws_bytes(int64_t n_tokens, int32_t d);
float* launch_colsq(void* stream, const void* X, int64_t n_tokens, int32_t d, pop_dtype dt, char* ws);
void launch_partition_lists(void* stream, const float* I, int32_t d_ff, int32_t c_low, int32_t c_high, int32_t* R,
                            int32_t* C, int32_t* P);

// Where pop_decode_ffn leaves z in its workspace (batch rows of the step's
// live R u C columns, R first; defined in decode.hip).
float* decode_ws_z(void* ws, int32_t batch, int32_t d, int32_t d_ff);

// pop_decode_ffn (or, with dense, pop_dense_ffn_decode) at batch 1 with
// y += FFN(x) instead of y = FFN(x), for a caller that adds the FFN to a
// residual stream; the caller has validated the arguments and ws holds
// pop_decode_workspace_bytes(1, d, d_ff).  Returns false, having enqueued
// nothing, when the step does not take the fused three-launch path (defined
// in decode.hip).
bool decode_ffn_accumulate_b1(const void* x, int32_t d, const void* W_gate, const void* W_up, const void* W_downT,
                              int32_t d_ff, pop_dtype dt, bool dense, const int32_t* R, int32_t n_R,
                              const int32_t* C, int32_t n_C, double r, float* y, int32_t* selected, void* ws,
                              void* stream);
// A kept step of the periodic mode at batch 1: the retained rows rows[0 ..
// n_R + k) (R, then the selection) in the fused stream, and the memory update
// memory[positions[j]] += |z of row n_R + j| in the step's last launch.
// Returns false, having launched nothing, when that form does not apply.
bool decode_periodic_kept_b1(const void* x, int32_t d, const void* W_gate, const void* W_up, const void* W_downT,
                             int32_t d_ff, pop_dtype dt, const int32_t* rows, int32_t n_R, int32_t k, float* memory,
                             const int32_t* positions, int32_t n_C, float* y, void* ws, void* stream);
// The refresh step of the periodic mode at batch 1 in the single-launch form:
// the candidates ranked by memory + |z| (memory [n_C] is read and cleared),
// the k best written to positions (into C) and selected (channels), y the
// FFN over R and them; ws a batch-1 decode workspace.  Returns false, having
// launched nothing, when that form does not apply (the caller then takes the
// staged calls).
bool decode_periodic_refresh_b1(const void* x, int32_t d, const void* W_gate, const void* W_up, const void* W_downT,
                                int32_t d_ff, pop_dtype dt, const int32_t* R, int32_t n_R, const int32_t* C,
                                int32_t n_C, int32_t k, float* memory, int32_t* positions, int32_t* selected, float* y,
                                void* ws, void* stream);

// Records the next caller-provided trace event on `stream` (no-op unless
// pop_set_trace_events armed this thread).
void trace_mark(void* stream);

// hipLaunchKernelGGL followed by a trace mark on the same stream.
#define POP_LAUNCH(kernel, grid, block, shmem, stream, ...)                  \
  do {                                                                        \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);      \
    ::pop::trace_mark((void*)(stream));                                       \
  } while (0)

}  // namespace pop
