// Periodic candidate refresh with an activation memory: the batch-wise
// pruning page ("Batch-wise adaptive pruning ... for language reasoning
// models", figure 1 and figure 2(b)) refreshes its mask by a top-k only every
// few steps and carries importance to the next refresh in an activation
// memory; its own definition is cut off in the pages, so it is read into POP's
// candidate set:
//   * step t refreshes when t % period == 0: gate/up over R u C, every
//     candidate's score (max over the batch of |z|) is added to the memory,
//     the k candidates of highest memory are selected (ties to the lower
//     position), the memory is cleared, and the down-projection runs over R
//     plus the selection;
//   * the other steps compute R plus the kept selection only (the step of
//     pop_decode_ffn with R followed by the selection, a list the refresh
//     writes, as its retained rows and no candidates), and add the selected
//     candidates' scores (max over the batch of |z|, read from that step's z)
//     to their memory.
// A refresh is composed from the stage entry points (gate/up, select, down);
// small kernels keep the memory and build the kept step's row list; nothing
// synchronises with the host.
#include <hip/hip_runtime.h>

#include "pop_device.h"
#include "pop_internal.h"

namespace pop {

__global__ __launch_bounds__(256) void k_mem_add(float* __restrict__ memory, const float* __restrict__ score, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) memory[i] += score[i];
}

__global__ __launch_bounds__(256) void k_mem_clear(float* __restrict__ memory, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) memory[i] = 0.f;
}

// memory[positions[j]] += score[j]: the positions of a selection are distinct
// memory[positions[j]] += max over the batch of |z[b][n_R + j]| (z rows of n_A values)
__global__ __launch_bounds__(256) void k_mem_add_z(float* __restrict__ memory, const int32_t* __restrict__ positions,
                                                   const float* __restrict__ z, int batch, int n_A, int n_R, int k,
                                                   int n_C) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= k) return;
  float m = 0.f;
  for (int b = 0; b < batch; ++b) m = fmaxf(m, fabsf(z[(int64_t)b * n_A + n_R + j]));
  const int p = positions[j];
  if (p >= 0 && p < n_C) memory[p] += m;
}

// rows = R followed by the selection
__global__ __launch_bounds__(256) void k_concat(int32_t* __restrict__ rows, const int32_t* __restrict__ R, int n_R,
                                                const int32_t* __restrict__ sel, int k) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n_R) rows[i] = R[i];
  else if (i < n_R + k) rows[i] = sel[i - n_R];
}

struct PeriodicWs {
  float* z;        // refresh: z over R u C
  float* score;    // refresh: candidate scores
  int32_t* rows;   // an empty R's stand-in (never read)
  char* down;      // refresh: the down-projection's workspace
  size_t down_bytes;
  char* step;      // kept step: pop_decode_ffn's workspace
  size_t step_bytes;
  size_t bytes;
};

static PeriodicWs periodic_ws(int32_t batch, int32_t d, int32_t d_ff, char* base) {
  PeriodicWs w;
  const size_t zb = align_up((size_t)(batch > 0 ? batch : 1) * d_ff * sizeof(float), 256);
  const size_t sb = align_up((size_t)d_ff * sizeof(float), 256);
  const size_t ib = align_up((size_t)d_ff * sizeof(int32_t), 256);
  w.down_bytes = align_up(pop_decode_down_workspace_bytes(batch, d, d_ff), 256);
  w.step_bytes = pop_decode_workspace_bytes(batch, d, d_ff);
  w.z = base ? (float*)base : nullptr;
  w.score = base ? (float*)(base + zb) : nullptr;
  w.rows = base ? (int32_t*)(base + zb + sb) : nullptr;
  w.down = base ? base + zb + sb + ib : nullptr;
  w.step = base ? base + zb + sb + ib + w.down_bytes : nullptr;
  w.bytes = zb + sb + ib + w.down_bytes + w.step_bytes;
  return w;
}

static dim3 blocks_for(int n) { return dim3((unsigned)((n + 255) / 256 > 0 ? (n + 255) / 256 : 1)); }

static pop_status launched_ok() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}

}  // namespace pop

using namespace pop;

extern "C" size_t pop_decode_periodic_workspace_bytes(int32_t batch, int32_t d, int32_t d_ff) {
  if (batch < 0 || d <= 0 || d_ff <= 0) return 0;
  return periodic_ws(batch, d, d_ff, nullptr).bytes;
}

extern "C" pop_status pop_decode_ffn_periodic(const void* x, int32_t batch, int32_t d, const void* W_gate,
                                              const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                              const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, double r,
                                              int32_t step, int32_t period, float* memory, int32_t* positions,
                                              int32_t* selected, int32_t* rows, float* y, void* ws, size_t ws_bytes,
                                              void* stream) {
  clear_error();
  // the shape checks of the decode entry points: the batch-1 steps below
  // launch their kernels directly
  if (const pop_status sc = check_dtype_width(dt, d); sc != POP_OK) return sc;
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (batch < 0 || batch > POP_MAX_BATCH) return fail(POP_ERR_BAD_SHAPE, "batch=%d outside [0, %d]", batch, POP_MAX_BATCH);
  if (period < 1) return fail(POP_ERR_INVALID_ARGUMENT, "period=%d must be at least 1", period);
  if (step < 0) return fail(POP_ERR_INVALID_ARGUMENT, "step=%d must be non-negative", step);
  if (!(r >= 0.0 && r < 1.0)) return fail(POP_ERR_INVALID_ARGUMENT, "r=%g outside [0, 1)", r);
  if (n_R < 0 || n_C < 0 || (int64_t)n_R + n_C > d_ff || d_ff < 1)
    return fail(POP_ERR_INVALID_ARGUMENT, "n_R=%d, n_C=%d inconsistent with d_ff=%d", n_R, n_C, d_ff);
  const int32_t k = topk_count(d_ff, r, n_R, n_C);
  if ((n_R > 0 && R == nullptr) || (n_C > 0 && C == nullptr) ||
      (k > 0 && (memory == nullptr || positions == nullptr || selected == nullptr)) ||
      (n_R + k > 0 && rows == nullptr) || ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "R, C, memory, positions, selected, rows and ws must be non-NULL");
  if (kDebugLists) {
    const pop_status sd = debug_check_device_lists(R, n_R, C, n_C, d_ff, stream);
    if (sd != POP_OK) return sd;
  }
  const DebugNested nest;  // the calls below pass the retained rows (R, then the selection)
  if ((batch > 0 && (x == nullptr || y == nullptr)) || W_gate == nullptr || W_up == nullptr || W_downT == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "x, y and the weights must be non-NULL");
  if (!aligned16(ws)) return fail(POP_ERR_MISALIGNED, "ws must be 16-byte aligned");
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_downT) || !aligned16(y))
    return fail(POP_ERR_MISALIGNED, "x, y and the weights must be 16-byte aligned");
  const PeriodicWs w0 = periodic_ws(batch, d, d_ff, nullptr);
  if (ws_bytes < w0.bytes) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, w0.bytes);
  const PeriodicWs w = periodic_ws(batch, d, d_ff, (char*)ws);
  hipStream_t st = (hipStream_t)stream;
  // an empty R is passed as a non-NULL list (NULL would mean the identity rows)
  const int32_t* Rk = R != nullptr ? R : w.rows;
  pop_status s;
  if (step % period == 0) {  // refresh
    // batch 1: the single-launch step ranks the candidates by memory + |z|
    // itself (and clears the memory); the retained rows for the kept steps follow
    if (batch == 1 && n_C > 0 && k > 0 &&
        decode_periodic_refresh_b1(x, d, W_gate, W_up, W_downT, d_ff, dt, Rk, n_R, C, n_C, k, memory, positions,
                                   selected, y, w.step, stream)) {
      POP_LAUNCH(k_concat, blocks_for(n_R + k), dim3(256), 0, st, rows, Rk, n_R, (const int32_t*)selected, k);
      return launched_ok();
    }
    if ((s = pop_decode_gateup(x, batch, d, W_gate, W_up, d_ff, dt, Rk, n_R, C, n_C, w.z, w.score, stream)) != POP_OK)
      return s;
    if (n_C > 0 && k > 0) {
      POP_LAUNCH(k_mem_add, blocks_for(n_C), dim3(256), 0, st, memory, (const float*)w.score, n_C);
      if ((s = pop_decode_select(memory, n_C, C, k, positions, selected, stream)) != POP_OK) return s;
    }
    if (n_C > 0 && memory != nullptr) POP_LAUNCH(k_mem_clear, blocks_for(n_C), dim3(256), 0, st, memory, n_C);
    // the kept steps' retained rows: R, then the selection
    if (n_R + k > 0)
      POP_LAUNCH(k_concat, blocks_for(n_R + k), dim3(256), 0, st, rows, Rk, n_R, (const int32_t*)selected, k);
    return pop_decode_down(w.z, batch, n_R + n_C, W_downT, d, d_ff, dt, Rk, n_R, selected, positions, k, y, w.down,
                           w.down_bytes, stream);
  }
  // between refreshes: the step over R plus the kept selection as retained
  // rows (no candidates), whose z of the selected rows joins the memory
  if (batch == 1 && k > 0 && n_C > 0 &&
      decode_periodic_kept_b1(x, d, W_gate, W_up, W_downT, d_ff, dt, rows, n_R, k, memory, positions, n_C, y, w.step,
                              stream))
    return launched_ok();
  if ((s = pop_decode_ffn(x, batch, d, W_gate, W_up, W_downT, d_ff, dt, n_R + k > 0 ? rows : w.rows, n_R + k,
                          nullptr, 0, r, y, nullptr,
                          w.step, w.step_bytes, stream)) != POP_OK)
    return s;
  if (k > 0 && batch > 0)
    POP_LAUNCH(k_mem_add_z, blocks_for(k), dim3(256), 0, st, memory, (const int32_t*)positions,
               (const float*)decode_ws_z(w.step, batch, d, d_ff), batch, n_R + k, n_R, k, n_C);
  return launched_ok();
}
