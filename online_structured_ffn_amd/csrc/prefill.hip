// Prefill three-region partition (POP notes, "Key design 1").
//
//   K1  column sum of squares  s2[k] = sum_n X[n,k]^2         (HBM-bound on X)
//   K1r fixed-order reduction of the K1 partial sums
//   K2  importance  I[i] = sqrt(sum_k W_up[i,k]^2 * s2[k])    (HBM-bound on W_up)
//   K3  one-workgroup radix select of the keys at ranks c_low and c_high and an
//       order-preserving compaction into P, C, R            (latency-bound)
#include <hip/hip_runtime.h>

#include "moe_route.h"
#include "pop_device.h"
#include "pop_internal.h"

namespace pop {

// ---------------------------------------------------------------- K1
// Block: 64 threads (one wave); thread t owns the Vec<T>::N columns starting at
// (blockIdx.x*64 + t)*N; blockIdx.y is a chunk of rows.  Each wave reads whole
// 16-byte vectors of consecutive columns of one row per instruction (1 KB of
// bf16 per row per wave, coalesced).
template <typename T>
__global__ __launch_bounds__(64) void k_colsq_partial(const T* __restrict__ X, int64_t n_tokens, int d,
                                                      int64_t rows_per_chunk, float* __restrict__ partial) {
  constexpr int V = Vec<T>::N;
  const int col = (blockIdx.x * 64 + threadIdx.x) * V;
  if (col >= d) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  int64_t r1 = r0 + rows_per_chunk;
  if (r1 > n_tokens) r1 = n_tokens;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  const T* p = X + col;
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    u32x4 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = ld16_stream(p + (r + j) * d);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float f[V];
      unpack(q[j], f, T{});
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = fmaf(f[v], f[v], acc[v]);
    }
  }
  for (; r < r1; ++r) {
    float f[V];
    unpack(ld16_stream(p + r * d), f, T{});
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = fmaf(f[v], f[v], acc[v]);
  }
  float* out = partial + (int64_t)blockIdx.y * d + col;
#pragma unroll
  for (int v = 0; v < V; ++v) out[v] = acc[v];
}

// ---------------------------------------------------------------- K1, MoE
// The column sums of squares of every expert in one pass over X: row r adds
// its squares to the accumulators of its two experts ex[2r], ex[2r + 1].  The
// accumulators live in LDS, [E][64 threads][V] (each thread's own slots).
// partial is [chunk][E][d].
template <typename T>
__global__ __launch_bounds__(64) void k_moe_colsq_partial(const T* __restrict__ X, int64_t n_tokens, int d,
                                                          const int32_t* __restrict__ ex, int E,
                                                          int64_t rows_per_chunk, float* __restrict__ partial) {
  constexpr int V = Vec<T>::N;
  extern __shared__ float acc_lds[];
  const int tid = threadIdx.x;
  const int col = (blockIdx.x * 64 + tid) * V;
  const bool on = col < d;
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int v = 0; v < V; ++v) acc_lds[(e * 64 + tid) * V + v] = 0.f;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = min(n_tokens, r0 + rows_per_chunk);
  if (on) {
    for (int64_t r = r0; r < r1; ++r) {
      const int e1 = ex[2 * r], e2 = ex[2 * r + 1];
      float f[V];
      unpack(ld16_stream(X + r * d + col), f, T{});
      float* a1 = acc_lds + (e1 * 64 + tid) * V;
      float* a2 = acc_lds + (e2 * 64 + tid) * V;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float q = f[v] * f[v];
        a1[v] += q;
        a2[v] += q;
      }
    }
    for (int e = 0; e < E; ++e) {
      float* out = partial + ((int64_t)blockIdx.y * E + e) * d + col;
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] = acc_lds[(e * 64 + tid) * V + v];
    }
  }
}

// ---------------------------------------------------------------- K2
// Block: 256 threads = 4 waves, one W_up row per wave at a time.  s2 sits in
// LDS; each lane reads 16-byte vectors of its row, 4 in flight.
// blockIdx.y selects an expert (MoE): its W_up, s2 and I follow the previous
// expert's contiguously; gridDim.y = 1 otherwise.
template <typename T>
__global__ __launch_bounds__(256) void k_importance(const T* __restrict__ W, int d_ff, int d,
                                                    const float* __restrict__ s2, float* __restrict__ I) {
  constexpr int V = Vec<T>::N;
  extern __shared__ float s2_lds[];
  W += (int64_t)blockIdx.y * d_ff * d;
  s2 += (int64_t)blockIdx.y * d;
  I += (int64_t)blockIdx.y * d_ff;
  for (int k = threadIdx.x; k < d; k += 256) s2_lds[k] = s2[k];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int STEP = 64 * V;
  for (int row = blockIdx.x * 4 + wave; row < d_ff; row += gridDim.x * 4) {
    const T* w = W + (int64_t)row * d;
    float acc = 0.f;
    int k0 = 0;
    for (; k0 + 4 * STEP <= d; k0 += 4 * STEP) {
      u32x4 q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) q[j] = ld16_stream(w + k0 + j * STEP + lane * V);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float f[V];
        unpack(q[j], f, T{});
        const float* sp = s2_lds + k0 + j * STEP + lane * V;
#pragma unroll
        for (int v = 0; v < V; ++v) acc = fmaf(f[v] * f[v], sp[v], acc);
      }
    }
    for (; k0 < d; k0 += STEP) {
      const int k = k0 + lane * V;
      if (k < d) {
        float f[V];
        unpack(ld16_stream(w + k), f, T{});
#pragma unroll
        for (int v = 0; v < V; ++v) acc = fmaf(f[v] * f[v], s2_lds[k + v], acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) I[row] = sqrtf(acc);
  }
}

// ---------------------------------------------------------------- K3
constexpr int kPartThreads = 1024;

// blockIdx.x selects an expert (MoE): its I and lists follow the previous
// expert's contiguously; one block otherwise.
__global__ __launch_bounds__(kPartThreads) void k_partition(const float* __restrict__ I, int n, int c_low, int c_high,
                                                           int32_t* __restrict__ R, int32_t* __restrict__ C,
                                                           int32_t* __restrict__ P) {
  __shared__ SelShared<kPartThreads> sh;
  I += (int64_t)blockIdx.x * n;
  R += (int64_t)blockIdx.x * (n - c_high);
  C += (int64_t)blockIdx.x * (c_high - c_low);
  P += (int64_t)blockIdx.x * c_low;
  sel_load(I, n, sh);
  const int ranks[2] = {c_low, c_high};
  select_thresholds(n, ranks, sh);
  const SelTarget lo = sh.tgt[0];
  const SelTarget hi = sh.tgt[1];
  const int E = (n + kPartThreads - 1) / kPartThreads;
  const int base = threadIdx.x * E;
  const int end = min(n, base + E);
  int pos[3] = {0, 0, 0};  // P, C, R
  for (int i = base; i < end; ++i) {
    const unsigned long long key = sel_key(sh.vals[i], i);
    if (sel_less(lo, key)) ++pos[0];
    else if (sel_less(hi, key)) ++pos[1];
    else ++pos[2];
  }
  int tot[3];
  block_exclusive_scan3(pos, tot, sh);
  // Positions are capped at the list sizes the host derived from the counts;
  // an exact select never reaches the caps.
  const int n_P = c_low, n_C = c_high - c_low, n_R = n - c_high;
  for (int i = base; i < end; ++i) {
    const unsigned long long key = sel_key(sh.vals[i], i);
    if (sel_less(lo, key)) {
      if (pos[0] < n_P) P[pos[0]] = i;
      ++pos[0];
    } else if (sel_less(hi, key)) {
      if (pos[1] < n_C) C[pos[1]] = i;
      ++pos[1];
    } else {
      if (pos[2] < n_R) R[pos[2]] = i;
      ++pos[2];
    }
  }
}

// ---------------------------------------------------------------- host
struct PrefillPlan {
  int64_t rows_per_chunk;
  int n_chunks;
  int col_blocks;
};

static PrefillPlan plan_prefill(int64_t n_tokens, int32_t d, int vec) {
  PrefillPlan p;
  p.col_blocks = (d + 64 * vec - 1) / (64 * vec);
  // About 2048 single-wave blocks, at least 16 rows per chunk, at most 512 chunks.
  int64_t want_chunks = (2048 + p.col_blocks - 1) / p.col_blocks;
  int64_t max_chunks = (n_tokens + 15) / 16;
  if (want_chunks > max_chunks) want_chunks = max_chunks;
  if (want_chunks > 512) want_chunks = 512;
  if (want_chunks < 1) want_chunks = 1;
  p.rows_per_chunk = (n_tokens + want_chunks - 1) / want_chunks;
  if (p.rows_per_chunk < 1) p.rows_per_chunk = 1;
  p.n_chunks = (int)((n_tokens + p.rows_per_chunk - 1) / p.rows_per_chunk);
  if (p.n_chunks < 1) p.n_chunks = 1;
  return p;
}

static size_t importance_ws_bytes(int64_t n_tokens, int32_t d) {
  // Widest plan over both dtypes (bf16 has fewer column blocks, hence more chunks).
  const PrefillPlan p = plan_prefill(n_tokens, d, 8);
  const PrefillPlan q = plan_prefill(n_tokens, d, 4);
  const int chunks = p.n_chunks > q.n_chunks ? p.n_chunks : q.n_chunks;
  return align_up((size_t)chunks * d * sizeof(float), 256)  // partial sums
         + align_up((size_t)d * sizeof(float), 256);        // s2
}

template <typename T>
static void launch_importance(hipStream_t st, const void* X, int64_t n_tokens, int32_t d, const void* W_up,
                              int32_t d_ff, float* I, char* ws) {
  const PrefillPlan p = plan_prefill(n_tokens, d, Vec<T>::N);
  const PrefillPlan pb = plan_prefill(n_tokens, d, 8), pf = plan_prefill(n_tokens, d, 4);
  const int max_chunks = pb.n_chunks > pf.n_chunks ? pb.n_chunks : pf.n_chunks;
  float* partial = (float*)ws;
  float* s2 = (float*)(ws + align_up((size_t)max_chunks * d * sizeof(float), 256));
  if (n_tokens > 0)
    POP_LAUNCH(k_colsq_partial<T>, dim3(p.col_blocks, p.n_chunks), dim3(64), 0, st, (const T*)X, n_tokens,
                       d, p.rows_per_chunk, partial);
  // With no prompt token the sum runs over zero chunks: s = 0, hence I = 0.
  POP_LAUNCH(k_sum_chunks<0>, dim3((d + 31) / 32), dim3(1024), 0, st, (const float*)partial,
                     n_tokens > 0 ? p.n_chunks : 0, (int64_t)d, s2, (unsigned int*)nullptr, 0);
  POP_LAUNCH(k_importance<T>, dim3((d_ff + 3) / 4), dim3(256), (size_t)d * sizeof(float), st, (const T*)W_up,
                     d_ff, d, (const float*)s2, I);
}

// ---- MoE prefill
struct MoePrefillPlan {
  int64_t rows_per_chunk;
  int n_chunks;
  int col_blocks;
};

// About 1024 single-wave blocks over all experts' accumulators in one pass.
static MoePrefillPlan plan_moe_prefill(int64_t n_tokens, int32_t d, int vec) {
  MoePrefillPlan p;
  p.col_blocks = (d + 64 * vec - 1) / (64 * vec);
  int64_t want = (1024 + p.col_blocks - 1) / p.col_blocks;
  const int64_t by_rows = (n_tokens + 15) / 16;
  if (want > by_rows) want = by_rows;
  if (want < 1) want = 1;
  p.rows_per_chunk = (n_tokens + want - 1) / want;
  if (p.rows_per_chunk < 1) p.rows_per_chunk = 1;
  p.n_chunks = (int)((n_tokens + p.rows_per_chunk - 1) / p.rows_per_chunk);
  if (p.n_chunks < 1) p.n_chunks = 1;
  return p;
}

struct MoePrefillWs {
  int32_t* ex;
  float* partial;
  float* s2;
  float* I;
  size_t bytes;
};

static MoePrefillWs moe_prefill_ws(int64_t n_tokens, int32_t d, int32_t d_ff, int32_t E, char* base) {
  const MoePrefillPlan pb = plan_moe_prefill(n_tokens, d, 8), pf = plan_moe_prefill(n_tokens, d, 4);
  const int chunks = pb.n_chunks > pf.n_chunks ? pb.n_chunks : pf.n_chunks;
  MoePrefillWs w;
  size_t o = 0;
  w.ex = (int32_t*)(base + o);
  o += align_up((size_t)(2 * n_tokens > 0 ? 2 * n_tokens : 1) * 4, 256);
  w.partial = (float*)(base + o);
  o += align_up((size_t)chunks * E * d * 4, 256);
  w.s2 = (float*)(base + o);
  o += align_up((size_t)E * d * 4, 256);
  w.I = (float*)(base + o);
  o += align_up((size_t)E * d_ff * 4, 256);
  w.bytes = o;
  return w;
}

template <typename T>
static void launch_moe_prefill(hipStream_t st, const void* X, int64_t n_tokens, int32_t d, const float* logits,
                               int32_t E, const void* W_up, int32_t d_ff, const pop_counts& c, int32_t* R,
                               int32_t* C, int32_t* P, float* I, const MoePrefillWs& w) {
  const MoePrefillPlan p = plan_moe_prefill(n_tokens, d, Vec<T>::N);
  if (n_tokens > 0) {
    POP_LAUNCH(k_moe_top2<0>, dim3((unsigned)((n_tokens + 255) / 256)), dim3(256), 0, st, logits, (int)n_tokens,
               (int)E, w.ex, (float*)nullptr);
    POP_LAUNCH(k_moe_colsq_partial<T>, dim3(p.col_blocks, p.n_chunks), dim3(64),
               (size_t)E * 64 * Vec<T>::N * sizeof(float), st, (const T*)X, n_tokens, d, (const int32_t*)w.ex,
               (int)E, p.rows_per_chunk, w.partial);
  }
  // An expert that no prompt token reaches gets s = 0, hence I = 0 (index order).
  POP_LAUNCH(k_sum_chunks<0>, dim3((unsigned)(((int64_t)E * d + 31) / 32)), dim3(1024), 0, st,
             (const float*)w.partial, n_tokens > 0 ? p.n_chunks : 0, (int64_t)E * d, w.s2, (unsigned int*)nullptr,
             0);
  POP_LAUNCH(k_importance<T>, dim3((d_ff + 3) / 4, E), dim3(256), (size_t)d * sizeof(float), st, (const T*)W_up,
             d_ff, d, (const float*)w.s2, I);
  POP_LAUNCH(k_partition, dim3(E), dim3(kPartThreads), 0, st, (const float*)I, d_ff, c.c_low, c.c_high, R, C, P);
}

static pop_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}

static pop_status check_importance_args(const void* X, int64_t n_tokens, int32_t d, const void* W_up, int32_t d_ff,
                                        pop_dtype dt) {
  pop_status s = check_dtype_width(dt, d);
  if (s != POP_OK) return s;
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (n_tokens < 0 || n_tokens > ((int64_t)1 << 40) / d)
    return fail(POP_ERR_BAD_SHAPE, "n_tokens=%lld out of range", (long long)n_tokens);
  if ((n_tokens > 0 && X == nullptr) || W_up == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "X and W_up must be non-NULL");
  if (!aligned16(X) || !aligned16(W_up)) return fail(POP_ERR_MISALIGNED, "X and W_up must be 16-byte aligned");
  return POP_OK;
}

}  // namespace pop

using namespace pop;

extern "C" size_t pop_prefill_importance_workspace_bytes(int64_t n_tokens, int32_t d) {
  if (n_tokens < 0 || d <= 0) return 0;
  return importance_ws_bytes(n_tokens, d);
}

extern "C" size_t pop_prefill_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff) {
  if (n_tokens < 0 || d <= 0 || d_ff <= 0) return 0;
  return importance_ws_bytes(n_tokens, d) + align_up((size_t)d_ff * sizeof(float), 256);
}

extern "C" pop_status pop_prefill_importance(const void* X, int64_t n_tokens, int32_t d, const void* W_up,
                                             int32_t d_ff, pop_dtype dt, float* importance, void* ws,
                                             size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_importance_args(X, n_tokens, d, W_up, d_ff, dt);
  if (s != POP_OK) return s;
  if (importance == nullptr || ws == nullptr) return fail(POP_ERR_INVALID_ARGUMENT, "importance and ws must be non-NULL");
  if (!aligned16(ws)) return fail(POP_ERR_MISALIGNED, "ws must be 16-byte aligned");
  const size_t need = importance_ws_bytes(n_tokens, d);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  trace_mark(stream);
  if (dt == POP_BF16)
    launch_importance<bf16s>((hipStream_t)stream, X, n_tokens, d, W_up, d_ff, importance, (char*)ws);
  else
    launch_importance<float>((hipStream_t)stream, X, n_tokens, d, W_up, d_ff, importance, (char*)ws);
  return launched();
}

extern "C" pop_status pop_partition_select(const float* importance, int32_t d_ff, double r, double gamma, int32_t* R,
                                           int32_t* C, int32_t* P, void* stream) {
  clear_error();
  pop_status s = check_rate(r, gamma);
  if (s != POP_OK) return s;
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  const pop_counts c = counts(d_ff, r, gamma);
  if (importance == nullptr || (c.n_R > 0 && R == nullptr) || (c.n_C > 0 && C == nullptr) ||
      (c.n_P > 0 && P == nullptr))
    return fail(POP_ERR_INVALID_ARGUMENT, "importance or an output list with a nonzero size is NULL");
  trace_mark(stream);
  POP_LAUNCH(k_partition, dim3(1), dim3(kPartThreads), 0, (hipStream_t)stream, importance, d_ff, c.c_low,
                     c.c_high, R, C, P);
  return launched();
}

extern "C" pop_status pop_prefill_partition(const void* X, int64_t n_tokens, int32_t d, const void* W_up,
                                            int32_t d_ff, pop_dtype dt, double r, double gamma, int32_t* R,
                                            int32_t* C, int32_t* P, float* importance, void* ws, size_t ws_bytes,
                                            void* stream) {
  clear_error();
  pop_status s = check_importance_args(X, n_tokens, d, W_up, d_ff, dt);
  if (s != POP_OK) return s;
  if ((s = check_rate(r, gamma)) != POP_OK) return s;
  const pop_counts c = counts(d_ff, r, gamma);
  if ((c.n_R > 0 && R == nullptr) || (c.n_C > 0 && C == nullptr) || (c.n_P > 0 && P == nullptr) || ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "ws or an output list with a nonzero size is NULL");
  if (!aligned16(ws) || !aligned16(importance))
    return fail(POP_ERR_MISALIGNED, "importance and ws must be 16-byte aligned");
  const size_t need = pop_prefill_workspace_bytes(n_tokens, d, d_ff);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  const size_t iw = importance_ws_bytes(n_tokens, d);
  float* I = importance ? importance : (float*)((char*)ws + iw);
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  if (dt == POP_BF16)
    launch_importance<bf16s>(st, X, n_tokens, d, W_up, d_ff, I, (char*)ws);
  else
    launch_importance<float>(st, X, n_tokens, d, W_up, d_ff, I, (char*)ws);
  POP_LAUNCH(k_partition, dim3(1), dim3(kPartThreads), 0, st, (const float*)I, d_ff, c.c_low, c.c_high, R, C,
                     P);
  return launched();
}

extern "C" size_t pop_moe_prefill_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff, int32_t n_experts) {
  if (n_tokens < 0 || d <= 0 || d_ff <= 0 || n_experts < 2 || n_experts > kMoeMaxExperts) return 0;
  return moe_prefill_ws(n_tokens, d, d_ff, n_experts, nullptr).bytes;
}

extern "C" pop_status pop_moe_prefill_partition(const void* X, int64_t n_tokens, int32_t d, const float* logits,
                                                int32_t n_experts, const void* W_up, int32_t d_ff, pop_dtype dt,
                                                double r, double gamma, int32_t* R, int32_t* C, int32_t* P,
                                                float* importance, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_importance_args(X, n_tokens, d, W_up, d_ff, dt);
  if (s != POP_OK) return s;
  if ((s = check_rate(r, gamma)) != POP_OK) return s;
  if (n_experts < 2 || n_experts > kMoeMaxExperts)
    return fail(POP_ERR_BAD_SHAPE, "n_experts=%d outside [2, %d]", n_experts, kMoeMaxExperts);
  if (n_tokens > POP_MAX_MOE_TOKENS)
    return fail(POP_ERR_BAD_SHAPE, "n_tokens=%lld above %d", (long long)n_tokens, POP_MAX_MOE_TOKENS);
  if ((size_t)n_experts * 64 * (dt == POP_BF16 ? 8 : 4) * sizeof(float) > 65536)
    return fail(POP_ERR_BAD_SHAPE, "n_experts=%d: too many experts for the LDS accumulators", n_experts);
  const pop_counts c = counts(d_ff, r, gamma);
  if ((n_tokens > 0 && logits == nullptr) || (c.n_R > 0 && R == nullptr) || (c.n_C > 0 && C == nullptr) ||
      (c.n_P > 0 && P == nullptr) || ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "logits, ws or an output list with a nonzero size is NULL");
  if (!aligned16(ws) || !aligned16(importance) || !aligned16(logits))
    return fail(POP_ERR_MISALIGNED, "logits, importance and ws must be 16-byte aligned");
  const MoePrefillWs w0 = moe_prefill_ws(n_tokens, d, d_ff, n_experts, nullptr);
  if (ws_bytes < w0.bytes) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, w0.bytes);
  const MoePrefillWs w = moe_prefill_ws(n_tokens, d, d_ff, n_experts, (char*)ws);
  float* I = importance ? importance : w.I;
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  if (dt == POP_BF16)
    launch_moe_prefill<bf16s>(st, X, n_tokens, d, logits, n_experts, W_up, d_ff, c, R, C, P, I, w);
  else
    launch_moe_prefill<float>(st, X, n_tokens, d, logits, n_experts, W_up, d_ff, c, R, C, P, I, w);
  return launched();
}
