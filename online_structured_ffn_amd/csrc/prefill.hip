// Prefill three-region partition (POP notes, "Key design 1").
//
//   K1  column sum of squares  s2[k] = sum_n X[n,k]^2         (HBM-bound on X)
//       one pass per column slice for prompts of up to 8192 tokens, else
//       partial sums over row chunks and (K1r) their fixed-order reduction
//   K2  importance items: sum_k W_up[i,k]^2 * s2[k] over pieces of each row,
//       in equal shares per wave                              (HBM-bound on W_up)
//   K3  one workgroup: I[i] = sqrt of the sum of row i's pieces, then the
//       select of the keys at ranks c_low and c_high and an order-preserving
//       compaction into P, C, R                               (latency-bound)
//   (k_importance, one row per wave, serves the per-expert MoE partition.)
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "moe_route.h"
#include "partition.h"
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

// ---------------------------------------------------------------- K1, one pass
// For prompts of up to kCsOnePassMax tokens: block b owns kCsCols columns and
// reads them from every row, so s2 comes out of one launch with no partial
// sums.  1024 threads = 16 waves; a row's kCsCols columns are kCsCols / V
// lanes x 16 bytes, so one wave instruction covers 64 / (kCsCols / V) rows.
// Per-lane sums are reduced across lanes (shuffles), then across waves in wave
// order (LDS): the same bits on every run.  Blocks sharing a 128-byte line of
// X are dealt to one XCD (blocks go to the eight XCDs round-robin).
constexpr int kCsCols = 16;
constexpr int kCsThreads = 1024;
constexpr int64_t kCsOnePassMax = 8192;

template <typename T>
__global__ __launch_bounds__(kCsThreads) void k_colsq_slices(const T* __restrict__ X, int64_t n_tokens, int d,
                                                             float* __restrict__ s2) {
  constexpr int V = Vec<T>::N;
  constexpr int LR = kCsCols / V;                       // lanes per row
  constexpr int RPW = 64 / LR;                          // rows per wave instruction
  constexpr int RPB = RPW * (kCsThreads / 64);          // rows per block instruction
  constexpr int NB = 4;                                 // row loads in flight per lane
  constexpr int SP = 128 / (kCsCols * (int)sizeof(T));  // slices per 128-byte line
  constexpr int G = 8 * SP;
  __shared__ float red[kCsThreads / 64][kCsCols];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int b = blockIdx.x;
  if (SP > 1 && (b | (G - 1)) < (int)gridDim.x) b = (b / G * 8 + b % 8) * SP + (b / 8) % SP;
  const int c0 = b * kCsCols;
  const int col = min(c0 + (lane % LR) * V, d - V);
  const int rl = wave * RPW + lane / LR;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  for (int64_t r0 = 0; r0 < n_tokens; r0 += NB * RPB) {
    u32x4 q[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int64_t r = min(r0 + u * RPB + rl, n_tokens - 1);
      q[u] = ld16_stream(X + r * d + col);
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool on = r0 + u * RPB + rl < n_tokens;
      float f[V];
      unpack(q[u], f, T{});
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] += on ? f[v] * f[v] : 0.f;
    }
  }
#pragma unroll
  for (int o = LR; o < 64; o <<= 1)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] += __shfl_xor(acc[v], o);
  if (lane < LR) {
#pragma unroll
    for (int v = 0; v < V; ++v) red[wave][lane * V + v] = acc[v];
  }
  __syncthreads();
  if (threadIdx.x < kCsCols && c0 + (int)threadIdx.x < d) {
    float t = red[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < kCsThreads / 64; ++w) t += red[w][threadIdx.x];
    s2[c0 + threadIdx.x] = t;
  }
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
// Block: 256 threads = 4 waves; wave w of block b takes rows b*4 + w,
// b*4 + w + 4*gridDim.x, ...  A row is read in chunks of kImpChunk columns
// (kImpLoads 16-byte vectors per lane, all issued together), and the next
// chunk's loads are in flight while the current one is reduced (double
// buffer over the wave's (row, chunk) items).  s2 sits in LDS, zero-padded to
// whole chunks, so the loads need no column mask (columns past d are clamped
// to the row's last vector and meet s2 = 0).  The order of the products in
// the sum is the same as for s2 in plain column order.
// blockIdx.y selects an expert (MoE): its W_up, s2 and I follow the previous
// expert's contiguously; gridDim.y = 1 otherwise.
constexpr int kImpLoads = 8;
#ifndef POP_IMP_BLOCKS
#define POP_IMP_BLOCKS 512
#endif
constexpr int kImpBlocks = POP_IMP_BLOCKS;

template <typename T>
struct ImpBuf {
  u32x4 q[kImpLoads];
};

template <typename T>
__global__ __launch_bounds__(256) void k_importance(const T* __restrict__ W, int d_ff, int d,
                                                    const float* __restrict__ s2, float* __restrict__ I) {
  constexpr int V = Vec<T>::N;
  constexpr int CH = kImpLoads * 64 * V;  // columns per chunk
  extern __shared__ float s2_lds[];
  W += (int64_t)blockIdx.y * d_ff * d;
  s2 += (int64_t)blockIdx.y * d;
  I += (int64_t)blockIdx.y * d_ff;
  const int n_ch = (d + CH - 1) / CH;
  // LDS layout: within each run of 64 * V columns (one load instruction of a
  // wave), lane l's V values are stored as V / 4 float4 groups at
  // (group * 64 + l) * 4, so that every LDS read below is a 16-byte read with
  // consecutive lanes 16 bytes apart (no bank conflicts).
  for (int k = threadIdx.x; k < n_ch * CH; k += 256) {
    const int run = k / (64 * V), l = (k / V) % 64, v = k % V;
    s2_lds[run * 64 * V + ((v / 4) * 64 + l) * 4 + v % 4] = k < d ? s2[k] : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = blockIdx.x * 4 + wave;
  const int rstep = gridDim.x * 4;
  const int n_rows = row0 < d_ff ? (d_ff - row0 + rstep - 1) / rstep : 0;
  const int n_items = n_rows * n_ch;
  if (n_items == 0) return;
  auto issue = [&](ImpBuf<T>& b, int it) {
    it = min(it, n_items - 1);  // past the end: reload the last item (unused)
    const int r = row0 + (it / n_ch) * rstep;
    const int c = it % n_ch;
    const T* w = W + (int64_t)r * d;
#pragma unroll
    for (int j = 0; j < kImpLoads; ++j) b.q[j] = ld16_stream(w + min(c * CH + j * 64 * V + lane * V, d - V));
  };
  float acc = 0.f;
  auto consume = [&](const ImpBuf<T>& b, int it) {
    if (it >= n_items) return;  // wave-uniform
    const int c = it % n_ch;
#pragma unroll
    for (int j = 0; j < kImpLoads; ++j) {
      float f[V];
      unpack(b.q[j], f, T{});
      const float* sp = s2_lds + c * CH + j * 64 * V + lane * 4;
#pragma unroll
      for (int g = 0; g < V / 4; ++g) {
        const float4 q4 = *reinterpret_cast<const float4*>(sp + g * 256);
        acc = fmaf(f[4 * g] * f[4 * g], q4.x, acc);
        acc = fmaf(f[4 * g + 1] * f[4 * g + 1], q4.y, acc);
        acc = fmaf(f[4 * g + 2] * f[4 * g + 2], q4.z, acc);
        acc = fmaf(f[4 * g + 3] * f[4 * g + 3], q4.w, acc);
      }
    }
    if (c == n_ch - 1) {
      const float t = wave_sum(acc);
      if (lane == 0) I[row0 + (it / n_ch) * rstep] = sqrtf(t);
      acc = 0.f;
    }
  };
  ImpBuf<T> A, B;
  issue(A, 0);
  for (int it = 0; it < n_items; it += 2) {
    issue(B, it + 1);
    __builtin_amdgcn_sched_barrier(0);
    consume(A, it);
    __builtin_amdgcn_sched_barrier(0);
    issue(A, it + 2);
    __builtin_amdgcn_sched_barrier(0);
    consume(B, it + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------- K3
constexpr int kPartThreads = 1024;

// One workgroup per split of n channels.  src holds, for channel i, either
// the importance itself (n_q = 0, src[i * stride]) or the n_q >= 1 item sums
// of k_importance_items at src[i * stride] (I_i = sqrt of their sum in item
// order, stored in I_out when it is not NULL).  blockIdx.x selects an expert (MoE), whose
// values and lists follow the previous expert's contiguously.  do_split = 0:
// I_out only.  Dynamic LDS: part_lds_bytes<kPartThreads>(n).
__global__ __launch_bounds__(kPartThreads) void k_partition(const float* __restrict__ src, int n, int n_q, int stride,
                                                           float* __restrict__ I_out, int c_low, int c_high,
                                                           int do_split, int32_t* __restrict__ R,
                                                           int32_t* __restrict__ C, int32_t* __restrict__ P) {
  extern __shared__ __align__(16) char smem[];
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
  PartShared<kPartThreads>& sh = *reinterpret_cast<PartShared<kPartThreads>*>(smem + part_keys_bytes<kPartThreads>(n));
  src += (int64_t)blockIdx.x * n * stride;
  R += (int64_t)blockIdx.x * (n - c_high);
  C += (int64_t)blockIdx.x * (c_high - c_low);
  P += (int64_t)blockIdx.x * c_low;
  if (n <= 0) return;
  uint32_t mn = 0xffffffffu, mx = 0u;
  // kPartBatch rows per thread at a time: their loads are in flight together
#ifndef POP_PART_BATCH
#define POP_PART_BATCH 12
#endif
  constexpr int kPartBatch = POP_PART_BATCH;
  for (int i0 = threadIdx.x; i0 < n; i0 += kPartBatch * kPartThreads) {
    float v[kPartBatch];
    if (n_q == 0) {
#pragma unroll
      for (int t = 0; t < kPartBatch; ++t) v[t] = src[(int64_t)min(i0 + t * kPartThreads, n - 1) * stride];
    } else if (n_q == 4 && stride == 4) {
      float4 q[kPartBatch];
#pragma unroll
      for (int t = 0; t < kPartBatch; ++t)
        q[t] = *reinterpret_cast<const float4*>(src + (int64_t)min(i0 + t * kPartThreads, n - 1) * 4);
#pragma unroll
      for (int t = 0; t < kPartBatch; ++t) v[t] = sqrtf(((q[t].x + q[t].y) + q[t].z) + q[t].w);
    } else {
#pragma unroll
      for (int t = 0; t < kPartBatch; ++t) {
        const float* p = src + (int64_t)min(i0 + t * kPartThreads, n - 1) * stride;
        float a = 0.f;
        for (int k = 0; k < n_q; ++k) a += p[k];
        v[t] = sqrtf(a);
      }
    }
#pragma unroll
    for (int t = 0; t < kPartBatch; ++t) {
      const int i = i0 + t * kPartThreads;
      if (i < n) {
        if (n_q != 0 && I_out != nullptr) I_out[(int64_t)blockIdx.x * n + i] = v[t];
        const uint32_t u = value_bits(v[t]);
        keys[i] = u;
        mn = min(mn, u);
        mx = max(mx, u);
      }
    }
  }
  if (do_split) partition_block<kPartThreads>(keys, n, mn, mx, c_low, c_high, R, C, P, sh);
}

// ---------------------------------------------------------------- K2, balanced
// k_importance_items: the weighted row norms in equal shares.  An item is
// kImpItemLoads 16-byte vectors per lane of one row (QC columns); the d_ff *
// n_q items are dealt to the gridDim.x * 16 waves in equal consecutive shares
// (a row's items may fall to two waves), so no wave waits on a longer share.
// Each wave issues its first chunk of W_up loads before staging s2 in LDS;
// the next chunk is in flight while the current one is reduced.  Each item's
// weighted sum of squares goes to ipart[row * n_qp + item]; k_partition adds
// a row's items in item order.
constexpr int kItemThreads = 1024;
constexpr int kItemWaves = kItemThreads / 64;
constexpr int kImpItemLoads = 2;  // 16-byte loads per lane per item
constexpr int kImpChunk = 4;      // items per buffer

template <typename T>
__host__ __device__ constexpr int item_cols() {
  return kImpItemLoads * 64 * Vec<T>::N;
}
__host__ __device__ inline int items_per_row(int d, int qc) { return (d + qc - 1) / qc; }
__host__ __device__ inline int items_stride(int n_q) { return (n_q + 3) & ~3; }

template <typename T>
__global__ __launch_bounds__(kItemThreads) void k_importance_items(const T* __restrict__ W, int d_ff, int d,
                                                                  const float* __restrict__ s2,
                                                                  float* __restrict__ ipart, int n_qp) {
  constexpr int V = Vec<T>::N;
  constexpr int QC = item_cols<T>();
  constexpr int NL = kImpChunk * kImpItemLoads;
  extern __shared__ __align__(16) float s2l[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_q = items_per_row(d, QC);
  const int64_t Q = (int64_t)d_ff * n_q;
  const int64_t NWv = (int64_t)gridDim.x * kItemWaves;
  const int64_t gw = (int64_t)blockIdx.x * kItemWaves + wave;
  const int i0 = (int)(Q * gw / NWv);
  const int n_it = (int)(Q * (gw + 1) / NWv - i0);
  const int n_ch = (n_it + kImpChunk - 1) / kImpChunk;
  auto issue = [&](u32x4(&q)[NL], int ch) {
#pragma unroll
    for (int u = 0; u < kImpChunk; ++u) {
      const int it = i0 + min(ch * kImpChunk + u, n_it - 1);  // past the share: its last item again (unused)
      const int row = it / n_q, qq = it % n_q;
      const T* w = W + (int64_t)row * d;
#pragma unroll
      for (int l = 0; l < kImpItemLoads; ++l)
        q[u * kImpItemLoads + l] = ld16_stream(w + min(qq * QC + l * 64 * V + lane * V, d - V));
    }
  };
  auto consume = [&](const u32x4(&q)[NL], int ch) {
#pragma unroll
    for (int u = 0; u < kImpChunk; ++u) {
      const int k = ch * kImpChunk + u;
      if (k >= n_it) break;  // wave-uniform
      const int it = i0 + k;
      const int row = it / n_q, qq = it % n_q;
      float acc = 0.f;
#pragma unroll
      for (int l = 0; l < kImpItemLoads; ++l) {
        float f[V];
        unpack(q[u * kImpItemLoads + l], f, T{});
        const float* sp = s2l + qq * QC + l * 64 * V + lane * 4;
#pragma unroll
        for (int g = 0; g < V / 4; ++g) {
          const float4 q4 = *reinterpret_cast<const float4*>(sp + g * 256);
          acc = fmaf(f[4 * g] * f[4 * g], q4.x, acc);
          acc = fmaf(f[4 * g + 1] * f[4 * g + 1], q4.y, acc);
          acc = fmaf(f[4 * g + 2] * f[4 * g + 2], q4.z, acc);
          acc = fmaf(f[4 * g + 3] * f[4 * g + 3], q4.w, acc);
        }
      }
      const float t = wave_sum(acc);
      if (lane == 0) ipart[(int64_t)row * n_qp + qq] = t;
    }
  };
  // s2 in LDS, zero-padded to whole items; within each run of 64 * V columns
  // (one load instruction of a wave) lane l's V values sit as V / 4 float4
  // groups at (group * 64 + l) * 4: the reads above are 16 bytes per lane
  // with consecutive lanes 16 bytes apart.  Staged 16 bytes at a time (four
  // consecutive columns land in one float4 group; d is a multiple of 4).  The
  // s2 loads go out before the first W_up chunk's: loads return in issue
  // order, and the staging waits only for its own.
  constexpr int kS2Per = 4;  // float4 loads of s2 per thread in flight (n_q * QC <= kS2Per * 4 * 1024 here)
  const int n4 = n_q * QC / 4;
  float4 s2q[kS2Per];
#pragma unroll
  for (int r = 0; r < kS2Per; ++r) {
    const int k = 4 * ((int)threadIdx.x + r * kItemThreads);
    s2q[r] = k < d ? *reinterpret_cast<const float4*>(s2 + k) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  u32x4 A[NL], B[NL];
  if (n_it > 0) issue(A, 0);  // wave-uniform; in flight while s2 is staged
#pragma unroll
  for (int r = 0; r < kS2Per; ++r) {
    const int k4 = (int)threadIdx.x + r * kItemThreads;
    if (k4 < n4) {
      const int k = 4 * k4;
      const int run = k / (64 * V), l = (k / V) % 64, v = k % V;
      *reinterpret_cast<float4*>(s2l + run * 64 * V + ((v / 4) * 64 + l) * 4) = s2q[r];
    }
  }
  // wider rows: the rest of s2, in order after the chunk
  for (int k4 = (int)threadIdx.x + kS2Per * kItemThreads; k4 < n4; k4 += kItemThreads) {
    const int k = 4 * k4;
    const int run = k / (64 * V), l = (k / V) % 64, v = k % V;
    const float4 q = k < d ? *reinterpret_cast<const float4*>(s2 + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(s2l + run * 64 * V + ((v / 4) * 64 + l) * 4) = q;
  }
  lds_barrier();  // the first chunk's loads stay in flight
  for (int ch = 0; ch < n_ch; ch += 2) {  // wave-uniform
    if (ch + 1 < n_ch) issue(B, ch + 1);
    __builtin_amdgcn_sched_barrier(0);
    consume(A, ch);
    __builtin_amdgcn_sched_barrier(0);
    if (ch + 2 < n_ch) issue(A, ch + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (ch + 1 < n_ch) consume(B, ch + 1);
    __builtin_amdgcn_sched_barrier(0);
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

static int imp_blocks(int32_t d_ff) {
  const int want = (d_ff + 3) / 4;
  return want < kImpBlocks ? want : kImpBlocks;
}

template <typename T>
static size_t imp_lds_bytes(int32_t d) {
  constexpr int CH = kImpLoads * 64 * Vec<T>::N;
  return (size_t)((d + CH - 1) / CH) * CH * sizeof(float);
}

static size_t importance_ws_bytes(int64_t n_tokens, int32_t d) {
  // Widest plan over both dtypes (bf16 has fewer column blocks, hence more chunks).
  const PrefillPlan p = plan_prefill(n_tokens, d, 8);
  const PrefillPlan q = plan_prefill(n_tokens, d, 4);
  const int chunks = p.n_chunks > q.n_chunks ? p.n_chunks : q.n_chunks;
  return align_up((size_t)chunks * d * sizeof(float), 256)  // partial sums
         + align_up((size_t)d * sizeof(float), 256);        // s2
}

// s2 into the workspace's s2 slot (after the partial sums); returns it.
template <typename T>
static float* launch_colsq_t(hipStream_t st, const void* X, int64_t n_tokens, int32_t d, char* ws) {
  const PrefillPlan p = plan_prefill(n_tokens, d, Vec<T>::N);
  const PrefillPlan pb = plan_prefill(n_tokens, d, 8), pf = plan_prefill(n_tokens, d, 4);
  const int max_chunks = pb.n_chunks > pf.n_chunks ? pb.n_chunks : pf.n_chunks;
  float* partial = (float*)ws;
  float* s2 = (float*)(ws + align_up((size_t)max_chunks * d * sizeof(float), 256));
  if (n_tokens <= kCsOnePassMax) {
    // With no prompt token every column sum is 0, hence I = 0.
    POP_LAUNCH(k_colsq_slices<T>, dim3((d + kCsCols - 1) / kCsCols), dim3(kCsThreads), 0, st, (const T*)X, n_tokens,
               d, s2);
  } else {
    POP_LAUNCH(k_colsq_partial<T>, dim3(p.col_blocks, p.n_chunks), dim3(64), 0, st, (const T*)X, n_tokens, d,
               p.rows_per_chunk, partial);
    POP_LAUNCH(k_sum_chunks<0>, dim3((d + 31) / 32), dim3(1024), 0, st, (const float*)partial, p.n_chunks,
               (int64_t)d, s2, (unsigned int*)nullptr, 0);
  }
  return s2;
}


// ---- the partition of one FFN: column norms, importance items, split
// Workspace of pop_prefill_partition / pop_prefill_importance: the column-norm
// workspace (partial sums, then s2), then the item sums [d_ff][stride].
static size_t pre_ws_bytes(int64_t n_tokens, int32_t d, int32_t d_ff) {
  // fp32 items are half as wide as bf16 ones: the larger stride
  const int stride = items_stride(items_per_row(d, item_cols<float>()));
  return importance_ws_bytes(n_tokens, d) + align_up((size_t)d_ff * stride * sizeof(float), 256);
}

static int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cache[dev] = cus;
}

// s2, then the item sums, then k_partition (split = false: I only, into I).
template <typename T>
static void launch_prefill(hipStream_t st, const void* X, int64_t n_tokens, int32_t d, const void* W_up, int32_t d_ff,
                           int c_low, int c_high, bool split, int32_t* R, int32_t* C, int32_t* P, float* I,
                           char* ws) {
  const float* s2 = launch_colsq_t<T>(st, X, n_tokens, d, ws);
  float* ipart = (float*)(ws + importance_ws_bytes(n_tokens, d));
  const int n_q = items_per_row(d, item_cols<T>());
  const int stride = items_stride(n_q);
  const int64_t items = (int64_t)d_ff * n_q;
  // one workgroup per CU, fewer when there are under two items per wave
  int64_t G = device_cus();
  const int64_t want = (items + 2 * kItemWaves - 1) / (2 * kItemWaves);
  if (G < 1 || G > want) G = want;
  if (G < 1) G = 1;
  const size_t lds = (size_t)n_q * item_cols<T>() * sizeof(float);
  POP_LAUNCH(k_importance_items<T>, dim3((unsigned)G), dim3(kItemThreads), lds, st, (const T*)W_up, d_ff, d, s2,
             ipart, stride);
  POP_LAUNCH(k_partition, dim3(1), dim3(kPartThreads), part_lds_bytes<kPartThreads>(d_ff), st, (const float*)ipart,
             d_ff, n_q, stride, I, c_low, c_high, split ? 1 : 0, R, C, P);
}

size_t colsq_ws_bytes(int64_t n_tokens, int32_t d) { return importance_ws_bytes(n_tokens, d); }

float* launch_colsq(void* stream, const void* X, int64_t n_tokens, int32_t d, pop_dtype dt, char* ws) {
  return dt == POP_BF16 ? launch_colsq_t<bf16s>((hipStream_t)stream, X, n_tokens, d, ws)
                        : launch_colsq_t<float>((hipStream_t)stream, X, n_tokens, d, ws);
}

void launch_partition_lists(void* stream, const float* I, int32_t d_ff, int32_t c_low, int32_t c_high, int32_t* R,
                            int32_t* C, int32_t* P) {
  POP_LAUNCH(k_partition, dim3(1), dim3(kPartThreads), part_lds_bytes<kPartThreads>(d_ff), (hipStream_t)stream, I,
             d_ff, 0, 1, (float*)nullptr, c_low, c_high, 1, R, C, P);
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
  POP_LAUNCH(k_importance<T>, dim3(imp_blocks(d_ff), E), dim3(256), imp_lds_bytes<T>(d), st, (const T*)W_up,
             d_ff, d, (const float*)w.s2, I);
  POP_LAUNCH(k_partition, dim3(E), dim3(kPartThreads), part_lds_bytes<kPartThreads>(d_ff), st, (const float*)I, d_ff,
             0, 1, (float*)nullptr, c.c_low, c.c_high, 1, R, C, P);
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

extern "C" size_t pop_prefill_importance_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff) {
  if (n_tokens < 0 || d <= 0 || d_ff <= 0) return 0;
  return pre_ws_bytes(n_tokens, d, d_ff);
}

extern "C" size_t pop_prefill_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff) {
  if (n_tokens < 0 || d <= 0 || d_ff <= 0) return 0;
  return pre_ws_bytes(n_tokens, d, d_ff);
}

extern "C" pop_status pop_prefill_importance(const void* X, int64_t n_tokens, int32_t d, const void* W_up,
                                             int32_t d_ff, pop_dtype dt, float* importance, void* ws,
                                             size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_importance_args(X, n_tokens, d, W_up, d_ff, dt);
  if (s != POP_OK) return s;
  if (importance == nullptr || ws == nullptr) return fail(POP_ERR_INVALID_ARGUMENT, "importance and ws must be non-NULL");
  if (!aligned16(ws)) return fail(POP_ERR_MISALIGNED, "ws must be 16-byte aligned");
  const size_t need = pre_ws_bytes(n_tokens, d, d_ff);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  if (dt == POP_BF16)
    launch_prefill<bf16s>(st, X, n_tokens, d, W_up, d_ff, 0, 0, false, nullptr, nullptr, nullptr, importance,
                          (char*)ws);
  else
    launch_prefill<float>(st, X, n_tokens, d, W_up, d_ff, 0, 0, false, nullptr, nullptr, nullptr, importance,
                          (char*)ws);
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
  POP_LAUNCH(k_partition, dim3(1), dim3(kPartThreads), part_lds_bytes<kPartThreads>(d_ff), (hipStream_t)stream,
             importance, d_ff, 0, 1, (float*)nullptr, c.c_low, c.c_high, 1, R, C, P);
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
  const size_t need = pre_ws_bytes(n_tokens, d, d_ff);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  trace_mark(st);
  if (dt == POP_BF16)
    launch_prefill<bf16s>(st, X, n_tokens, d, W_up, d_ff, c.c_low, c.c_high, true, R, C, P, importance, (char*)ws);
  else
    launch_prefill<float>(st, X, n_tokens, d, W_up, d_ff, c.c_low, c.c_high, true, R, C, P, importance, (char*)ws);
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
