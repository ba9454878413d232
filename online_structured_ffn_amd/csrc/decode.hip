// Per-step candidate-masked decode FFN (POP notes, "Key design 2" and
// "Overall framework") and the dense decode baseline.
//
//   K4  gate/up GEMV over the rows R then C: z = SiLU(W_gate x) * (W_up x),
//       fused candidate score max_b |z_b|                (HBM-bound)
//   K5  one-workgroup radix top-k over the candidate scores   (latency-bound)
//   K6  down-projection over R and the selected rows of W_downT, partial sums
//       per row chunk                                      (HBM-bound)
//   K6r fixed-order reduction of the partial sums into y
#include <hip/hip_runtime.h>

#include "pop_device.h"
#include "pop_internal.h"

namespace pop {

// Channel of gate/up position p: R[p] for p < n_R, then C[p - n_R];
// identity when R is NULL (dense).
// Channel ids read from caller lists are clamped into [0, d_ff): an invalid
// list gives a wrong result, never an out-of-bounds read.
__device__ __forceinline__ int clamp_channel(int ch, int d_ff) { return min(max(ch, 0), d_ff - 1); }

__device__ __forceinline__ int gateup_channel(const int32_t* R, int n_R, const int32_t* C, int p, int d_ff) {
  if (R == nullptr) return p;
  return clamp_channel(p < n_R ? R[p] : C[p - n_R], d_ff);
}

// ---------------------------------------------------------------- K4
// Block: 256 threads = 4 waves; one gate/up row pair per wave at a time.
// Each lane reads 16-byte vectors of the gate and up rows (two rows, U
// vectors each in flight) and the matching vectors of x (cache-resident).
// BT batch rows are accumulated per pass over the weights.
template <typename T, int BT>
__global__ __launch_bounds__(256) void k_gateup(const T* __restrict__ x, int B, int d, const T* __restrict__ Wg,
                                                const T* __restrict__ Wu, int d_ff, const int32_t* __restrict__ R,
                                                int n_R, const int32_t* __restrict__ C, int n_C, float* __restrict__ z,
                                                float* __restrict__ score) {
  constexpr int V = Vec<T>::N;
  constexpr int STEP = 64 * V;
  constexpr int U = 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_A = n_R + n_C;
  for (int p = blockIdx.x * 4 + wave; p < n_A; p += gridDim.x * 4) {
    const int ch = gateup_channel(R, n_R, C, p, d_ff);
    const T* wg = Wg + (int64_t)ch * d;
    const T* wu = Wu + (int64_t)ch * d;
    float smax = 0.f;
    for (int b0 = 0; b0 < B; b0 += BT) {
      float ag[BT], au[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) ag[b] = au[b] = 0.f;
      int k0 = 0;
      for (; k0 + U * STEP <= d; k0 += U * STEP) {
        u32x4 qg[U], qu[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          qg[j] = ld16_stream(wg + k0 + j * STEP + lane * V);
          qu[j] = ld16_stream(wu + k0 + j * STEP + lane * V);
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
          float g[V], u[V];
          unpack(qg[j], g, T{});
          unpack(qu[j], u, T{});
          const int k = k0 + j * STEP + lane * V;
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            if (b0 + b < B) {
              float xv[V];
              unpack(ld16(x + (int64_t)(b0 + b) * d + k), xv, T{});
#pragma unroll
              for (int v = 0; v < V; ++v) {
                ag[b] = fmaf(g[v], xv[v], ag[b]);
                au[b] = fmaf(u[v], xv[v], au[b]);
              }
            }
          }
        }
      }
      for (; k0 < d; k0 += STEP) {
        const int k = k0 + lane * V;
        if (k < d) {
          float g[V], u[V];
          unpack(ld16_stream(wg + k), g, T{});
          unpack(ld16_stream(wu + k), u, T{});
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            if (b0 + b < B) {
              float xv[V];
              unpack(ld16(x + (int64_t)(b0 + b) * d + k), xv, T{});
#pragma unroll
              for (int v = 0; v < V; ++v) {
                ag[b] = fmaf(g[v], xv[v], ag[b]);
                au[b] = fmaf(u[v], xv[v], au[b]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const float gs = wave_sum(ag[b]);
        const float us = wave_sum(au[b]);
        if (b0 + b < B) {
          const float zz = silu(gs) * us;
          if (lane == 0) z[(int64_t)(b0 + b) * n_A + p] = zz;
          smax = fmaxf(smax, fabsf(zz));
        }
      }
    }
    if (lane == 0 && score != nullptr && p >= n_R) score[p - n_R] = smax;
  }
}

// ---------------------------------------------------------------- K5
// S = the k most important candidates (score descending, position ascending on
// ties); written as ascending positions Q into C and, optionally, as channels.
__global__ __launch_bounds__(kSelThreads) void k_topk(const float* __restrict__ score, int n, int k,
                                                      const int32_t* __restrict__ C, int32_t* __restrict__ Q,
                                                      int32_t* __restrict__ selected) {
  __shared__ SelShared sh;
  sel_load(score, n, sh);
  const int ranks[1] = {n - k};
  select_thresholds<1>(n, ranks, sh);
  const SelTarget t = sh.tgt[0];
  const int E = (n + kSelThreads - 1) / kSelThreads;
  const int base = threadIdx.x * E;
  const int end = min(n, base + E);
  int pos[3] = {0, 0, 0};
  for (int i = base; i < end; ++i)
    if (!sel_less(t, sel_key(sh.vals[i], i))) ++pos[0];
  int tot[3];
  block_exclusive_scan3(pos, tot, sh);
  for (int i = base; i < end; ++i) {
    if (!sel_less(t, sel_key(sh.vals[i], i))) {
      if (pos[0] < k) {  // an exact select never reaches the cap
        Q[pos[0]] = i;
        if (selected != nullptr) selected[pos[0]] = C[i];
      }
      ++pos[0];
    }
  }
}

// ---------------------------------------------------------------- K6
// Block: 256 threads = 4 waves sharing one column slice of 64*V columns; the
// block's chunk of live rows is dealt round-robin to the waves, each lane
// reading one 16-byte vector per row (a wave reads 1 KB of a bf16 row).  The
// four wave accumulators are combined in wave order through LDS and written as
// this chunk's partial sum.
template <typename T, int BT>
__global__ __launch_bounds__(256) void k_down_partial(const float* __restrict__ z, int n_A, int B,
                                                      const T* __restrict__ WdT, int d, int d_ff,
                                                      const int32_t* __restrict__ R,
                                                      int n_R, const int32_t* __restrict__ C,
                                                      const int32_t* __restrict__ Q, int n_live, int rows_per_chunk,
                                                      float* __restrict__ partial) {
  constexpr int V = Vec<T>::N;
  constexpr int U = 4;
  __shared__ float red[3][BT * V][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (blockIdx.x * 64 + lane) * V;
  const bool on = col < d;
  const int q0 = blockIdx.y * rows_per_chunk;
  const int q1 = min(n_live, q0 + rows_per_chunk);
  for (int b0 = 0; b0 < B; b0 += BT) {
    float acc[BT][V];
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int v = 0; v < V; ++v) acc[b][v] = 0.f;
    int q = q0 + wave;
    for (; q + 4 * (U - 1) < q1; q += 4 * U) {
      int ch[U], zp[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int qq = q + 4 * j;
        if (R == nullptr) {
          ch[j] = qq;
          zp[j] = qq;
        } else if (qq < n_R) {
          ch[j] = clamp_channel(R[qq], d_ff);
          zp[j] = qq;
        } else {
          const int pj = Q[qq - n_R];
          ch[j] = clamp_channel(C[pj], d_ff);
          zp[j] = n_R + pj;
        }
      }
      u32x4 w[U];
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (on) w[j] = ld16_stream(WdT + (int64_t)ch[j] * d + col);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        float f[V];
        if (on) unpack(w[j], f, T{});
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b0 + b < B && on) {
            const float zb = z[(int64_t)(b0 + b) * n_A + zp[j]];
#pragma unroll
            for (int v = 0; v < V; ++v) acc[b][v] = fmaf(zb, f[v], acc[b][v]);
          }
        }
      }
    }
    for (; q < q1; q += 4) {
      int ch, zpp;
      if (R == nullptr) {
        ch = q;
        zpp = q;
      } else if (q < n_R) {
        ch = clamp_channel(R[q], d_ff);
        zpp = q;
      } else {
        const int pj = Q[q - n_R];
        ch = clamp_channel(C[pj], d_ff);
        zpp = n_R + pj;
      }
      if (on) {
        float f[V];
        unpack(ld16_stream(WdT + (int64_t)ch * d + col), f, T{});
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b0 + b < B) {
            const float zb = z[(int64_t)(b0 + b) * n_A + zpp];
#pragma unroll
            for (int v = 0; v < V; ++v) acc[b][v] = fmaf(zb, f[v], acc[b][v]);
          }
        }
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int v = 0; v < V; ++v) red[wave - 1][b * V + v][lane] = acc[b][v];
    }
    __syncthreads();
    if (wave == 0 && on) {
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        if (b0 + b < B) {
          float* out = partial + ((int64_t)blockIdx.y * B + b0 + b) * d + col;
#pragma unroll
          for (int v = 0; v < V; ++v) {
            float s = acc[b][v];
            s += red[0][b * V + v][lane];
            s += red[1][b * V + v][lane];
            s += red[2][b * V + v][lane];
            out[v] = s;
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- host
struct DownPlan {
  int col_blocks;
  int n_chunks;
  int rows_per_chunk;
};

static DownPlan plan_down(int n_live, int B, int d, int vec) {
  DownPlan p;
  p.col_blocks = (d + 64 * vec - 1) / (64 * vec);
  int want = (1024 + p.col_blocks - 1) / p.col_blocks;     // ~1024 blocks of 4 waves
  const int by_rows = (n_live + 15) / 16;                  // >= 16 rows per chunk
  const int by_bytes = B > 0 ? (n_live + 8 * B - 1) / (8 * B) : want;  // partials <= ~1/4 of the row bytes
  if (want > by_rows) want = by_rows;
  if (want > by_bytes) want = by_bytes;
  if (want > 256) want = 256;
  if (want < 1) want = 1;
  p.rows_per_chunk = n_live > 0 ? (n_live + want - 1) / want : 1;
  p.n_chunks = n_live > 0 ? (n_live + p.rows_per_chunk - 1) / p.rows_per_chunk : 1;
  return p;
}

struct DecodeWs {
  float* z;
  float* score;
  int32_t* Q;
  float* partial;
};

static size_t decode_ws_layout(int32_t batch, int32_t d, int32_t d_ff, char* base, DecodeWs* out) {
  size_t off = 0;
  const size_t zb = align_up((size_t)batch * d_ff * sizeof(float) + 16, 256);
  const size_t sb = align_up((size_t)d_ff * sizeof(float), 256);
  const size_t qb = align_up((size_t)d_ff * sizeof(int32_t), 256);
  if (out) out->z = (float*)(base + off);
  off += zb;
  if (out) out->score = (float*)(base + off);
  off += sb;
  if (out) out->Q = (int32_t*)(base + off);
  off += qb;
  if (out) out->partial = (float*)(base + off);
  const int b = batch > 0 ? batch : 1;
  off += align_up((size_t)256 * b * d * sizeof(float), 256);  // at most 256 chunks
  return off;
}

template <typename T, int BT>
static void launch_gateup(hipStream_t st, int grid, const void* x, int B, int d, const void* Wg, const void* Wu,
                          int d_ff, const int32_t* R, int n_R, const int32_t* C, int n_C, float* z, float* score) {
  hipLaunchKernelGGL((k_gateup<T, BT>), dim3(grid), dim3(256), 0, st, (const T*)x, B, d, (const T*)Wg,
                     (const T*)Wu, d_ff, R, n_R, C, n_C, z, score);
}

template <typename T, int BT>
static void launch_down(hipStream_t st, const DownPlan& p, const float* z, int n_A, int B, const void* WdT, int d,
                        int d_ff, const int32_t* R, int n_R, const int32_t* C, const int32_t* Q, int n_live,
                        float* partial) {
  hipLaunchKernelGGL((k_down_partial<T, BT>), dim3(p.col_blocks, p.n_chunks), dim3(256), 0, st, z, n_A, B,
                     (const T*)WdT, d, d_ff, R, n_R, C, Q, n_live, p.rows_per_chunk, partial);
}

template <typename T>
static void run_decode(hipStream_t st, const void* x, int B, int d, int d_ff, const void* Wg, const void* Wu,
                       const void* WdT, const int32_t* R, int n_R, const int32_t* C, int n_C, int k, float* y, int32_t* selected,
                       const DecodeWs& w) {
  const int n_A = n_R + n_C;
  const int vec = Vec<T>::N;
  int grid = (n_A + 3) / 4;
  if (grid < 1) grid = 1;
  if (B <= 1)
    launch_gateup<T, 1>(st, grid, x, B, d, Wg, Wu, d_ff, R, n_R, C, n_C, w.z, w.score);
  else if (B <= 2)
    launch_gateup<T, 2>(st, grid, x, B, d, Wg, Wu, d_ff, R, n_R, C, n_C, w.z, w.score);
  else
    launch_gateup<T, 4>(st, grid, x, B, d, Wg, Wu, d_ff, R, n_R, C, n_C, w.z, w.score);
  if (R != nullptr && n_C > 0)
    hipLaunchKernelGGL(k_topk, dim3(1), dim3(kSelThreads), 0, st, (const float*)w.score, n_C, k, C, w.Q, selected);
  const int n_live = n_R + k;
  if (B == 0) return;
  const DownPlan p = plan_down(n_live, B, d, vec);
  if (B <= 1)
    launch_down<T, 1>(st, p, w.z, n_A, B, WdT, d, d_ff, R, n_R, C, w.Q, n_live, w.partial);
  else if (B <= 2)
    launch_down<T, 2>(st, p, w.z, n_A, B, WdT, d, d_ff, R, n_R, C, w.Q, n_live, w.partial);
  else
    launch_down<T, 4>(st, p, w.z, n_A, B, WdT, d, d_ff, R, n_R, C, w.Q, n_live, w.partial);
  const int64_t n_out = (int64_t)B * d;
  hipLaunchKernelGGL(k_sum_chunks<0>, dim3((unsigned)((n_out + 31) / 32)), dim3(256), 0, st, (const float*)w.partial,
                     n_live > 0 ? p.n_chunks : 0, n_out, y);
}

static pop_status check_decode_common(const void* x, int32_t batch, int32_t d, const void* Wg, const void* Wu,
                                      const void* WdT, int32_t d_ff, pop_dtype dt, float* y, void* ws,
                                      size_t ws_bytes) {
  pop_status s = check_dtype_width(dt, d);
  if (s != POP_OK) return s;
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (batch < 0 || batch > POP_MAX_BATCH) return fail(POP_ERR_BAD_SHAPE, "batch=%d outside [0, %d]", batch, POP_MAX_BATCH);
  if ((batch > 0 && (x == nullptr || y == nullptr)) || Wg == nullptr || Wu == nullptr || WdT == nullptr ||
      ws == nullptr)
    return fail(POP_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(Wg) || !aligned16(Wu) || !aligned16(WdT) || !aligned16(y) || !aligned16(ws))
    return fail(POP_ERR_MISALIGNED, "x, weights, y and ws must be 16-byte aligned");
  const size_t need = pop_decode_workspace_bytes(batch, d, d_ff);
  if (ws_bytes < need) return fail(POP_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  return POP_OK;
}

}  // namespace pop

using namespace pop;

extern "C" size_t pop_decode_workspace_bytes(int32_t batch, int32_t d, int32_t d_ff) {
  if (batch < 0 || d <= 0 || d_ff <= 0) return 0;
  return decode_ws_layout(batch, d, d_ff, nullptr, nullptr);
}

extern "C" pop_status pop_decode_ffn(const void* x, int32_t batch, int32_t d, const void* W_gate, const void* W_up,
                                     const void* W_downT, int32_t d_ff, pop_dtype dt, const int32_t* R, int32_t n_R,
                                     const int32_t* C, int32_t n_C, double r, float* y, int32_t* selected, void* ws,
                                     size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_decode_common(x, batch, d, W_gate, W_up, W_downT, d_ff, dt, y, ws, ws_bytes);
  if (s != POP_OK) return s;
  if (!(r >= 0.0 && r < 1.0)) return fail(POP_ERR_INVALID_ARGUMENT, "r=%g outside [0, 1)", r);
  if (n_R < 0 || n_C < 0 || (int64_t)n_R + n_C > d_ff)
    return fail(POP_ERR_INVALID_ARGUMENT, "n_R=%d, n_C=%d inconsistent with d_ff=%d", n_R, n_C, d_ff);
  if ((n_R > 0 && R == nullptr) || (n_C > 0 && C == nullptr))
    return fail(POP_ERR_INVALID_ARGUMENT, "R or C is NULL with a nonzero size");
  const int32_t k = topk_count(d_ff, r, n_R, n_C);
  DecodeWs w;
  decode_ws_layout(batch, d, d_ff, (char*)ws, &w);
  // R == NULL selects the identity channel map inside the kernels; give the
  // kernels a non-NULL R even when it is empty.
  const int32_t* Rk = R != nullptr ? R : w.Q;
  const int32_t* Ck = C != nullptr ? C : w.Q;
  hipStream_t st = (hipStream_t)stream;
  if (dt == POP_BF16)
    run_decode<bf16s>(st, x, batch, d, d_ff, W_gate, W_up, W_downT, Rk, n_R, Ck, n_C, k, y, selected, w);
  else
    run_decode<float>(st, x, batch, d, d_ff, W_gate, W_up, W_downT, Rk, n_R, Ck, n_C, k, y, selected, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}

extern "C" pop_status pop_dense_ffn_decode(const void* x, int32_t batch, int32_t d, const void* W_gate,
                                           const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                           float* y, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  pop_status s = check_decode_common(x, batch, d, W_gate, W_up, W_downT, d_ff, dt, y, ws, ws_bytes);
  if (s != POP_OK) return s;
  DecodeWs w;
  decode_ws_layout(batch, d, d_ff, (char*)ws, &w);
  hipStream_t st = (hipStream_t)stream;
  if (dt == POP_BF16)
    run_decode<bf16s>(st, x, batch, d, d_ff, W_gate, W_up, W_downT, nullptr, d_ff, nullptr, 0, 0, y, nullptr, w);
  else
    run_decode<float>(st, x, batch, d, d_ff, W_gate, W_up, W_downT, nullptr, d_ff, nullptr, 0, 0, y, nullptr, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(POP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return POP_OK;
}
